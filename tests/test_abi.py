"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, rejects bad arguments on the host before touching the device, and
its host-side bag validator agrees with the oracle."""
import ctypes

import numpy as np
import pytest

from oracle import dlrm_oracle as orc
from sparse_embedding_lookup_dlrm_amd import ops

E_INVAL, E_UNSUPPORTED, E_WORKSPACE, E_ALIGN = -1, -2, -3, -5


@pytest.fixture(scope="module")
def lib():
    return ops.lib()


def test_exports_every_header_function(lib):
    names = ops.header_functions()
    assert set(names) >= {"dlrm_embbag_fwd", "dlrm_interact", "dlrm_embbag_bwd_update", "dlrm_lengths_to_offsets",
                          "dlrm_embbag_bwd_workspace_bytes", "dlrm_validate_bags", "dlrm_status_string",
                          "dlrm_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(ops.status_string(code), str) and ops.status_string(code)
    assert ops.version() >= 100


# Fake device addresses: the calls below must fail validation before any HIP call,
# so these are never dereferenced.
A16 = 0x7F0000000000
MIS = A16 + 4


def _fwd(lib, T=2, B=4, D=16, dtype=0, tables=(A16, A16), rows=(10, 10), offsets=A16, indices=A16, nnz=8,
         e0=A16, pooled=None, inter=A16):
    tp = (ctypes.c_void_p * len(tables))(*tables) if tables is not None else None
    rp = (ctypes.c_int64 * len(rows))(*rows) if rows is not None else None
    return lib.dlrm_embbag_fwd(T, B, D, dtype, tp, rp, offsets, indices, nnz, e0, pooled, inter, None, None)


def test_fwd_rejects_bad_arguments(lib):
    assert _fwd(lib, T=0, tables=(), rows=()) == E_INVAL
    assert _fwd(lib, B=0) == E_INVAL
    assert _fwd(lib, D=0) == E_INVAL
    assert _fwd(lib, nnz=-1) == E_INVAL
    assert _fwd(lib, tables=None) == E_INVAL
    assert _fwd(lib, rows=None) == E_INVAL
    assert _fwd(lib, offsets=None) == E_INVAL
    assert _fwd(lib, indices=None) == E_INVAL
    assert _fwd(lib, tables=(A16, None)) == E_INVAL
    assert _fwd(lib, rows=(10, 0)) == E_INVAL
    assert _fwd(lib, rows=(10, 2 ** 31)) == E_INVAL
    assert _fwd(lib, inter=None, pooled=None) == E_INVAL
    assert _fwd(lib, e0=None) == E_INVAL
    assert _fwd(lib, dtype=3) == E_UNSUPPORTED
    assert _fwd(lib, D=12) == E_UNSUPPORTED          # 48-byte rows
    assert _fwd(lib, D=512) == E_UNSUPPORTED         # 2 KB fp32 rows
    assert _fwd(lib, D=2, dtype=1) == E_UNSUPPORTED  # 4-byte half rows
    assert _fwd(lib, T=129, tables=(A16,) * 129, rows=(10,) * 129) == E_UNSUPPORTED
    assert _fwd(lib, tables=(A16, MIS)) == E_ALIGN
    assert _fwd(lib, e0=MIS) == E_ALIGN
    assert _fwd(lib, pooled=MIS) == E_ALIGN
    assert _fwd(lib, offsets=A16 + 2) == E_ALIGN
    assert _fwd(lib, B=2 ** 30) == E_INVAL           # T*B + 1 >= 2^31


def test_interact_and_offsets_reject_bad_arguments(lib):
    assert lib.dlrm_interact(0, 4, 16, A16, A16, A16, None) == E_INVAL
    assert lib.dlrm_interact(2, 4, 16, None, A16, A16, None) == E_INVAL
    assert lib.dlrm_interact(2, 4, 6, A16, A16, A16, None) == E_UNSUPPORTED
    assert lib.dlrm_interact(2, 4, 16, MIS, A16, A16, None) == E_ALIGN
    assert lib.dlrm_interact(128, 4, 1024, A16, A16, A16, None) == E_UNSUPPORTED  # tile > LDS
    assert lib.dlrm_lengths_to_offsets(-1, A16, A16, None, None) == E_INVAL
    assert lib.dlrm_lengths_to_offsets(4, None, A16, None, None) == E_INVAL
    assert lib.dlrm_lengths_to_offsets(4, A16, None, None, None) == E_INVAL


def test_bwd_rejects_bad_arguments(lib):
    rows = (ctypes.c_int64 * 2)(10, 10)
    need = ctypes.c_size_t(0)
    assert lib.dlrm_embbag_bwd_workspace_bytes(2, 4, 16, 8, rows, ctypes.byref(need)) == 0
    assert need.value > 0
    assert lib.dlrm_embbag_bwd_workspace_bytes(0, 4, 16, 8, rows, ctypes.byref(need)) == E_INVAL
    tp = (ctypes.c_void_p * 2)(A16, A16)

    def call(ws_bytes=need.value, ws=A16, d_out=A16, rows_=rows, D=16, lr=0.01):
        return lib.dlrm_embbag_bwd_update(2, 4, D, 0, tp, rows_, A16, A16, 8, A16, A16, d_out, lr, None, None, None,
                                          None, None, ws, ws_bytes, None, None)

    assert call(ws_bytes=need.value - 1) == E_WORKSPACE
    assert call(ws=None) == E_INVAL
    assert call(d_out=None) == E_INVAL
    assert call(ws=A16 + 16) == E_ALIGN
    big = (ctypes.c_int64 * 2)(2 ** 31 - 2, 10)
    assert call(rows_=big) == E_UNSUPPORTED  # sum(rows) must fit int32 keys


@pytest.mark.parametrize("seed", range(8))
def test_host_validator_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    T, B = 3, 5
    rows = [4, 9, 2]
    lengths = rng.integers(0, 4, size=T * B)
    off = orc.lengths_to_offsets(lengths)
    idx = np.concatenate([rng.integers(0, rows[t], size=int(lengths[t * B:(t + 1) * B].sum()))
                          for t in range(T)]).astype(np.int32)
    kind = seed % 4
    if kind == 1 and len(idx):
        idx[rng.integers(len(idx))] = rows[0] + 7
    elif kind == 2:
        off = off.copy()
        off[3], off[4] = off[4] + 1, off[3]
    elif kind == 3 and len(idx):
        idx[-1] = -3
    want = orc.bag_status(T, B, rows, off, idx)
    assert ops.validate_bags(T, B, rows, off, idx) == want


def _ibwd_lds(T, D):
    F = T + 1
    return (F * (D + 4) + ((F + 3) & ~3) * F) * 4


def test_bwd_plan_interaction_backward_placement(lib):
    """Batches of at most 2048 occurrences per table on average sort per table (two
    launches, the interaction backward riding on both); larger ones take the radix passes
    over all keys, on whose launches the interaction backward rides only where one
    sample's LDS fits beside the sort kernel's own within 160 KiB."""
    # 26 fp32 tables, D = 128, one index per bag: per table, rows of 16 bits: two passes
    p = ops.bwd_plan(26, 2048, 128, 53248, [40_000] * 26)
    assert (p["table_sort"], p["radix_bits"], p["passes"], p["interact_bwd_shared"]) == (True, 8, 2, True)
    assert p["max_lds"] <= 160 * 1024
    # one occurrence more: radix passes over the 22-bit keys, three 8-bit passes, shared
    p = ops.bwd_plan(26, 2048, 128, 53249, [40_000] * 26)
    assert (p["table_sort"], p["radix_bits"], p["passes"], p["interact_bwd_shared"]) == (False, 8, 3, True)
    # per table, the passes follow the largest table (1000 and 70000 rows: 17 bits)
    p = ops.bwd_plan(2, 100, 16, 300, [1000, 70_000])
    assert (p["table_sort"], p["passes"]) == (True, 3)
    # a batch past 65536 samples takes the radix passes
    assert not ops.bwd_plan(2, 65537, 16, 300, [1000, 1000])["table_sort"]
    # 68 tables, D = 512: one sample's tile (152 KiB) fits beside table_place's few bytes...
    assert _ibwd_lds(68, 512) <= 160 * 1024
    p = ops.bwd_plan(68, 16, 512, 1000, [2000] * 68)
    assert p["table_sort"] and p["interact_bwd_shared"] is True
    # ... but not beside the radix scatter's static LDS
    p = ops.bwd_plan(68, 16, 512, 140_000, [2000] * 68)
    assert not p["table_sort"] and p["interact_bwd_shared"] is False
    assert p["max_lds"] <= 160 * 1024
    # 65 tables, D = 512, 17-bit keys: two 9-bit passes (their scatter keeps 10 KiB of LDS): own launch
    p = ops.bwd_plan(65, 24, 512, 140_000, [2000] * 65)
    assert (p["table_sort"], p["radix_bits"], p["passes"], p["interact_bwd_shared"]) == (False, 9, 2, False)
    # the same with 24-bit keys (three 8-bit passes, a 5 KiB scatter): still too large together
    p = ops.bwd_plan(65, 24, 512, 140_000, [200_000] * 65)
    assert (p["radix_bits"], p["passes"]) == (8, 3)
    assert p["interact_bwd_shared"] is (_ibwd_lds(65, 512) + 5136 + 256 <= 160 * 1024)
    # no occurrences: no sort passes, the interaction backward runs alone
    p = ops.bwd_plan(4, 8, 16, 0, [10] * 4)
    assert p["passes"] == 0 and p["interact_bwd_shared"] is False and p["table_sort"] is False
    # one sample's tile alone beyond 160 KiB
    plan = (ctypes.c_int32 * 5)()
    rows = (ctypes.c_int64 * 128)(*([10] * 128))
    assert lib.dlrm_embbag_bwd_plan(128, 4, 512, 8, rows, 1, plan) == E_UNSUPPORTED
    assert lib.dlrm_embbag_bwd_plan(0, 4, 512, 8, rows, 1, plan) == E_INVAL


def test_binding_rejects_wrong_sized_buffers_before_any_call():
    """The C ABI takes raw pointers and cannot see an undersized caller buffer, so the
    binding checks every buffer's element count and dtype first (host tensors here: the
    size check fires before the device check)."""
    import torch

    T, B, D = 3, 4, 16
    P = ops.pair_count(T)
    tabs = [torch.zeros((10, D), dtype=torch.float32) for _ in range(T)]
    off = torch.zeros(T * B + 1, dtype=torch.int32)
    idx = torch.zeros(0, dtype=torch.int32)
    e0 = torch.zeros((B, D), dtype=torch.float32)

    def fwd(**kw):
        args = dict(offsets=off, indices=idx, e0=e0)
        args.update(kw)
        return ops.embbag_fwd(tabs, args["offsets"], args["indices"], B, args["e0"],
                              out_inter=kw.get("out_inter"), out_pooled=kw.get("out_pooled"),
                              status=kw.get("status"))

    with pytest.raises(ValueError, match="offsets has"):
        fwd(offsets=torch.zeros(T * B, dtype=torch.int32))
    with pytest.raises(ValueError, match="offsets must be"):
        fwd(offsets=torch.zeros(T * B + 1, dtype=torch.int64))
    with pytest.raises(ValueError, match="indices must be"):
        fwd(indices=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="e0 has"):
        fwd(e0=torch.zeros((B - 1, D), dtype=torch.float32))
    with pytest.raises(ValueError, match="out_inter has"):
        fwd(out_inter=torch.zeros((B, D + P - 1), dtype=torch.float32))
    with pytest.raises(ValueError, match="out_pooled has"):
        fwd(out_pooled=torch.zeros((B, T, D - 4), dtype=torch.float32))
    with pytest.raises(ValueError, match="out_pooled must be"):
        fwd(out_pooled=torch.zeros((B, T, D), dtype=torch.float16))
    with pytest.raises(ValueError, match="status has"):
        fwd(status=torch.zeros(0, dtype=torch.int32))
    # correctly sized host tensors pass the size checks and stop at the device check
    with pytest.raises(ValueError, match="CUDA"):
        fwd(out_inter=torch.zeros((B, D + P), dtype=torch.float32))

    pooled = torch.zeros((B, T, D), dtype=torch.float32)
    d_out = torch.zeros((B, D + P), dtype=torch.float32)
    with pytest.raises(ValueError, match="pooled has"):
        ops.embbag_bwd_update(tabs, off, idx, B, e0, pooled[:, :-1], d_out, 0.01)
    with pytest.raises(ValueError, match="d_out has"):
        ops.embbag_bwd_update(tabs, off, idx, B, e0, pooled, d_out[:, :-1], 0.01)
    with pytest.raises(ValueError, match="workspace has"):
        ops.embbag_bwd_update(tabs, off, idx, B, e0, pooled, d_out, 0.01, workspace=torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="d_e0 has"):
        ops.BwdPlan(tabs, off, idx, B, e0, pooled, d_out, 0.01, d_e0=torch.zeros(B * D - 1))
    with pytest.raises(ValueError, match="CUDA"):
        ops.embbag_bwd_update(tabs, off, idx, B, e0, pooled, d_out, 0.01)
    with pytest.raises(ValueError, match="out has"):
        ops.interact(e0, pooled, out=torch.zeros((B, D + P + 1), dtype=torch.float32))
    with pytest.raises(ValueError, match="d_pooled has"):
        ops.interact_bwd(e0, pooled, d_out, d_pooled=torch.zeros((B, T, D + 4), dtype=torch.float32))
    with pytest.raises(ValueError, match="lengths must be"):
        ops.lengths_to_offsets(torch.zeros(4, dtype=torch.int64))
