"""GPU parity of the sparse backward + SGD update against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import dlrm_oracle as orc
from sparse_embedding_lookup_dlrm_amd import ops, synth

from gpu_util import DeviceBatch, RTOL, abs_tables, assert_mag_close, host_tables, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _round_storage(x64, dtype):
    x32 = torch.from_numpy(np.asarray(x64, dtype=np.float32))
    if dtype == "f32":
        return x32.numpy()
    if dtype == "f16":
        return x64.astype(np.float32).astype(np.float16)
    return x32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def set_lengths(b: synth.Batch, lengths) -> None:
    """Give the batch other bag lengths (table-major), with fresh indices for them."""
    b.lengths = np.asarray(lengths, dtype=np.int32)
    b.indices = synth.gen_indices(b.w, b.rows, b.lengths)


def sort_plan(w: synth.Workload, nnz: int) -> dict:
    return ops.bwd_plan(w.T, w.B, w.D, nnz, synth.table_rows(w))


def run_bwd(w: synth.Workload, lr=0.01, exact=False, twice=False, fused_fwd=True, layout=0, lengths=None,
            table_sort=None):
    """Backward + SGD against the oracle. lengths replaces the bag lengths; table_sort, if
    given, is whether the call must sort per table (else by radix passes over all keys)."""
    b = synth.make_batch(w, with_dout=True)
    if lengths is not None:
        set_lengths(b, lengths)
    if table_sort is not None:
        assert sort_plan(w, len(b.indices))["table_sort"] is table_sort
    self_pairs = bool(layout & ops.PAIRS_SELF)
    with_emb = bool(layout & ops.WITH_EMBEDDINGS)
    if layout:
        b.dout = synth.gen_dout(w, ops.out_width(w.T, w.D, layout))
    db = DeviceBatch(b)
    pooled, _ = db.fwd(want_pooled=True, want_inter=fused_fwd, layout=layout)
    d_out = torch.from_numpy(b.dout).cuda()
    before = [t.clone() for t in db.tables]
    res = ops.embbag_bwd_update(db.tables, db.offsets, db.indices, w.B, db.e0, pooled, d_out, lr, status=db.status,
                                layout=layout)
    torch.cuda.synchronize()
    assert db.status.item() == 0
    if twice:
        tabs2 = [t.clone() for t in before]
        res2 = ops.embbag_bwd_update(tabs2, db.offsets, db.indices, w.B, db.e0, pooled, d_out, lr, layout=layout)
        torch.cuda.synchronize()
        U1 = int(res["num_unique"].item())
        assert U1 == int(res2["num_unique"].item())
        nnz = int(db.indices.numel())
        lim = {"d_e0": None, "perm": nnz, "unique_keys": U1, "seg_offsets": U1 + 1}
        for k, n in lim.items():
            assert torch.equal(res[k][:n], res2[k][:n]), k
        for t1, t2 in zip(db.tables, tabs2):
            assert torch.equal(t1.view(torch.int16) if t1.dtype != torch.float32 else t1,
                               t2.view(torch.int16) if t2.dtype != torch.float32 else t2)
        # without the segment outputs (not built then): the same update and d_e0, bit for bit
        tabs3 = [t.clone() for t in before]
        res3 = ops.embbag_bwd_update(tabs3, db.offsets, db.indices, w.B, db.e0, pooled, d_out, lr,
                                     want_segments=False, layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(res["d_e0"], res3["d_e0"])
        for t1, t3 in zip(db.tables, tabs3):
            assert torch.equal(t1.view(torch.int16) if t1.dtype != torch.float32 else t1,
                               t3.view(torch.int16) if t3.dtype != torch.float32 else t3)

    # oracle (own pooled, own offsets)
    off = orc.lengths_to_offsets(b.lengths)
    fwd = orc.embbag_fwd(b.tables, w.dtype, w.B, off, b.indices, b.e0)
    r = orc.embbag_bwd_update(b.tables, w.dtype, w.B, off, b.indices, b.e0, fwd["pooled"], b.dout, lr,
                              self_pairs=self_pairs, with_embeddings=with_emb)
    # magnitudes: the same computation on absolute values
    at = abs_tables(b.tables, w.dtype)
    pm = orc.embbag_pool(at, w.dtype, w.B, off, b.indices)
    rm = orc.embbag_bwd_update(at, w.dtype, w.B, off, b.indices, np.abs(b.e0), pm, np.abs(b.dout), lr,
                               self_pairs=self_pairs, with_embeddings=with_emb)

    U = int(res["num_unique"].item())
    nnz = len(b.indices)
    assert U == len(r["unique_keys"])
    np.testing.assert_array_equal(res["perm"].cpu().numpy()[:nnz], r["perm"].astype(np.int32))
    np.testing.assert_array_equal(res["unique_keys"].cpu().numpy()[:U], r["unique_keys"].astype(np.int32))
    np.testing.assert_array_equal(res["seg_offsets"].cpu().numpy()[:U + 1], r["seg_offsets"].astype(np.int32))
    rtol = 0.0 if exact else RTOL[w.dtype]
    de0_mag = np.abs(b.dout[:, :w.D]) + rm["dZ"][:, 0]
    assert_mag_close(res["d_e0"].cpu().numpy(), r["d_e0"], de0_mag, rtol, "d_e0")

    # tables: touched rows updated, untouched rows bit-identical
    after = host_tables(db.tables, w.dtype)
    orig = host_tables(before, w.dtype)
    base = r["base"]
    touched = [np.zeros(t.shape[0], bool) for t in orig]
    for k in r["unique_keys"]:
        t = int(np.searchsorted(base, k, side="right") - 1)
        touched[t][k - base[t]] = True
    for t in range(w.T):
        np.testing.assert_array_equal(after[t][~touched[t]], orig[t][~touched[t]])
    keys = np.asarray(r["unique_keys"], dtype=np.int64)
    tix = np.searchsorted(base, keys, side="right") - 1
    rix = keys - base[tix]
    got_rows = np.array([orc.decode(after[t][i][None], w.dtype)[0] for t, i in zip(tix, rix)]).reshape(U, w.D)
    W_mag = np.abs(np.array([orc.decode(orig[t][i][None], w.dtype)[0] for t, i in zip(tix, rix)]).reshape(U, w.D))
    if exact:
        want = _round_storage(r["new_rows"], w.dtype)
        np.testing.assert_array_equal(got_rows, orc.decode(want, w.dtype))
    else:
        # storage rounding of the result adds half an ulp of the stored format
        store_ulp = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[w.dtype]
        mag = W_mag + lr * rm["grad"]
        lim_mag = mag + (store_ulp / rtol) * np.abs(r["new_rows"])
        assert_mag_close(got_rows, r["new_rows"], lim_mag, rtol, "updated rows")
    return res, r


def test_backward_zipf_26_tables_full():
    """Backward + SGD (lr = 0.01) on the 26-table Zipf(1.05) workload, full size (one
    index per bag: 2048 occurrences per table, sorted per table)."""
    run_bwd(synth.WORKLOADS["bwd-zipf-26t-d128-b2048"], lr=0.01, twice=True, table_sort=True)


@pytest.mark.parametrize("name", ["tiny-4t1k-d16-b128", "bwd-zipf-26t-d128-b2048"])
def test_backward_exact_arithmetic(name):
    w = synth.WORKLOADS[name].replace(values="int")
    run_bwd(w, lr=2.0 ** -7, exact=True)


@pytest.mark.parametrize("layout", [1, 2, 3])
@pytest.mark.parametrize("T,D,dtype,B", [(26, 128, "bf16", 300), (3, 16, "f32", 50), (30, 64, "f32", 70)])
def test_backward_interaction_layouts(layout, T, D, dtype, B):
    """The sparse backward for a forward in each interaction layout (self-pairs, the
    embeddings concatenated, both): the interaction-backward share inside the sort and,
    at T = 3, the small case."""
    w = synth.Workload(f"blayout-{T}t-d{D}", T=T, rows=500, D=D, dtype=dtype, B=B, bag=("uniform", 0, 6),
                       dist=("zipf", 1.1), seed=T * 7 + layout)
    run_bwd(w, lr=0.01, twice=(T == 26), layout=layout)


@pytest.mark.parametrize("layout", [1, 2, 3])
def test_backward_interaction_layouts_exact(layout):
    w = synth.WORKLOADS["tiny-4t1k-d16-b128"].replace(values="int")
    run_bwd(w, lr=2.0 ** -7, exact=True, layout=layout)


def test_backward_interaction_layout_own_launch():
    """Self-pairs and the embeddings at T = 65, D = 512 bf16: the interaction backward in
    its own launch, in the layout."""
    w = synth.Workload("ibwd-own-layout", T=65, rows=2000, D=512, dtype="bf16", B=24, bag=("uniform", 85, 95),
                       dist=("zipf", 1.1), seed=653)
    nnz = int(synth.make_batch(w).indices.size)
    p = ops.bwd_plan(w.T, w.B, w.D, nnz, [2000] * w.T)
    assert not p["interact_bwd_shared"] and not p["table_sort"]
    run_bwd(w, lr=0.01, fused_fwd=False, layout=3)


def test_backward_multihot_fp16():
    w = synth.WORKLOADS["multihot-8t4m-d64-fp16-b4096"].replace(B=512, rows=200_000)
    run_bwd(w, lr=0.01, table_sort=False)


def test_backward_capacity_shape_bf16():
    w = synth.WORKLOADS[synth.CAPACITY].replace(B=48, rows=3000)
    run_bwd(w, lr=0.01, twice=True)


@pytest.mark.parametrize("T,D,B", [(1, 4, 1), (3, 16, 5), (7, 256, 9), (20, 32, 300)])
def test_backward_shapes(T, D, B):
    w = synth.Workload("bshape", T=T, rows=40, D=D, dtype="f32", B=B, bag=("uniform", 0, 12),
                       dist=("zipf", 1.2), seed=T * 100 + D)
    run_bwd(w, lr=0.05)


def test_backward_many_keys_9bit_digits():
    """sum(rows) = 18M: 25-bit keys, sorted in three 9-bit passes (8-bit digits would
    need four)."""
    w = synth.Workload("bigkeys", T=3, rows=6_000_000, D=8, dtype="bf16", B=700, bag=("uniform", 0, 9),
                       dist=("zipf", 1.05), seed=77)
    run_bwd(w, lr=0.01, table_sort=False)


def test_backward_9bit_digits_row_scan():
    """25-bit keys (three 9-bit passes) over about 410K occurrences: about 200 sort tiles,
    so each digit's offsets come from the row-scan launch, over 512 digit rows."""
    w = synth.Workload("bigkeys-rs", T=3, rows=6_000_000, D=8, dtype="bf16", B=2100, bag=("uniform", 60, 70),
                       dist=("zipf", 1.05), seed=78)
    run_bwd(w, lr=0.01, table_sort=False)


@pytest.mark.parametrize("T,rows,B,bag", [
    (1, 200, 600, ("uniform", 0, 12)),  # 8-bit keys: one 8-bit pass
    (1, 400, 600, ("uniform", 0, 12)),  # 9 bits: one 9-bit pass
    (3, 500, 1200, ("uniform", 0, 12)),  # 11 bits: two 8-bit passes
    (2, 50_000, 900, ("uniform", 0, 12)),  # 17 bits: two 9-bit passes
    (3, 1_000_000, 2000, ("uniform", 10, 14)),  # 22 bits: three 8-bit passes, 36 tiles
    (2, 5_000_000, 500, ("uniform", 0, 12)),  # 24 bits: three 8-bit passes, the last digit full
])
def test_backward_sort_pass_counts(T, rows, B, bag):
    """The sort takes as many passes as the key width needs (the sentinel sum(rows)
    included), with 9-bit digits where they save a pass: one to three passes here, three
    9-bit passes of 25-bit keys in the test above."""
    w = synth.Workload("passes", T=T, rows=rows, D=8, dtype="f32", B=B, bag=bag, dist=("zipf", 1.05),
                       seed=rows % 997 + B)
    run_bwd(w, lr=0.01, table_sort=False)


@pytest.mark.parametrize("B,bag", [(2100, ("uniform", 60, 70)), (8200, ("uniform", 62, 68))])
def test_backward_sort_and_segment_paths(B, bag):
    """About 273K occurrences (134 sort tiles of 2048: the sort's offsets come from a
    device-wide scan rather than inside each tile) and about 1.07M (more than 256 scan
    chunks of 4096: the segment scan also takes the device-wide path)."""
    w = synth.Workload("paths", T=2, rows=3000, D=8, dtype="f32", B=B, bag=bag, dist=("zipf", 1.05), seed=B)
    run_bwd(w, lr=0.01, table_sort=False)


@pytest.mark.parametrize("B,twice", [(2048, True), (2040, False), (2064, False)])
def test_backward_sort_tile_count_boundary(B, twice):
    """Bags of exactly 64 over 2 tables: 128 full sort tiles (the most whose scatter sums its
    digit offsets from the count table itself), 127.5 tiles (a ragged last tile) and 129 tiles
    (the offsets come from a per-digit scan launch). The run twice matches bit for bit."""
    w = synth.Workload("tiles", T=2, rows=3000, D=8, dtype="f32", B=B, bag=("fixed", 64),
                       dist=("zipf", 1.05), seed=B + 5)
    res, r = run_bwd(w, lr=0.01, twice=twice, table_sort=False)
    assert len(r["perm"]) == 2 * 64 * B


@pytest.mark.parametrize("name,T,rows,B,spec", [
    # about 4096 occurrences in table 0 (two tiles, sorted through the workspace), 13-bit rows
    ("long-table", 4, 5000, 512, [(4, 12), (0, 2), (0, 2), (0, 2)]),
    # about 4800 occurrences in table 1 (three tiles) with 17-bit rows: three passes
    ("long-table-3p", 3, 100_000, 600, [(0, 1), (6, 10), (0, 1)]),
    # the last of five tables holds about 4000 occurrences (two tiles); the others one tile each
    ("long-last", 5, 5000, 400, [(0, 2)] * 4 + [(8, 12)]),
    # 2049 occurrences in table 0 (one more than a tile) and 2047 in table 1
    ("tile-plus-one", 2, 3000, 2049, None),
    # an empty table between two others
    ("empty-table", 3, 700, 400, [(1, 5), (0, 0), (1, 5)]),
    # 256 rows: the out-of-range key 256 needs a ninth bit, so two passes
    ("pow2-rows", 3, 256, 300, [(0, 6)] * 3),
    # a single row per table: keys 0 or 1, one pass
    ("one-row", 2, 1, 100, [(0, 3)] * 2),
])
def test_backward_per_table_sort(name, T, rows, B, spec):
    """Batches of at most 2048 occurrences per table on average sort per table: table
    ranges longer than one tile (first, middle or last table; the final order then comes
    from the placement launch, not from the ranges written in place), a tile plus one, an
    empty table, rows at a power of two and a single row; perm, segments and U bit-exact,
    the update within tolerance, and a second run bit-identical."""
    w = synth.Workload(name, T=T, rows=rows, D=16, dtype="f32", B=B, bag=("uniform", 0, 1),
                       dist=("zipf", 1.1), seed=len(name) * 31 + B)
    rng = np.random.default_rng(w.seed)
    if spec is None:
        lengths = np.ones(T * B, np.int32)
        lengths[B + rng.choice(B, 2, replace=False)] = 0
    else:
        lengths = np.concatenate([rng.integers(lo, hi + 1, B) for lo, hi in spec]).astype(np.int32)
    run_bwd(w, lr=0.01, twice=True, lengths=lengths, table_sort=True)


@pytest.mark.parametrize("B", [8192, 8193])
def test_backward_segment_outputs_chunk_boundary(B):
    """D = 8 reduces 32 sorted positions per chunk. Bags of exactly 64 over 2 tables give
    32768 chunks (the most for which the combine step writes the segment outputs from the
    reduce's head counts) and 32772 (a device-wide scan builds them)."""
    w = synth.Workload("segs", T=2, rows=3000, D=8, dtype="f32", B=B, bag=("fixed", 64),
                       dist=("zipf", 1.05), seed=B + 11)
    run_bwd(w, lr=0.01, twice=True)


def test_backward_segment_outputs_one_pass_scan():
    """D = 256 reduces 8 positions per chunk: 307,200 occurrences are 38,400 chunks (too
    many for the combine step) but 75 scan chunks of 4096, so the segment outputs come from
    the chunk totals and one scan-and-write pass."""
    w = synth.Workload("segs1", T=2, rows=3000, D=256, dtype="f32", B=2400, bag=("fixed", 64),
                       dist=("zipf", 1.05), seed=2411)
    run_bwd(w, lr=0.01, twice=True)


@pytest.mark.parametrize("B,table_sort", [(50, True), (2000, False)])
def test_backward_positions_outside_every_bag_are_skipped(B, table_sort):
    """Offsets that start at 3 and end 5 short of nnz (invalid, flagged): the positions
    before the first offset and from the last one on belong to no bag and add nothing
    (sorted per table, and by radix passes over all keys)."""
    w = synth.Workload("gaps", T=3, rows=200, D=32, dtype="f32", B=B, bag=("uniform", 0, 8),
                       dist=("zipf", 1.1), seed=91)
    b = synth.make_batch(w, with_dout=True)
    assert sort_plan(w, len(b.indices) + 8)["table_sort"] is table_sort
    db = DeviceBatch(b)
    pooled, _ = db.fwd(want_pooled=True)
    d_out = torch.from_numpy(b.dout).cuda()
    rng = np.random.default_rng(5)
    off = orc.lengths_to_offsets(b.lengths)
    nnz = len(b.indices)
    # three extra occurrences in front, five behind: the offsets shift by 3 and nnz grows by 8
    idx = np.concatenate([rng.integers(0, 200, 3), b.indices, rng.integers(0, 200, 5)]).astype(np.int32)
    off_dev = torch.from_numpy((off + 3).astype(np.int32)).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    before = [t.clone() for t in db.tables]
    res = ops.embbag_bwd_update(db.tables, off_dev, torch.from_numpy(idx).cuda(), w.B, db.e0, pooled, d_out, 0.01,
                                status=st)
    torch.cuda.synchronize()
    assert st.item() & ops.STATUS_BAD_OFFSETS
    # the same update as the valid batch
    tabs2 = [t.clone() for t in before]
    ops.embbag_bwd_update(tabs2, db.offsets, db.indices, w.B, db.e0, pooled, d_out, 0.01)
    torch.cuda.synchronize()
    for t1, t2 in zip(db.tables, tabs2):
        assert torch.equal(t1, t2)
    assert int(res["num_unique"].item()) == len(np.unique(b.indices + np.repeat(
        np.array([0, 200, 400]), [int(b.lengths[t * w.B:(t + 1) * w.B].sum()) for t in range(w.T)])))
    assert nnz + 8 == len(idx)


@pytest.mark.parametrize("T,rows,B", [(3, 200, 50), (26, 40_000, 300), (2, 3000, 1500)])
def test_backward_overlapping_bags_stay_in_bounds(T, rows, B):
    """Offsets that decrease (invalid, flagged) make later bags cover positions that an
    earlier bag already covers. The call still finishes in bounds: the status carries
    the flag, rows that no index references stay bit-identical, the distinct rows are
    strictly increasing keys of referenced rows, and d_e0 is the interaction gradient."""
    w = synth.Workload("overlap", T=T, rows=rows, D=32, dtype="f32", B=B, bag=("uniform", 1, 8),
                       dist=("zipf", 1.1), seed=T + B)
    b = synth.make_batch(w, with_dout=True)
    db = DeviceBatch(b)
    pooled, _ = db.fwd(want_pooled=True)
    d_out = torch.from_numpy(b.dout).cuda()
    off = orc.lengths_to_offsets(b.lengths).astype(np.int64)
    # bag 4 now runs to the end of bag 8; bag 5 (from there to its old end) is empty
    # and bags 6..8 are covered twice
    bad = off.copy()
    bad[5] = off[9]
    assert bad[5] > bad[6] > bad[4]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    before = [t.clone() for t in db.tables]
    res = ops.embbag_bwd_update(db.tables, torch.from_numpy(bad.astype(np.int32)).cuda(), db.indices, w.B, db.e0,
                                pooled, d_out, 0.01, status=st)
    ref = ops.embbag_bwd_update([t.clone() for t in before], db.offsets, db.indices, w.B, db.e0, pooled, d_out, 0.01)
    torch.cuda.synchronize()
    assert st.item() & ops.STATUS_BAD_OFFSETS
    assert torch.equal(res["d_e0"], ref["d_e0"])
    base = np.arange(T + 1, dtype=np.int64) * rows
    U = int(res["num_unique"].item())
    uk = res["unique_keys"].cpu().numpy()[:U].astype(np.int64)
    assert np.all(np.diff(uk) > 0)
    for t in range(T):
        referenced = np.zeros(rows, dtype=bool)
        referenced[b.indices[off[t * B]:off[(t + 1) * B]]] = True
        mine = uk[(uk >= base[t]) & (uk < base[t + 1])] - base[t]
        assert referenced[mine].all()
        untouched = torch.from_numpy(~referenced).cuda()
        assert torch.equal(before[t][untouched], db.tables[t][untouched])


def test_backward_hot_rows_span_many_chunks():
    """Multi-hot fp16 bags with a Zipf(1.1) hot row per table: its occurrences fill
    dozens of consecutive reduction chunks, whose partial sums are chained in order
    (and must give the same bits on a second run)."""
    w = synth.Workload("hot-8t20k-d64-fp16-b1024", T=8, rows=20_000, D=64, dtype="f16", B=1024,
                       bag=("poisson", 20, 100), dist=("zipf", 1.1), seed=41)
    run_bwd(w, lr=0.01, twice=True)


@pytest.mark.parametrize("B", [32, 64, 65, 96, 1000])
def test_backward_single_row_whole_batch(B):
    """Every occurrence hits the same row: one segment across every chunk, for batch
    sizes that end on and off a chunk boundary."""
    w = synth.Workload("onerow", T=1, rows=1, D=128, dtype="f32", B=B, bag=("fixed", 1),
                       dist=("uniform",), seed=B)
    run_bwd(w, lr=0.01, twice=True)


@pytest.mark.parametrize("D,B,dtype", [(16, 5000, "f32"), (256, 1000, "bf16"), (512, 3000, "bf16")])
def test_backward_single_row_long_segment_widths(D, B, dtype):
    """One row takes every occurrence at 1, 4 and 8 gradient columns per lane (16 of 64 lanes
    holding a row at D = 16): its partial sums span hundreds of chunks, most of them summed
    per reduce workgroup before the combine step adds them; sorted per table (B = 1000) and
    by radix passes (B = 3000, 5000)."""
    w = synth.Workload("onerow-w", T=1, rows=1, D=D, dtype=dtype, B=B, bag=("fixed", 1),
                       dist=("uniform",), seed=B + D)
    run_bwd(w, lr=0.01, twice=True, table_sort=(B <= 2048))


def _random_case(i):
    """Seeded shapes across both sorts, the four gradient widths and the three storage
    types (bags uniform in [0, hi], rows per table a few hundred to a few hundred thousand)."""
    rng = np.random.default_rng(9000 + i)
    T = int(rng.integers(1, 40))
    D = int(rng.choice([16, 32, 64, 128, 256, 512]))
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    B = int(rng.integers(1, 700))
    hi = int(rng.choice([1, 3, 8, 40]))
    rows = int(rng.choice([100, 3000, 70_000, 300_000]))
    rows = min(rows, 20_000_000 // (T * D))  # at most 20M table elements
    return synth.Workload(f"rand{i}", T=T, rows=rows, D=D, dtype=dtype, B=B, bag=("uniform", 0, hi),
                          dist=("zipf", float(rng.choice([1.05, 1.2]))), seed=9000 + i)


@pytest.mark.parametrize("i", range(12))
def test_backward_random_shapes(i):
    """Backward + SGD on seeded random shapes against the oracle (perm, segments and U
    bit-exact, the update within tolerance, a second run bit-identical)."""
    run_bwd(_random_case(i), lr=0.01, twice=True)


def test_backward_wide_rows_bf16():
    """D = 512 bf16 (eight fp32 gradient columns per lane)."""
    w = synth.Workload("wide", T=2, rows=50, D=512, dtype="bf16", B=40, bag=("uniform", 0, 20),
                       dist=("zipf", 1.2), seed=512)
    run_bwd(w, lr=0.01, twice=True)


def run_bwd_adagrad(w: synth.Workload, lr=0.05, eps=1e-6, steps=2, layout=0):
    """Row-wise AdaGrad over `steps` identical backward calls (the state carries over),
    checked after every step against the oracle run from the same tables and state."""
    b = synth.make_batch(w, with_dout=True)
    self_pairs = bool(layout & ops.PAIRS_SELF)
    with_emb = bool(layout & ops.WITH_EMBEDDINGS)
    if layout:
        b.dout = synth.gen_dout(w, ops.out_width(w.T, w.D, layout))
    db = DeviceBatch(b)
    pooled, _ = db.fwd(want_pooled=True)
    d_out = torch.from_numpy(b.dout).cuda()
    rng = np.random.default_rng(w.seed)
    state_h = [rng.uniform(0.0, 1e-4, size=n).astype(np.float32) for n in (t.shape[0] for t in b.tables)]
    state = [torch.from_numpy(s).cuda() for s in state_h]
    off = orc.lengths_to_offsets(b.lengths)
    fwd = orc.embbag_fwd(b.tables, w.dtype, w.B, off, b.indices, b.e0)
    at = abs_tables(b.tables, w.dtype)
    pm = orc.embbag_pool(at, w.dtype, w.B, off, b.indices)
    rm = orc.embbag_bwd_update(at, w.dtype, w.B, off, b.indices, np.abs(b.e0), pm, np.abs(b.dout), lr,
                               self_pairs=self_pairs, with_embeddings=with_emb)
    tabs_now = [t.copy() for t in b.tables]
    rtol = RTOL[w.dtype]
    store_ulp = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[w.dtype]
    for step in range(steps):
        before_state = [s.clone() for s in state]
        res = ops.embbag_bwd_update(db.tables, db.offsets, db.indices, w.B, db.e0, pooled, d_out, lr,
                                    status=db.status, row_state=state, eps=eps, layout=layout)
        torch.cuda.synchronize()
        assert db.status.item() == 0
        s_prev = [s.cpu().numpy().astype(np.float64) for s in before_state]
        # the oracle keeps the pooled vectors of the original tables, as the GPU call does
        r = orc.embbag_bwd_update(tabs_now, w.dtype, w.B, off, b.indices, b.e0, fwd["pooled"], b.dout, lr,
                                  optimizer="rowwise_adagrad", state=s_prev, eps=eps, self_pairs=self_pairs,
                                  with_embeddings=with_emb)
        U = int(res["num_unique"].item())
        assert U == len(r["unique_keys"])
        base = r["base"]
        keys = np.asarray(r["unique_keys"], dtype=np.int64)
        tix = np.searchsorted(base, keys, side="right") - 1
        rix = keys - base[tix]
        after = host_tables(db.tables, w.dtype)
        got_rows = np.array([orc.decode(after[t][i][None], w.dtype)[0] for t, i in zip(tix, rix)]).reshape(U, w.D)
        was = np.array([orc.decode(tabs_now[t][i][None], w.dtype)[0] for t, i in zip(tix, rix)]).reshape(U, w.D)
        got_state = np.array([state[t][i].item() for t, i in zip(tix, rix)])
        s_old = np.array([s_prev[t][i] for t, i in zip(tix, rix)])
        # tolerances: G is within rtol * M_G; s = s_old + mean(G^2) then moves by at most
        # 2 rtol mean(|G| M_G) (plus its own rounding); the step lr G / (sqrt(s) + eps)
        # by at most rtol lr (M_G + |G| mean(|G| M_G) / s) / sqrt(s)
        g, mg = r["grad"], rm["grad"]
        sm = (s_old + 2 * np.mean(np.abs(g) * mg, axis=1)) + np.abs(r["new_state"])
        assert_mag_close(got_state, r["new_state"], sm, rtol, "state")
        root = np.sqrt(r["new_state"])[:, None] + eps
        cross = (np.mean(np.abs(g) * mg, axis=1) / r["new_state"])[:, None]
        step_mag = lr * (mg + np.abs(g) * cross) / root
        lim = np.abs(was) + 3 * step_mag + (store_ulp / rtol) * np.abs(r["new_rows"])
        assert_mag_close(got_rows, r["new_rows"], lim, rtol, f"updated rows, step {step}")
        # untouched rows and states stay as they were
        touched = [np.zeros(t.shape[0], bool) for t in tabs_now]
        for t, i in zip(tix, rix):
            touched[t][i] = True
        for t in range(w.T):
            np.testing.assert_array_equal(after[t][~touched[t]], tabs_now[t][~touched[t]])
            np.testing.assert_array_equal(state[t].cpu().numpy()[~touched[t]], before_state[t].cpu().numpy()[~touched[t]])
        tabs_now = [a.copy() for a in after]


def test_backward_rowwise_adagrad_zipf_26_tables():
    run_bwd_adagrad(synth.WORKLOADS["bwd-zipf-26t-d128-b2048"], lr=0.01)


def test_backward_rowwise_adagrad_single_row_long_segment():
    """Row-wise AdaGrad where one row takes all 4000 occurrences (D = 64): the state step of a
    segment summed through hundreds of chunks and their workgroup sums."""
    w = synth.Workload("onerow-ada", T=1, rows=1, D=64, dtype="f32", B=4000, bag=("fixed", 1),
                       dist=("uniform",), seed=4064)
    run_bwd_adagrad(w, lr=0.01)


def test_backward_rowwise_adagrad_hot_rows_fp16():
    w = synth.Workload("hot-ada-8t5k-d64-fp16-b512", T=8, rows=5_000, D=64, dtype="f16", B=512,
                       bag=("poisson", 20, 100), dist=("zipf", 1.1), seed=43)
    run_bwd_adagrad(w, lr=0.01)


@pytest.mark.parametrize("T,D,B,dtype", [(3, 16, 40, "f32"), (2, 256, 30, "bf16"), (1, 512, 20, "bf16")])
def test_backward_rowwise_adagrad_shapes(T, D, B, dtype):
    w = synth.Workload("ada-shape", T=T, rows=60, D=D, dtype=dtype, B=B, bag=("uniform", 0, 10),
                       dist=("zipf", 1.2), seed=T * 10 + D)
    run_bwd_adagrad(w, lr=0.02, steps=3)


@pytest.mark.parametrize("layout", [1, 2, 3])
def test_backward_rowwise_adagrad_layouts(layout):
    """Row-wise AdaGrad through dlrm_embbag_bwd_update_ex for a forward in each layout."""
    w = synth.Workload("ada-layout", T=26, rows=400, D=64, dtype="bf16", B=80, bag=("uniform", 0, 6),
                       dist=("zipf", 1.1), seed=300 + layout)
    run_bwd_adagrad(w, lr=0.02, steps=2, layout=layout)


def test_backward_plan_matches_call_sgd_and_adagrad():
    """BwdPlan (arguments marshalled once, as the benchmark times it) gives the same bits as
    embbag_bwd_update for SGD and for row-wise AdaGrad, over two steps (tables and row states
    carried from the first step to the second)."""
    w = synth.Workload("plan-6t-d64-f32", T=6, rows=300, D=64, dtype="f32", B=200, bag=("uniform", 0, 9),
                       dist=("zipf", 1.1), seed=91)
    b = synth.make_batch(w, with_dout=True)
    db = DeviceBatch(b)
    pooled, _ = db.fwd(want_pooled=True)
    d_out = torch.from_numpy(b.dout).cuda()
    for adagrad in (False, True):
        tabs_a = [t.clone() for t in db.tables]
        tabs_b = [t.clone() for t in db.tables]
        st_a = [torch.zeros(t.shape[0], dtype=torch.float32, device="cuda") for t in db.tables] if adagrad else None
        st_b = [s.clone() for s in st_a] if adagrad else None
        d_e0 = torch.empty((w.B, w.D), dtype=torch.float32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        plan = ops.BwdPlan(tabs_b, db.offsets, db.indices, w.B, db.e0, pooled, d_out, 0.01, d_e0=d_e0,
                           status=status, row_state=st_b)
        for _ in range(2):
            res = ops.embbag_bwd_update(tabs_a, db.offsets, db.indices, w.B, db.e0, pooled, d_out, 0.01,
                                        row_state=st_a)
            plan.run()
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            assert torch.equal(res["d_e0"], d_e0)
            U = int(res["num_unique"].item())
            assert U == int(plan.num_unique.item())
            assert torch.equal(res["unique_keys"][:U], plan.unique_keys[:U])
            assert torch.equal(res["seg_offsets"][:U + 1], plan.seg_offsets[:U + 1])
            for ta, tb in zip(tabs_a, tabs_b):
                assert torch.equal(ta, tb)
            if adagrad:
                for sa, sb in zip(st_a, st_b):
                    assert torch.equal(sa, sb)


def test_backward_interaction_backward_own_launch():
    """65 bf16 tables with D = 512 and 17-bit keys (two 9-bit sort passes): one sample's
    interaction-backward LDS does not fit beside the 9-bit scatter's own within 160 KiB, so
    the interaction backward runs as a launch of its own instead of riding on the sort's."""
    w = synth.Workload("ibwd-own-65t-d512-bf16", T=65, rows=2000, D=512, dtype="bf16", B=24,
                       bag=("uniform", 85, 95), dist=("zipf", 1.1), seed=655)
    nnz = int(synth.make_batch(w).indices.size)
    p = ops.bwd_plan(w.T, w.B, w.D, nnz, [2000] * w.T)
    assert (p["radix_bits"], p["passes"], p["interact_bwd_shared"], p["table_sort"]) == (9, 2, False, False)
    run_bwd(w, lr=0.01, twice=True, fused_fwd=False)


@pytest.mark.parametrize("dtype,T,D,B,long0,table_sort", [
    ("f32", 5, 32, 64, False, True),
    ("bf16", 26, 128, 64, False, True),
    ("f32", 5, 32, 300, True, True),  # table 0 holds about 3000 occurrences: sorted tile by tile
    ("f32", 2, 32, 1500, False, False),  # radix passes over all keys
])
def test_backward_out_of_range_indices_dropped(dtype, T, D, B, long0, table_sort):
    """One out-of-range index per table (one of them negative): the status carries the
    bad-index bit, and perm, the distinct rows, the segment bounds and U equal the oracle's
    on the batch without those occurrences (positions mapped back; the dropped ones sort
    last, in CSR order, and seg_offsets[U] counts the valid occurrences only); d_e0 and the
    updated rows match within tolerance; rows nothing references stay bit-identical."""
    w = synth.Workload("badidx", T=T, rows=300, D=D, dtype=dtype, B=B, bag=("uniform", 1, 6),
                       dist=("zipf", 1.1), seed=T * 7 + D)
    b = synth.make_batch(w, with_dout=True)
    if long0:
        lengths = b.lengths.copy()
        lengths[:B] = np.random.default_rng(w.seed).integers(8, 13, B)
        set_lengths(b, lengths)
        assert b.lengths[:B].sum() > 2048
    assert sort_plan(w, len(b.indices))["table_sort"] is table_sort
    off = orc.lengths_to_offsets(b.lengths)
    idx = b.indices.copy()
    rng = np.random.default_rng(w.seed)
    bad = []
    for t in range(T):
        p = int(rng.integers(off[t * w.B], off[(t + 1) * w.B]))
        idx[p] = -1 - int(rng.integers(0, 5)) if t == 1 else 300 + int(rng.integers(0, 50))
        bad.append(p)
    bad = np.array(sorted(bad))
    keep = np.ones(len(idx), bool)
    keep[bad] = False
    # the valid sub-batch the oracle sees
    sub_len = np.array([int(keep[off[i]:off[i + 1]].sum()) for i in range(T * w.B)], dtype=np.int32)
    sub_off = orc.lengths_to_offsets(sub_len)
    sub_idx = idx[keep]
    fwd = orc.embbag_fwd(b.tables, dtype, w.B, sub_off, sub_idx, b.e0)
    r = orc.embbag_bwd_update(b.tables, dtype, w.B, sub_off, sub_idx, b.e0, fwd["pooled"], b.dout, 0.01)
    at = abs_tables(b.tables, dtype)
    pm = orc.embbag_pool(at, dtype, w.B, sub_off, sub_idx)
    rm = orc.embbag_bwd_update(at, dtype, w.B, sub_off, sub_idx, np.abs(b.e0), pm, np.abs(b.dout), 0.01)

    db = DeviceBatch(b)
    db.indices = torch.from_numpy(idx).cuda()
    db.status.zero_()
    pooled, _ = db.fwd(want_pooled=True)
    torch.cuda.synchronize()
    assert db.status.item() == ops.STATUS_BAD_INDEX
    d_out = torch.from_numpy(b.dout).cuda()
    before = [t.clone() for t in db.tables]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = ops.embbag_bwd_update(db.tables, db.offsets, db.indices, w.B, db.e0, pooled, d_out, 0.01, status=st)
    torch.cuda.synchronize()
    assert st.item() == ops.STATUS_BAD_INDEX
    nnz = len(idx)
    kept_pos = np.flatnonzero(keep)
    want_perm = np.concatenate([kept_pos[r["perm"]], bad]).astype(np.int32)
    np.testing.assert_array_equal(res["perm"].cpu().numpy()[:nnz], want_perm)
    U = int(res["num_unique"].item())
    assert U == len(r["unique_keys"])
    np.testing.assert_array_equal(res["unique_keys"].cpu().numpy()[:U], r["unique_keys"].astype(np.int32))
    np.testing.assert_array_equal(res["seg_offsets"].cpu().numpy()[:U + 1], r["seg_offsets"].astype(np.int32))
    assert int(res["seg_offsets"][U].item()) == nnz - len(bad)
    rtol = RTOL[dtype]
    assert_mag_close(res["d_e0"].cpu().numpy(), r["d_e0"], np.abs(b.dout[:, :D]) + rm["dZ"][:, 0], rtol, "d_e0")
    after = host_tables(db.tables, dtype)
    orig = host_tables(before, dtype)
    base = r["base"]
    keys = np.asarray(r["unique_keys"], dtype=np.int64)
    tix = np.searchsorted(base, keys, side="right") - 1
    rix = keys - base[tix]
    touched = [np.zeros(t.shape[0], bool) for t in orig]
    for t, i in zip(tix, rix):
        touched[t][i] = True
    for t in range(T):
        np.testing.assert_array_equal(after[t][~touched[t]], orig[t][~touched[t]])
    got_rows = np.array([orc.decode(after[t][i][None], dtype)[0] for t, i in zip(tix, rix)]).reshape(U, D)
    W_mag = np.abs(np.array([orc.decode(orig[t][i][None], dtype)[0] for t, i in zip(tix, rix)]).reshape(U, D))
    store_ulp = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[dtype]
    lim_mag = W_mag + 0.01 * rm["grad"] + (store_ulp / rtol) * np.abs(r["new_rows"])
    assert_mag_close(got_rows, r["new_rows"], lim_mag, rtol, "updated rows")
