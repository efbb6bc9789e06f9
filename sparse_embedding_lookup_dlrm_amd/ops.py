"""Thin ctypes binding over libdlrm_embbag.so (C ABI: include/dlrm_embbag.h).

Only argument marshalling happens here: torch supplies device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels. The names mirror the C entry points. If the library is missing or
cannot be loaded, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdlrm_embbag.so")
INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, "dlrm_embbag.h"), os.path.join(INCLUDE, "dlrm_probe.h")]

DLRM_F32, DLRM_F16, DLRM_BF16 = 0, 1, 2
PAIRS_SELF, WITH_EMBEDDINGS = 1, 2  # interaction layout bits
STATUS_BAD_INDEX = 1
STATUS_BAD_OFFSETS = 2
MAX_TABLES = 128

_TORCH_DT = {torch.float32: DLRM_F32, torch.float16: DLRM_F16, torch.bfloat16: DLRM_BF16}

_c_void_p = ctypes.c_void_p
_i32, _i64, _f32, _size_t = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_P = ctypes.POINTER

_SIGNATURES = {
    "dlrm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dlrm_version": (ctypes.c_int, []),
    "dlrm_lengths_to_offsets": (ctypes.c_int, [_i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "dlrm_embbag_fwd": (ctypes.c_int, [_i32, _i32, _i32, _i32, _P(_c_void_p), _P(_i64), _c_void_p, _c_void_p, _i64,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "dlrm_embbag_fwd_ex": (ctypes.c_int, [_i32, _i32, _i32, _i32, _P(_c_void_p), _P(_i64), _c_void_p, _c_void_p,
                                          _i64, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p]),
    "dlrm_embbag_fwd_q4": (ctypes.c_int, [_i32, _i32, _i32, _P(_c_void_p), _P(_i64), _c_void_p, _c_void_p, _i64,
                                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "dlrm_embbag_fwd_q8t": (ctypes.c_int, [_i32, _i32, _i32, _P(_c_void_p), _P(_f32), _P(_i64), _c_void_p,
                                           _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                           _c_void_p]),
    "dlrm_interact": (ctypes.c_int, [_i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "dlrm_interact_ex": (ctypes.c_int, [_i32, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "dlrm_interact_bwd": (ctypes.c_int, [_i32, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _c_void_p]),
    "dlrm_embbag_bwd_workspace_bytes": (ctypes.c_int, [_i32, _i32, _i32, _i64, _P(_i64), _P(_size_t)]),
    "dlrm_embbag_bwd_update": (ctypes.c_int, [_i32, _i32, _i32, _i32, _P(_c_void_p), _P(_i64), _c_void_p, _c_void_p,
                                              _i64, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p, _c_void_p,
                                              _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t, _c_void_p,
                                              _c_void_p]),
    "dlrm_embbag_bwd_update_adagrad": (ctypes.c_int, [_i32, _i32, _i32, _i32, _P(_c_void_p), _P(_i64), _c_void_p,
                                                      _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _f32, _f32,
                                                      _P(_c_void_p), _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                      _c_void_p, _c_void_p, _size_t, _c_void_p, _c_void_p]),
    "dlrm_validate_bags": (ctypes.c_int, [_i32, _i32, _P(_i64), _P(_i32), _P(_i32), _i64]),
    "dlrm_embbag_bwd_update_ex": (ctypes.c_int, [_i32, _i32, _i32, _i32, _P(_c_void_p), _P(_i64), _c_void_p,
                                                 _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _i32, _f32, _f32,
                                                 _P(_c_void_p), _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                 _c_void_p, _c_void_p, _size_t, _c_void_p, _c_void_p]),
    "dlrm_embbag_bwd_plan": (ctypes.c_int, [_i32, _i32, _i32, _i64, _P(_i64), _i32, _P(_i32)]),
    "dlrm_probe_row_gather": (ctypes.c_int, [_i32, _i32, _i32, _P(_c_void_p), _P(_i64), _P(_i64), _c_void_p, _i64,
                                             _c_void_p, _c_void_p]),
    "dlrm_embbag_bwd_update_noalloc": (ctypes.c_int, [_i32, _i32, _i32, _i32, _P(_c_void_p), _P(_i64), _c_void_p,
                                                      _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _f32,
                                                      _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                      _c_void_p, _c_void_p]),
}

_lib: Optional[ctypes.CDLL] = None


class DlrmError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {status_string(code)} ({code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libdlrm_embbag.so (built in-tree). Raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_embedding_lookup_dlrm_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def header_functions() -> List[str]:
    """Names of the functions declared in the library's headers (include/*.h)."""
    names = set()
    for h in HEADERS:
        with open(h) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(dlrm_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def status_string(code: int) -> str:
    return lib().dlrm_status_string(code).decode()


def version() -> int:
    return lib().dlrm_version()


def _check(code: int, where: str) -> None:
    if code != 0:
        raise DlrmError(code, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _require_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("device tensors must be contiguous CUDA (HIP) tensors")


def _expect(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, numel: int, at_least: bool = False) -> None:
    """Size and dtype of a tensor handed to the C ABI, which takes raw pointers and cannot
    see an undersized buffer: checked here, before any call."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    n = t.numel()
    if (n < numel) if at_least else (n != numel):
        raise ValueError(f"{name} has {n} elements, needs {'at least ' if at_least else ''}{numel}")


def _check_bags(offsets: torch.Tensor, indices: torch.Tensor, T: int, B: int) -> None:
    _expect(offsets, "offsets", torch.int32, T * B + 1)
    if indices.dtype != torch.int32:
        raise ValueError(f"indices must be torch.int32, got {indices.dtype}")


def _table_args(tables: Sequence[torch.Tensor]):
    T = len(tables)
    if T < 1:
        raise ValueError("need at least one table")
    dt = tables[0].dtype
    if dt not in _TORCH_DT:
        raise ValueError(f"unsupported table dtype {dt}")
    D = tables[0].shape[1]
    for t in tables:
        if t.dtype != dt or t.dim() != 2 or t.shape[1] != D:
            raise ValueError("all tables must be 2-D with the same dtype and width")
    ptrs = (_c_void_p * T)(*[t.data_ptr() for t in tables])
    rows = (_i64 * T)(*[t.shape[0] for t in tables])
    return T, D, _TORCH_DT[dt], ptrs, rows


def pair_count(T: int, self_pairs: bool = False) -> int:
    F = T + 1
    return F * (F + 1) // 2 if self_pairs else F * (F - 1) // 2


def layout_bits(self_pairs: bool = False, with_embeddings: bool = False) -> int:
    return (PAIRS_SELF if self_pairs else 0) | (WITH_EMBEDDINGS if with_embeddings else 0)


def out_width(T: int, D: int, layout: int = 0) -> int:
    """Floats per sample of the interaction output in a layout."""
    return (T + 1) * D * bool(layout & WITH_EMBEDDINGS) + D * (not layout & WITH_EMBEDDINGS) + \
        pair_count(T, bool(layout & PAIRS_SELF))


def lengths_to_offsets(lengths: torch.Tensor, offsets: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int32 bag lengths (device) -> int32 CSR offsets (device, n + 1 entries)."""
    _expect(lengths, "lengths", torch.int32, lengths.numel())
    n = lengths.numel()
    _expect(offsets, "offsets", torch.int32, n + 1)
    _expect(status, "status", torch.int32, 1, at_least=True)
    _require_cuda(lengths, offsets, status)
    if offsets is None:
        offsets = torch.empty(n + 1, dtype=torch.int32, device=lengths.device)
    _check(lib().dlrm_lengths_to_offsets(n, _ptr(lengths), _ptr(offsets), _ptr(status), _stream(stream)),
           "dlrm_lengths_to_offsets")
    return offsets


def _check_fwd_buffers(T, B, D, offsets, indices, e0, out_pooled, out_inter, status, layout=0):
    _check_bags(offsets, indices, T, B)
    _expect(e0, "e0", torch.float32, B * D)
    _expect(out_pooled, "out_pooled", torch.float32, B * T * D)
    _expect(out_inter, "out_inter", torch.float32, B * out_width(T, D, layout))
    _expect(status, "status", torch.int32, 1, at_least=True)


def embbag_fwd(tables: Sequence[torch.Tensor], offsets: torch.Tensor, indices: torch.Tensor, B: int,
               e0: Optional[torch.Tensor] = None, *, want_pooled: bool = False, want_inter: bool = True,
               out_pooled: Optional[torch.Tensor] = None, out_inter: Optional[torch.Tensor] = None,
               status: Optional[torch.Tensor] = None, stream=None,
               layout: int = 0) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Embedding-bag forward; returns (pooled [B,T,D] or None, interaction output [B, W] or None):
    [e0 | dots] with layout 0 (dlrm_embbag_fwd), else the layout bits PAIRS_SELF and
    WITH_EMBEDDINGS (dlrm_embbag_fwd_ex)."""
    T, D, dt, ptrs, rows = _table_args(tables)
    _check_fwd_buffers(T, B, D, offsets, indices, e0, out_pooled, out_inter, status, layout)
    _require_cuda(*tables, offsets, indices, e0, out_pooled, out_inter, status)
    dev = tables[0].device
    if want_pooled and out_pooled is None:
        out_pooled = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    if want_inter and out_inter is None:
        out_inter = torch.empty((B, out_width(T, D, layout)), dtype=torch.float32, device=dev)
    if layout == 0:
        _check(lib().dlrm_embbag_fwd(T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), indices.numel(),
                                     _ptr(e0), _ptr(out_pooled), _ptr(out_inter), _ptr(status), _stream(stream)),
               "dlrm_embbag_fwd")
    else:
        _check(lib().dlrm_embbag_fwd_ex(T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), indices.numel(),
                                        _ptr(e0), _ptr(out_pooled), _ptr(out_inter), layout, _ptr(status),
                                        _stream(stream)),
               "dlrm_embbag_fwd_ex")
    return out_pooled, out_inter


def embbag_fwd_q4(tables: Sequence[torch.Tensor], offsets: torch.Tensor, indices: torch.Tensor, B: int,
                  e0: torch.Tensor, *, want_pooled: bool = False, out_pooled: Optional[torch.Tensor] = None,
                  out_inter: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """Fused forward on row-wise 4-bit tables: uint8 [rows, D] per table (D = 128, 256 or 512;
    a row is D/2 code bytes, its fp32 scale and bias, then padding: synth.pack_q4_rows builds
    them); returns (pooled or None, [e0 | dots])."""
    T = len(tables)
    if T < 1:
        raise ValueError("need at least one table")
    D = tables[0].shape[1]
    for t in tables:
        if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[1] != D or not t.is_contiguous():
            raise ValueError("4-bit tables must be contiguous uint8 [rows, D] with the same D")
    _check_fwd_buffers(T, B, D, offsets, indices, e0, out_pooled, out_inter, status)
    _require_cuda(*tables, offsets, indices, e0, out_pooled, out_inter, status)
    ptrs = (_c_void_p * T)(*[t.data_ptr() for t in tables])
    rows = (_i64 * T)(*[t.shape[0] for t in tables])
    dev = tables[0].device
    if want_pooled and out_pooled is None:
        out_pooled = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    if out_inter is None:
        out_inter = torch.empty((B, D + pair_count(T)), dtype=torch.float32, device=dev)
    _check(lib().dlrm_embbag_fwd_q4(T, B, D, ptrs, rows, _ptr(offsets), _ptr(indices), indices.numel(), _ptr(e0),
                                    _ptr(out_pooled), _ptr(out_inter), _ptr(status), _stream(stream)),
           "dlrm_embbag_fwd_q4")
    return out_pooled, out_inter


def embbag_fwd_q8t(tables: Sequence[torch.Tensor], scale_bias, offsets: torch.Tensor, indices: torch.Tensor,
                   B: int, e0: torch.Tensor, *, want_pooled: bool = False,
                   out_pooled: Optional[torch.Tensor] = None, out_inter: Optional[torch.Tensor] = None,
                   status: Optional[torch.Tensor] = None, stream=None) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """Fused forward on table-wise 8-bit tables: uint8 [rows, D] codes per table and one
    (scale, bias) pair per table (host sequence of T pairs); returns (pooled or None, [e0 | dots])."""
    T = len(tables)
    if T < 1:
        raise ValueError("need at least one table")
    D = tables[0].shape[1]
    for t in tables:
        if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[1] != D or not t.is_contiguous():
            raise ValueError("8-bit tables must be contiguous uint8 [rows, D] with the same D")
    sb = [float(v) for pair in scale_bias for v in pair]
    if len(sb) != 2 * T:
        raise ValueError("need one (scale, bias) pair per table")
    _check_fwd_buffers(T, B, D, offsets, indices, e0, out_pooled, out_inter, status)
    _require_cuda(*tables, offsets, indices, e0, out_pooled, out_inter, status)
    ptrs = (_c_void_p * T)(*[t.data_ptr() for t in tables])
    rows = (_i64 * T)(*[t.shape[0] for t in tables])
    dev = tables[0].device
    if want_pooled and out_pooled is None:
        out_pooled = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    if out_inter is None:
        out_inter = torch.empty((B, D + pair_count(T)), dtype=torch.float32, device=dev)
    _check(lib().dlrm_embbag_fwd_q8t(T, B, D, ptrs, (_f32 * (2 * T))(*sb), rows, _ptr(offsets), _ptr(indices),
                                     indices.numel(), _ptr(e0), _ptr(out_pooled), _ptr(out_inter), _ptr(status),
                                     _stream(stream)),
           "dlrm_embbag_fwd_q8t")
    return out_pooled, out_inter


def interact(e0: torch.Tensor, pooled: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None,
             self_pairs: bool = False, with_embeddings: bool = False) -> torch.Tensor:
    """[e0 | lower-triangle dots of Z = [e0; pooled]] from pooled [B, T, D] fp32: pairs i > j
    (dlrm_interact); i >= j with self_pairs, and [Z rows | dots] with with_embeddings
    (dlrm_interact_ex)."""
    B, T, D = pooled.shape
    layout = layout_bits(self_pairs, with_embeddings)
    W = out_width(T, D, layout)
    _expect(pooled, "pooled", torch.float32, B * T * D)
    _expect(e0, "e0", torch.float32, B * D)
    _expect(out, "out", torch.float32, B * W)
    _require_cuda(e0, pooled, out)
    if out is None:
        out = torch.empty((B, W), dtype=torch.float32, device=pooled.device)
    if layout:
        _check(lib().dlrm_interact_ex(T, B, D, layout, _ptr(e0), _ptr(pooled), _ptr(out), _stream(stream)),
               "dlrm_interact_ex")
    else:
        _check(lib().dlrm_interact(T, B, D, _ptr(e0), _ptr(pooled), _ptr(out), _stream(stream)), "dlrm_interact")
    return out


def interact_bwd(e0: torch.Tensor, pooled: torch.Tensor, d_out: torch.Tensor, self_pairs: bool = False,
                 d_e0: Optional[torch.Tensor] = None, d_pooled: Optional[torch.Tensor] = None,
                 want_d_e0: bool = True, stream=None,
                 with_embeddings: bool = False) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """(dL/de0, dL/dpooled) of the interaction from dL/dout (dlrm_interact_bwd)."""
    B, T, D = pooled.shape
    layout = layout_bits(self_pairs, with_embeddings)
    _expect(pooled, "pooled", torch.float32, B * T * D)
    _expect(e0, "e0", torch.float32, B * D)
    _expect(d_out, "d_out", torch.float32, B * out_width(T, D, layout))
    _expect(d_e0, "d_e0", torch.float32, B * D)
    _expect(d_pooled, "d_pooled", torch.float32, B * T * D)
    _require_cuda(e0, pooled, d_out, d_e0, d_pooled)
    if d_pooled is None:
        d_pooled = torch.empty((B, T, D), dtype=torch.float32, device=pooled.device)
    if d_e0 is None and want_d_e0:
        d_e0 = torch.empty((B, D), dtype=torch.float32, device=pooled.device)
    _check(lib().dlrm_interact_bwd(T, B, D, layout, _ptr(e0), _ptr(pooled), _ptr(d_out), _ptr(d_e0),
                                   _ptr(d_pooled), _stream(stream)), "dlrm_interact_bwd")
    return d_e0, d_pooled


def bwd_workspace_bytes(T: int, B: int, D: int, nnz: int, rows: Sequence[int]) -> int:
    r = (_i64 * T)(*rows)
    out = _size_t(0)
    _check(lib().dlrm_embbag_bwd_workspace_bytes(T, B, D, nnz, r, ctypes.byref(out)),
           "dlrm_embbag_bwd_workspace_bytes")
    return out.value


def _check_bwd_buffers(T, B, D, offsets, indices, e0, pooled, d_out, d_e0, status, layout=0):
    _check_bags(offsets, indices, T, B)
    _expect(e0, "e0", torch.float32, B * D)
    _expect(pooled, "pooled", torch.float32, B * T * D)
    _expect(d_out, "d_out", torch.float32, B * out_width(T, D, layout))
    _expect(d_e0, "d_e0", torch.float32, B * D)
    _expect(status, "status", torch.int32, 1, at_least=True)


def bwd_plan(T: int, B: int, D: int, nnz: int, rows: Sequence[int], want_segments: bool = True) -> dict:
    """How the sparse backward will run for these sizes (dlrm_embbag_bwd_plan; host only)."""
    plan = (_i32 * 5)()
    _check(lib().dlrm_embbag_bwd_plan(T, B, D, nnz, (_i64 * T)(*rows), 1 if want_segments else 0, plan),
           "dlrm_embbag_bwd_plan")
    return {"radix_bits": plan[0], "passes": plan[1], "interact_bwd_shared": bool(plan[2]), "max_lds": plan[3],
            "table_sort": bool(plan[4])}


def embbag_bwd_update(tables: Sequence[torch.Tensor], offsets: torch.Tensor, indices: torch.Tensor, B: int,
                      e0: torch.Tensor, pooled: torch.Tensor, d_out: torch.Tensor, lr: float, *,
                      want_d_e0: bool = True, want_segments: bool = True, workspace: Optional[torch.Tensor] = None,
                      status: Optional[torch.Tensor] = None, stream=None,
                      row_state: Optional[Sequence[torch.Tensor]] = None, eps: float = 1e-8,
                      layout: int = 0) -> dict:
    """Sparse backward + update of the touched rows (tables are updated in place): SGD, or
    row-wise AdaGrad when row_state (one fp32 [rows_t] tensor per table, updated in
    place) is given (dlrm_embbag_bwd_update_adagrad); d_out in the interaction layout
    `layout` (dlrm_embbag_bwd_update_ex when it is not 0)."""
    T, D, dt, ptrs, rows = _table_args(tables)
    _check_bwd_buffers(T, B, D, offsets, indices, e0, pooled, d_out, None, status, layout)
    if row_state is not None:
        if len(row_state) != T:
            raise ValueError("row_state needs one tensor per table")
        for st_, t in zip(row_state, tables):
            _require_cuda(st_)
            if st_.dtype != torch.float32 or st_.numel() != t.shape[0] or not st_.is_contiguous():
                raise ValueError("row_state[t] must be a contiguous fp32 tensor with one value per row")
    nnz = indices.numel()
    dev = tables[0].device
    need = bwd_workspace_bytes(T, B, D, nnz, [t.shape[0] for t in tables])
    _expect(workspace, "workspace", torch.uint8, need, at_least=True)
    _require_cuda(*tables, offsets, indices, e0, pooled, d_out, workspace, status)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    res = {"d_e0": torch.empty((B, D), dtype=torch.float32, device=dev) if want_d_e0 else None}
    if want_segments:
        res["unique_keys"] = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        res["seg_offsets"] = torch.empty(nnz + 1, dtype=torch.int32, device=dev)
        res["num_unique"] = torch.empty(1, dtype=torch.int32, device=dev)
        res["perm"] = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    g = res.get
    if layout != 0:
        sptr = (_c_void_p * T)(*[s_.data_ptr() for s_ in row_state]) if row_state is not None else None
        _check(lib().dlrm_embbag_bwd_update_ex(T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), nnz, _ptr(e0),
                                               _ptr(pooled), _ptr(d_out), int(layout), float(lr), float(eps), sptr,
                                               _ptr(g("d_e0")), _ptr(g("unique_keys")), _ptr(g("seg_offsets")),
                                               _ptr(g("num_unique")), _ptr(g("perm")), _ptr(workspace),
                                               workspace.numel(), _ptr(status), _stream(stream)),
               "dlrm_embbag_bwd_update_ex")
    elif row_state is None:
        _check(lib().dlrm_embbag_bwd_update(T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), nnz, _ptr(e0),
                                            _ptr(pooled), _ptr(d_out), float(lr), _ptr(g("d_e0")),
                                            _ptr(g("unique_keys")), _ptr(g("seg_offsets")), _ptr(g("num_unique")),
                                            _ptr(g("perm")), _ptr(workspace), workspace.numel(), _ptr(status),
                                            _stream(stream)),
               "dlrm_embbag_bwd_update")
    else:
        sptr = (_c_void_p * T)(*[s_.data_ptr() for s_ in row_state])
        _check(lib().dlrm_embbag_bwd_update_adagrad(T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), nnz,
                                                    _ptr(e0), _ptr(pooled), _ptr(d_out), float(lr), float(eps), sptr,
                                                    _ptr(g("d_e0")), _ptr(g("unique_keys")), _ptr(g("seg_offsets")),
                                                    _ptr(g("num_unique")), _ptr(g("perm")), _ptr(workspace),
                                                    workspace.numel(), _ptr(status), _stream(stream)),
               "dlrm_embbag_bwd_update_adagrad")
    return res


PROBE_SINK_FLOATS = 4096 * 256


class ProbeGatherPlan:
    """dlrm_probe_row_gather (measurement kernel: the bare random-row gather of a batch)
    with its arguments marshalled once. table_start: host CSR position of each table's
    first occurrence, T + 1 entries."""

    def __init__(self, tables, table_start: Sequence[int], indices: torch.Tensor, sink: torch.Tensor, stream=None):
        T, D, dt, ptrs, rows = _table_args(tables)
        if len(table_start) != T + 1:
            raise ValueError("table_start needs T + 1 entries")
        _expect(sink, "sink", torch.float32, PROBE_SINK_FLOATS, at_least=True)
        _require_cuda(*tables, indices, sink)
        starts = (_i64 * (T + 1))(*[int(x) for x in table_start])
        self._keep = (tables, indices, sink, ptrs, rows, starts)
        self._args = (T, D, dt, ptrs, rows, starts, _ptr(indices), indices.numel(), _ptr(sink), _stream(stream))
        self._fn = lib().dlrm_probe_row_gather

    def run(self):
        _check(self._fn(*self._args), "dlrm_probe_row_gather")


NOALLOC_SCRATCH_BYTES = 64 << 20


def embbag_bwd_update_noalloc(tables: Sequence[torch.Tensor], offsets: torch.Tensor, indices: torch.Tensor, B: int,
                              e0: torch.Tensor, pooled: torch.Tensor, d_out: torch.Tensor, lr: float, *,
                              d_e0: Optional[torch.Tensor] = None, unique_keys: Optional[torch.Tensor] = None,
                              seg_offsets: Optional[torch.Tensor] = None, num_unique: Optional[torch.Tensor] = None,
                              perm: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                              stream=None) -> None:
    """dlrm_embbag_bwd_update_noalloc: the SGD backward with the library's own static scratch
    (no workspace). Every output is a caller tensor (or None); this call allocates nothing."""
    T, D, dt, ptrs, rows = _table_args(tables)
    nnz = indices.numel()
    _check_bwd_buffers(T, B, D, offsets, indices, e0, pooled, d_out, d_e0, status)
    _expect(unique_keys, "unique_keys", torch.int32, nnz, at_least=True)
    _expect(seg_offsets, "seg_offsets", torch.int32, nnz + 1, at_least=True)
    _expect(num_unique, "num_unique", torch.int32, 1, at_least=True)
    _expect(perm, "perm", torch.int32, nnz, at_least=True)
    _require_cuda(*tables, offsets, indices, e0, pooled, d_out, d_e0, unique_keys, seg_offsets, num_unique, perm,
                  status)
    _check(lib().dlrm_embbag_bwd_update_noalloc(T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), nnz, _ptr(e0),
                                                _ptr(pooled), _ptr(d_out), float(lr), _ptr(d_e0), _ptr(unique_keys),
                                                _ptr(seg_offsets), _ptr(num_unique), _ptr(perm), _ptr(status),
                                                _stream(stream)),
           "dlrm_embbag_bwd_update_noalloc")


def validate_bags(T: int, B: int, rows: Sequence[int], offsets, indices) -> int:
    """Host check of a bag description (numpy/int sequences); returns the status bits."""
    import numpy as np

    off = np.ascontiguousarray(offsets, dtype=np.int32)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    r = (_i64 * T)(*rows)
    return lib().dlrm_validate_bags(T, B, r, off.ctypes.data_as(_P(_i32)), idx.ctypes.data_as(_P(_i32)), len(idx))


class FwdPlan:
    """dlrm_embbag_fwd with its arguments marshalled once, for repeated calls on
    resident inputs (same tensors every call)."""

    def __init__(self, tables, offsets, indices, B, e0=None, *, out_pooled=None, out_inter=None, status=None,
                 stream=None, layout: int = 0):
        T, D, dt, ptrs, rows = _table_args(tables)
        _check_fwd_buffers(T, B, D, offsets, indices, e0, out_pooled, out_inter, status, layout)
        _require_cuda(*tables, offsets, indices, e0, out_pooled, out_inter, status)
        self._keep = (tables, offsets, indices, e0, out_pooled, out_inter, status, ptrs, rows)
        if layout == 0:
            self._args = (T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), indices.numel(), _ptr(e0),
                          _ptr(out_pooled), _ptr(out_inter), _ptr(status), _stream(stream))
            self._name = "dlrm_embbag_fwd"
        else:
            self._args = (T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), indices.numel(), _ptr(e0),
                          _ptr(out_pooled), _ptr(out_inter), layout, _ptr(status), _stream(stream))
            self._name = "dlrm_embbag_fwd_ex"
        self._fn = getattr(lib(), self._name)

    def run(self):
        _check(self._fn(*self._args), self._name)


class BwdPlan:
    """dlrm_embbag_bwd_update (or, with row_state, dlrm_embbag_bwd_update_adagrad) with its
    arguments marshalled once (tables, and the row states, updated in place each run)."""

    def __init__(self, tables, offsets, indices, B, e0, pooled, d_out, lr, *, d_e0=None, workspace=None,
                 status=None, stream=None, row_state=None, eps: float = 1e-8):
        T, D, dt, ptrs, rows = _table_args(tables)
        nnz = indices.numel()
        dev = tables[0].device
        self.unique_keys = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        self.seg_offsets = torch.empty(nnz + 1, dtype=torch.int32, device=dev)
        self.num_unique = torch.empty(1, dtype=torch.int32, device=dev)
        self.perm = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
        need = bwd_workspace_bytes(T, B, D, nnz, [t.shape[0] for t in tables])
        _expect(workspace, "workspace", torch.uint8, need, at_least=True)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _check_bwd_buffers(T, B, D, offsets, indices, e0, pooled, d_out, d_e0, status)
        _require_cuda(*tables, offsets, indices, e0, pooled, d_out, d_e0, workspace, status)
        opt = ()
        sptr = None
        self._name = "dlrm_embbag_bwd_update"
        if row_state is not None:
            if len(row_state) != T:
                raise ValueError("row_state needs one tensor per table")
            for st_, t in zip(row_state, tables):
                _require_cuda(st_)
                if st_.dtype != torch.float32 or st_.numel() != t.shape[0] or not st_.is_contiguous():
                    raise ValueError("row_state[t] must be a contiguous fp32 tensor with one value per row")
            sptr = (_c_void_p * T)(*[s_.data_ptr() for s_ in row_state])
            opt = (float(eps), sptr)
            self._name = "dlrm_embbag_bwd_update_adagrad"
        self._keep = (tables, offsets, indices, e0, pooled, d_out, d_e0, workspace, status, ptrs, rows, row_state,
                      sptr)
        self._args = (T, B, D, dt, ptrs, rows, _ptr(offsets), _ptr(indices), nnz, _ptr(e0), _ptr(pooled),
                      _ptr(d_out), float(lr), *opt, _ptr(d_e0), _ptr(self.unique_keys), _ptr(self.seg_offsets),
                      _ptr(self.num_unique), _ptr(self.perm), _ptr(workspace), workspace.numel(), _ptr(status),
                      _stream(stream))
        self._fn = getattr(lib(), self._name)

    def run(self):
        _check(self._fn(*self._args), self._name)
