"""Seeded synthetic inputs for the DLRM embedding-bag + interaction path.

This module only draws random inputs (table values, bag lengths, row indices,
bottom-MLP outputs e0, upstream gradients). It holds none of the method's
arithmetic: no pooling, no dot products, no offsets, no sorting. Both the HIP
path (through its tests and the benchmark) and the CPU oracle receive the same
arrays from here.

The workload shapes follow the problem statement of the DLRM pages: one
embedding table per categorical feature ("DLRM" note, section 2, The
Architecture), an ID list per feature and sample, and a bottom-MLP output e0 in
the embedding dimension (section 3, The Pairwise Interaction Layer). No public
dataset is used; every array is drawn from a seeded numpy PCG64 stream.

Readings taken where the pages are silent:
  * table rows are N(0, 0.01) with 0.01 the standard deviation, rounded to the
    storage dtype (round-to-nearest-even);
  * "Zipf(alpha)" over a table of n rows is the finite law P(rank k) ~ k^-alpha,
    k = 1..n, sampled by inverse CDF, and rank k is row k-1 (row 0 is hottest);
  * "log-uniform rows in [1e3, 1e6]" is round(exp(U(ln 1e3, ln 1e6)));
  * multi-hot bag lengths are min(Poisson(mean), cap) (zero allowed) or
    uniform on [lo, hi] inclusive.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16")
STORAGE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic batch.

    rows: either an int (every table has that many rows) or ("loguniform", lo, hi).
    bag:  ("fixed", L) | ("poisson", mean, cap) | ("uniform", lo, hi).
    dist: ("uniform",) | ("zipf", alpha).
    values: "normal" (N(0, sigma) rows, N(0,1) e0) or "int" (small integers, so
            every sum and dot is exact in fp32 whatever the order).
    """

    name: str
    T: int
    rows: object
    D: int
    dtype: str
    B: int
    bag: tuple
    dist: tuple
    seed: int
    sigma: float = 0.01
    values: str = "normal"

    @property
    def F(self) -> int:
        return self.T + 1

    @property
    def P(self) -> int:
        return self.F * (self.F - 1) // 2

    @property
    def out_width(self) -> int:
        return self.D + self.P

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny one, a 26-table Zipf one (single index per bag),
# a multi-hot fp16 one, the 164 GB capacity one (one GPU's shard of tables),
# and the backward on the 26-table shapes.
WORKLOADS: Dict[str, Workload] = {
    "tiny-4t1k-d16-b128": Workload(
        "tiny-4t1k-d16-b128", T=4, rows=1000, D=16, dtype="f32", B=128,
        bag=("fixed", 1), dist=("uniform",), seed=1),
    "zipf-26t-d128-b2048": Workload(
        "zipf-26t-d128-b2048", T=26, rows=("loguniform", 1e3, 1e6), D=128, dtype="f32",
        B=2048, bag=("fixed", 1), dist=("zipf", 1.05), seed=2),
    "multihot-8t4m-d64-fp16-b4096": Workload(
        "multihot-8t4m-d64-fp16-b4096", T=8, rows=4_000_000, D=64, dtype="f16", B=4096,
        bag=("poisson", 20, 100), dist=("zipf", 1.1), seed=3),
    "capacity-64t10m-d128-bf16-b16384": Workload(
        "capacity-64t10m-d128-bf16-b16384", T=64, rows=10_000_000, D=128, dtype="bf16",
        B=16384, bag=("uniform", 1, 32), dist=("uniform",), seed=4),
    "bwd-zipf-26t-d128-b2048": Workload(
        "bwd-zipf-26t-d128-b2048", T=26, rows=("loguniform", 1e3, 1e6), D=128, dtype="f32",
        B=2048, bag=("fixed", 1), dist=("zipf", 1.05), seed=5),
}

CAPACITY = "capacity-64t10m-d128-bf16-b16384"

# Named streams spawned from each workload's master seed.
_STREAMS = ("rows", "values", "lengths", "indices", "e0", "dout")


def _streams(seed: int) -> Dict[str, np.random.Generator]:
    ss = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(_STREAMS, ss)}


def stream_seed(seed: int, name: str) -> int:
    """A 63-bit integer seed derived from stream `name` (for torch device RNG)."""
    ss = np.random.SeedSequence(seed).spawn(len(_STREAMS))[_STREAMS.index(name)]
    return int(ss.generate_state(2, dtype=np.uint64)[0] >> np.uint64(1))


def table_rows(w: Workload) -> List[int]:
    if isinstance(w.rows, int):
        return [int(w.rows)] * w.T
    kind, lo, hi = w.rows
    assert kind == "loguniform"
    rng = _streams(w.seed)["rows"]
    u = rng.uniform(math.log(lo), math.log(hi), size=w.T)
    return [int(round(math.exp(x))) for x in u]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    raise ValueError(dtype)


def gen_tables_host(w: Workload, rows: Optional[Sequence[int]] = None) -> List[np.ndarray]:
    """Host tables in storage form: float32, float16, or uint16 bit patterns for bf16."""
    rows = table_rows(w) if rows is None else rows
    rng = _streams(w.seed)["values"]
    out = []
    for n in rows:
        if w.values == "int":
            v = rng.integers(-4, 5, size=(n, w.D)).astype(np.float32)
        else:
            v = (rng.standard_normal(size=(n, w.D), dtype=np.float32) * np.float32(w.sigma))
        out.append(_to_storage(v, w.dtype))
    return out


def quantize_rows_q4(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row-wise 4-bit codes of an fp32 table: per row, scale = (max - min) / 15 (1 for a
    constant row), bias = min, codes = round((x - min) / scale) clipped to [0, 15].
    Returns (uint8 codes 0..15 [rows, D], fp32 (scale, bias) [rows, 2])."""
    x = np.asarray(x, dtype=np.float32)
    lo = x.min(axis=1)
    hi = x.max(axis=1)
    scale = ((hi - lo) / np.float32(15)).astype(np.float32)
    scale[scale == 0] = 1.0
    codes = np.clip(np.rint((x - lo[:, None]) / scale[:, None]), 0, 15).astype(np.uint8)
    return codes, np.stack([scale, lo], axis=1).astype(np.float32)


def q4_row_stride(D: int) -> int:
    """Bytes from one stored row-wise 4-bit row to the next: D/2 code bytes and 8 bytes of
    scale and bias, rounded up to a power of two (= D for D = 128, 256, 512)."""
    s = 16
    while s < D // 2 + 8:
        s *= 2
    return s


def pack_q4_rows(codes: np.ndarray, scale_bias: np.ndarray) -> np.ndarray:
    """The stored form of a row-wise 4-bit table: per row, D/2 bytes of codes (column 2k in
    the low 4 bits of byte k, 2k + 1 in the high 4 bits), the fp32 scale and bias, zero
    padding to q4_row_stride(D) bytes (uint8 [rows, stride])."""
    n, D = codes.shape
    out = np.zeros((n, q4_row_stride(D)), dtype=np.uint8)
    c = codes.astype(np.uint8)
    out[:, :D // 2] = (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)
    out[:, D // 2:D // 2 + 8] = np.ascontiguousarray(scale_bias, dtype=np.float32).view(np.uint8).reshape(n, 8)
    return out


def gen_tables_q4_host(w: Workload, rows: Optional[Sequence[int]] = None):
    """Row-wise 4-bit tables: the fp32 N(0, sigma) rows (or, for values="int", small
    dyadic ones: codes 0..15, scale in {0.5, 1, 2}, bias in {-1, 0, 1}, every sum exact)
    quantized per row. Returns a list of (codes, scale_bias)."""
    rows = table_rows(w) if rows is None else rows
    rng = _streams(w.seed)["values"]
    out = []
    for n in rows:
        if w.values == "int":
            codes = rng.integers(0, 16, size=(n, w.D)).astype(np.uint8)
            sb = np.stack([rng.choice([0.5, 1.0, 2.0], size=n), rng.choice([-1.0, 0.0, 1.0], size=n)],
                          axis=1).astype(np.float32)
            out.append((codes, sb))
        else:
            v = rng.standard_normal(size=(n, w.D), dtype=np.float32) * np.float32(w.sigma)
            out.append(quantize_rows_q4(v))
    return out


def quantize_table_q8(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Table-wise 8-bit codes of an fp32 table: one scale = (max - min) / 255 (1 for a
    constant table) and bias = min for the whole table, codes = round((x - min) / scale)
    clipped to [0, 255]. Returns (uint8 codes [rows, D], fp32 (scale, bias) [2])."""
    x = np.asarray(x, dtype=np.float32)
    lo, hi = x.min(), x.max()
    scale = np.float32((hi - lo) / np.float32(255))
    if scale == 0:
        scale = np.float32(1)
    codes = np.clip(np.rint((x - lo) / scale), 0, 255).astype(np.uint8)
    return codes, np.array([scale, lo], dtype=np.float32)


def gen_tables_q8t_host(w: Workload, rows: Optional[Sequence[int]] = None):
    """Table-wise 8-bit tables: the fp32 N(0, sigma) tables (or, for values="int", codes
    0..4 with scale in {0.5, 1, 2} and bias in {-1, 0, 1}, every sum exact) quantized per
    table. Returns (list of codes, fp32 scale_bias [T, 2])."""
    rows = table_rows(w) if rows is None else rows
    rng = _streams(w.seed)["values"]
    codes, sb = [], []
    for n in rows:
        if w.values == "int":
            codes.append(rng.integers(0, 5, size=(n, w.D)).astype(np.uint8))
            sb.append([rng.choice([0.5, 1.0, 2.0]), rng.choice([-1.0, 0.0, 1.0])])
        else:
            v = rng.standard_normal(size=(n, w.D), dtype=np.float32) * np.float32(w.sigma)
            c, p = quantize_table_q8(v)
            codes.append(c)
            sb.append(p)
    return codes, np.asarray(sb, dtype=np.float32).reshape(len(rows), 2)


def gen_tables_device(w: Workload, device, rows: Optional[Sequence[int]] = None):
    """Device tables filled by torch's device RNG (for shards too large for host RAM).

    Returns a list of torch tensors of shape [rows_t, D] in the storage dtype
    (bf16/fp16/fp32). The values are N(0, sigma)-like; they are not the same
    numbers gen_tables_host would draw.
    """
    import torch

    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    rows = table_rows(w) if rows is None else rows
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(w.seed, "values"))
    out = []
    for n in rows:
        t = torch.empty((n, w.D), dtype=tdt, device=device)
        if w.values == "int":
            t.random_(-4, 5, generator=g)
        else:
            t.normal_(0.0, w.sigma, generator=g)
        out.append(t)
    return out


def gen_lengths(w: Workload) -> np.ndarray:
    """Bag lengths, table-major: entry t*B + b is the length of bag (t, b)."""
    rng = _streams(w.seed)["lengths"]
    n = w.T * w.B
    kind = w.bag[0]
    if kind == "fixed":
        L = np.full(n, w.bag[1], dtype=np.int64)
    elif kind == "poisson":
        L = np.minimum(rng.poisson(w.bag[1], size=n), w.bag[2])
    elif kind == "uniform":
        L = rng.integers(w.bag[1], w.bag[2] + 1, size=n)
    else:
        raise ValueError(kind)
    return L.astype(np.int32)


_ZIPF_CDF: Dict[Tuple[int, float], np.ndarray] = {}


def _zipf_cdf(n: int, alpha: float) -> np.ndarray:
    key = (n, alpha)
    if key not in _ZIPF_CDF:
        w = np.arange(1, n + 1, dtype=np.float64) ** (-alpha)
        c = np.cumsum(w)
        c /= c[-1]
        c[-1] = 1.0
        if len(_ZIPF_CDF) > 64:
            _ZIPF_CDF.clear()
        _ZIPF_CDF[key] = c
    return _ZIPF_CDF[key]


def sample_zipf(rng: np.random.Generator, n: int, alpha: float, size: int) -> np.ndarray:
    """Rows 0..n-1 with P(row r) ~ (r+1)^-alpha (inverse-CDF sampling)."""
    u = rng.random(size)
    return np.searchsorted(_zipf_cdf(n, alpha), u, side="right").astype(np.int64)


def gen_indices(w: Workload, rows: Sequence[int], lengths: np.ndarray) -> np.ndarray:
    """Row indices for every bag, laid out table-major then sample-major (CSR order)."""
    rng = _streams(w.seed)["indices"]
    per_table = lengths.reshape(w.T, w.B).sum(axis=1)
    parts = []
    for t in range(w.T):
        n = int(per_table[t])
        if w.dist[0] == "uniform":
            parts.append(rng.integers(0, rows[t], size=n))
        elif w.dist[0] == "zipf":
            parts.append(sample_zipf(rng, rows[t], w.dist[1], n))
        else:
            raise ValueError(w.dist)
    return np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)


def gen_e0(w: Workload) -> np.ndarray:
    rng = _streams(w.seed)["e0"]
    if w.values == "int":
        return rng.integers(-4, 5, size=(w.B, w.D)).astype(np.float32)
    return rng.standard_normal(size=(w.B, w.D), dtype=np.float32)


def gen_dout(w: Workload, width: Optional[int] = None) -> np.ndarray:
    """Upstream gradient of the interaction output [B, width]; width defaults to the plain
    layout's D + F(F-1)/2 (another layout passes its own output width)."""
    rng = _streams(w.seed)["dout"]
    W = w.out_width if width is None else int(width)
    if w.values == "int":
        return rng.integers(-2, 3, size=(w.B, W)).astype(np.float32)
    return rng.standard_normal(size=(w.B, W), dtype=np.float32)


@dataclasses.dataclass
class Batch:
    w: Workload
    rows: List[int]
    tables: Optional[List[np.ndarray]]
    lengths: np.ndarray
    indices: np.ndarray
    e0: np.ndarray
    dout: Optional[np.ndarray] = None


def make_batch(w: Workload, with_tables: bool = True, with_dout: bool = False) -> Batch:
    rows = table_rows(w)
    lengths = gen_lengths(w)
    indices = gen_indices(w, rows, lengths)
    tables = gen_tables_host(w, rows) if with_tables else None
    return Batch(w, rows, tables, lengths, indices, gen_e0(w), gen_dout(w) if with_dout else None)
