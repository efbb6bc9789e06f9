"""CPU oracle for the DLRM embedding-bag + pairwise-interaction hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module; only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library.

Everything is computed in float64 with plain numpy, straight from the
definitions, one bag / one pair / one occurrence at a time:

  * Embedding lookup and pooling -- "DLRM" note (vault-aram), section 2, The
    Architecture: one embedding table per categorical feature, each ID maps to
    one learned row. The pages say only that multi-valued features are
    "aggregated" (section 9, Weaknesses); the reading here is a sum over the
    bag, an empty bag giving the zero vector, a repeated ID counted as often as
    it appears.
  * Interaction -- same note, section 3, The Pairwise Interaction Layer: dot
    products e_i . e_j over the embeddings and the bottom-MLP output e_0, then
    concatenation with e_0. The variant without self-pairs (mentioned in that
    section) is the default: pairs i > j over Z = [e_0, e_1 .. e_T], in
    row-major order of the strict lower triangle (k = i(i-1)/2 + j), output
    [e_0 | dots]. The section's own formula (self-pairs i >= j) and the variant
    that concatenates the original embeddings alongside the dots are options.
  * Backward -- the pages give no backward; it is the exact gradient of the
    forward above: dZ_i = sum_{j != i} g_{ij} Z_j with g the upstream gradient
    of pair (i, j), the gradient of an embedding row is the sum of dZ over
    every occurrence of that row, and the update is plain SGD, W <- W - lr * G,
    on the touched rows only. (The "DLRM" note, section 5, Training, names
    adaptive optimizers; plain SGD is the reading taken for this path.)
  * Grouping of occurrences by row -- a stable sort of the occurrences by
    global row id (table base + row), then run boundaries of equal keys.

Validity of the bag description (CSR offsets, index range) is checked first;
invalid input raises BagError carrying the same status bits the GPU library
reports (1 = an index outside its table, 2 = offsets that are not a valid CSR).

Functions here are pinned by tests/test_oracle.py against hand-worked values
(tests/golden/), closed forms and brute-force reformulations.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

STATUS_BAD_INDEX = 1
STATUS_BAD_OFFSETS = 2


class BagError(ValueError):
    def __init__(self, bits: int, msg: str):
        super().__init__(msg)
        self.bits = bits


# ---------------------------------------------------------------------------
# Storage decoding (exact: every fp32/fp16/bf16 value is an fp64 value)
# ---------------------------------------------------------------------------
class Q8Table:
    """Affine 8-bit table: codes uint8 [rows, D] and fp32 (scale, bias) [rows, 2];
    row r stands for scale_r * codes[r] + bias_r. Indexing a row gives (codes, pair).
    The table-wise form (one pair for the whole table) is built by table_wise."""

    def __init__(self, codes: np.ndarray, scale_bias: np.ndarray):
        assert codes.dtype == np.uint8 and scale_bias.dtype == np.float32
        assert codes.ndim == 2 and scale_bias.shape == (codes.shape[0], 2)
        self.codes, self.scale_bias = codes, scale_bias
        self.shape = codes.shape

    def __getitem__(self, r):
        return self.codes[r], self.scale_bias[r]

    @classmethod
    def table_wise(cls, codes: np.ndarray, scale: float, bias: float) -> "Q8Table":
        """Table-wise 8-bit table: one (scale, bias) pair for every row, i.e. the
        row-wise form with that pair repeated."""
        pair = np.array([scale, bias], dtype=np.float32)
        return cls(codes, np.tile(pair, (codes.shape[0], 1)))


class Q4Table:
    """Row-wise 4-bit table in its stored form: uint8 [rows, S] with S >= D/2 + 8. Row r
    holds D/2 code bytes (column 2k in the low 4 bits of byte k, column 2k + 1 in the high
    4 bits), then the row's fp32 scale and fp32 bias (little-endian), then padding; it
    stands for scale_r * q + bias_r. Indexing a row gives (its bytes, D)."""

    def __init__(self, packed: np.ndarray, D: int):
        assert packed.dtype == np.uint8 and packed.ndim == 2 and packed.shape[1] >= D // 2 + 8 and D % 2 == 0
        self.packed, self.D = packed, D
        self.shape = (packed.shape[0], D)

    def __getitem__(self, r):
        return self.packed[r], self.D


def decode_q4_row(row: np.ndarray, D: int) -> np.ndarray:
    """One stored 4-bit row -> float64 [D], nibble by nibble."""
    q = np.zeros(D, dtype=np.float64)
    for k in range(D // 2):
        byte = int(row[k])
        q[2 * k] = byte & 0xF
        q[2 * k + 1] = byte >> 4
    scale = float(np.frombuffer(bytes(row[D // 2:D // 2 + 4]), dtype="<f4")[0])
    bias = float(np.frombuffer(bytes(row[D // 2 + 4:D // 2 + 8]), dtype="<f4")[0])
    return scale * q + bias


def decode(table, dtype: str) -> np.ndarray:
    """Stored table (or row) -> float64. bf16 tables arrive as uint16 bit patterns;
    "q8" rows arrive as (codes, (scale, bias)) from a Q8Table, "q4" rows as
    (stored bytes, D) from a Q4Table.

    "f64" (float64 tables) is accepted for the finite-difference pins only.
    """
    if dtype == "q4":
        row, D = table
        return decode_q4_row(row, D)
    if dtype == "q8":
        codes, sb = table
        sb = np.asarray(sb, dtype=np.float64)
        return sb[..., 0:1] * codes.astype(np.float64) + sb[..., 1:2] if codes.ndim > 1 else \
            sb[0] * codes.astype(np.float64) + sb[1]
    if dtype == "f64":
        assert table.dtype == np.float64
        return table.copy()
    if dtype == "f32":
        assert table.dtype == np.float32
        return table.astype(np.float64)
    if dtype == "f16":
        assert table.dtype == np.float16
        return table.astype(np.float64)
    if dtype == "bf16":
        assert table.dtype == np.uint16
        bits = table.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Bag description
# ---------------------------------------------------------------------------
def lengths_to_offsets(lengths: Sequence[int]) -> np.ndarray:
    """CSR offsets from bag lengths: offsets[0] = 0, offsets[i+1] = offsets[i] + len[i]."""
    n = len(lengths)
    off = np.zeros(n + 1, dtype=np.int64)
    for i in range(n):
        off[i + 1] = off[i] + int(lengths[i])
    return off


def bag_status(T: int, B: int, rows: Sequence[int], offsets: np.ndarray, indices: np.ndarray) -> int:
    """Status bits of a table-major CSR batch (bag (t,b) = indices[off[tB+b]:off[tB+b+1]])."""
    nnz = len(indices)
    bits = 0
    off = [int(x) for x in offsets]
    if len(off) != T * B + 1 or off[0] != 0 or off[-1] != nnz:
        bits |= STATUS_BAD_OFFSETS
    for i in range(len(off) - 1):
        if off[i] > off[i + 1] or off[i] < 0 or off[i + 1] > nnz:
            bits |= STATUS_BAD_OFFSETS
    if bits & STATUS_BAD_OFFSETS:
        # indices cannot be attributed to tables reliably; check them against
        # whichever bag covers them only when the offsets are valid.
        return bits
    for t in range(T):
        for b in range(B):
            for p in range(off[t * B + b], off[t * B + b + 1]):
                if not (0 <= int(indices[p]) < rows[t]):
                    bits |= STATUS_BAD_INDEX
    return bits


def check_bags(T, B, rows, offsets, indices) -> None:
    bits = bag_status(T, B, rows, offsets, indices)
    if bits:
        raise BagError(bits, f"invalid bag description (status bits {bits})")


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------
def embbag_pool(tables: List[np.ndarray], dtype: str, B: int, offsets: np.ndarray,
                indices: np.ndarray) -> np.ndarray:
    """pooled[b, t, :] = sum over the bag (t, b) of table_t[index, :], in float64."""
    T = len(tables)
    rows = [tb.shape[0] for tb in tables]
    check_bags(T, B, rows, offsets, indices)
    D = tables[0].shape[1]
    pooled = np.zeros((B, T, D), dtype=np.float64)
    for t in range(T):
        for b in range(B):
            s, e = int(offsets[t * B + b]), int(offsets[t * B + b + 1])
            acc = np.zeros(D, dtype=np.float64)
            for p in range(s, e):
                acc += decode(tables[t][int(indices[p])], dtype)
            pooled[b, t] = acc
    return pooled


def pair_count(F: int, self_pairs: bool = False) -> int:
    """Number of unordered pairs among F vectors, without (F(F-1)/2) or with
    (F(F+1)/2) the pairs of a vector with itself."""
    return F * (F + 1) // 2 if self_pairs else F * (F - 1) // 2


def pairs(F: int, self_pairs: bool = False):
    """(k, i, j) over the lower triangle, row-major. Strict (the default, i > j):
    (1,0),(2,0),(2,1),(3,0),... With self-pairs (i >= j, the form of the dot
    products in the "DLRM" note, section 3): (0,0),(1,0),(1,1),(2,0),..."""
    k = 0
    for i in range(F):
        for j in range(i + 1 if self_pairs else i):
            yield k, i, j
            k += 1


def stack_z(e0: np.ndarray, pooled: np.ndarray) -> np.ndarray:
    """Z[b] = [e0[b]; pooled[b, 0]; ...; pooled[b, T-1]] (F = T + 1 rows)."""
    B, T, D = pooled.shape
    Z = np.zeros((B, T + 1, D), dtype=np.float64)
    Z[:, 0] = e0
    Z[:, 1:] = pooled
    return Z


def interact(e0: np.ndarray, pooled: np.ndarray, self_pairs: bool = False,
             with_embeddings: bool = False) -> np.ndarray:
    """out[b] = [e0[b] | Z[b,i] . Z[b,j] for i > j (or i >= j with self_pairs)], float64.

    with_embeddings: the variant of the "DLRM" note, section 3, that concatenates the
    original embeddings alongside the interaction vector; the reading taken is
    out[b] = [Z[b,0] | Z[b,1] | ... | Z[b,T] | dots], every vector of Z in Z's order
    (e0 first, as in the plain layout), then the dots.
    """
    B, T, D = pooled.shape
    F = T + 1
    Z = stack_z(np.asarray(e0, dtype=np.float64), pooled)
    head = F * D if with_embeddings else D
    out = np.zeros((B, head + pair_count(F, self_pairs)), dtype=np.float64)
    if with_embeddings:
        for f in range(F):
            out[:, f * D:(f + 1) * D] = Z[:, f]
    else:
        out[:, :D] = e0
    for k, i, j in pairs(F, self_pairs):
        out[:, head + k] = (Z[:, i, :] * Z[:, j, :]).sum(axis=1)
    return out


def embbag_fwd(tables, dtype, B, offsets, indices, e0, self_pairs: bool = False,
               with_embeddings: bool = False) -> Dict[str, np.ndarray]:
    pooled = embbag_pool(tables, dtype, B, offsets, indices)
    return {"pooled": pooled, "out": interact(e0, pooled, self_pairs, with_embeddings)}


# ---------------------------------------------------------------------------
# Backward + update
# ---------------------------------------------------------------------------
def interact_bwd(e0: np.ndarray, pooled: np.ndarray, d_out: np.ndarray,
                 self_pairs: bool = False, with_embeddings: bool = False) -> Dict[str, np.ndarray]:
    """Gradient of the interaction output with respect to e0 and the pooled vectors.

    d(Z_i . Z_j)/dZ_i = Z_j and d(Z_i . Z_j)/dZ_j = Z_i, so every pair (i, j) with
    upstream gradient g adds g * Z_j to dZ_i and g * Z_i to dZ_j (a self-pair
    (i, i) thus adds 2 g Z_i); "dZ" holds this part. The vectors that appear in
    the output themselves also get their own upstream gradient: e0 always (the
    first D columns), and with with_embeddings every Z row. So
    d_e0 = d_out[:, :D] + dZ[:, 0], and d_pooled[:, t] = dZ[:, 1 + t] plus, with
    with_embeddings, the output gradient of pooled row t.
    """
    B, T, D = pooled.shape
    F = T + 1
    Z = stack_z(np.asarray(e0, dtype=np.float64), pooled)
    d_out = np.asarray(d_out, dtype=np.float64)
    head = F * D if with_embeddings else D
    dZ = np.zeros_like(Z)
    for k, i, j in pairs(F, self_pairs):
        g = d_out[:, head + k][:, None]
        dZ[:, i] += g * Z[:, j]
        dZ[:, j] += g * Z[:, i]
    d_e0 = d_out[:, :D] + dZ[:, 0]
    d_pooled = dZ[:, 1:].copy()
    if with_embeddings:
        for t in range(T):
            d_pooled[:, t] += d_out[:, (1 + t) * D:(2 + t) * D]
    return {"dZ": dZ, "d_e0": d_e0, "d_pooled": d_pooled}


def occurrence_keys(rows: Sequence[int], B: int, offsets: np.ndarray, indices: np.ndarray):
    """Per occurrence p (CSR order): global row key base_t + index, its table and sample."""
    T = len(rows)
    base = [0] * T
    for t in range(1, T):
        base[t] = base[t - 1] + int(rows[t - 1])
    nnz = len(indices)
    key = np.zeros(nnz, dtype=np.int64)
    tab = np.zeros(nnz, dtype=np.int64)
    smp = np.zeros(nnz, dtype=np.int64)
    for t in range(T):
        for b in range(B):
            for p in range(int(offsets[t * B + b]), int(offsets[t * B + b + 1])):
                key[p] = base[t] + int(indices[p])
                tab[p] = t
                smp[p] = b
    return key, tab, smp, base


def stable_order(keys: np.ndarray) -> np.ndarray:
    """Permutation sorting keys ascending; equal keys keep their original order."""
    return np.argsort(keys, kind="stable")


def segments(sorted_keys: np.ndarray):
    """Runs of equal keys in a sorted key array: (unique_keys, seg_offsets with a final nnz)."""
    n = len(sorted_keys)
    uniq, starts = [], []
    for i in range(n):
        if i == 0 or sorted_keys[i] != sorted_keys[i - 1]:
            uniq.append(int(sorted_keys[i]))
            starts.append(i)
    starts.append(n)
    return np.array(uniq, dtype=np.int64), np.array(starts, dtype=np.int64)


def embbag_bwd_update(tables: List[np.ndarray], dtype: str, B: int, offsets, indices, e0,
                      pooled, d_out, lr: float, optimizer: str = "sgd", state=None,
                      eps: float = 1e-8, self_pairs: bool = False,
                      with_embeddings: bool = False) -> Dict[str, object]:
    """Interaction backward, per-row gradient, update of the touched rows (all float64).

    optimizer "sgd": W <- W - lr * G. optimizer "rowwise_adagrad" (the "DLRM" note,
    section 5, Training, names AdaGrad; the reading taken is the row-wise form, one
    state value per row): s <- s + mean over the row of G^2, then
    W <- W - lr * G / (sqrt(s) + eps). state is a list of per-table arrays [rows_t]
    (None = zeros).

    Returns d_e0, dZ, perm (stable order of occurrences by key), unique_keys,
    seg_offsets, grad (one row per unique key), new_rows: the updated value
    (float64) of every touched row, keyed like unique_keys, and for AdaGrad
    new_state, keyed the same way. Untouched rows keep their stored value.
    """
    T = len(tables)
    rows = [tb.shape[0] for tb in tables]
    check_bags(T, B, rows, offsets, indices)
    D = tables[0].shape[1]
    bw = interact_bwd(e0, pooled, d_out, self_pairs, with_embeddings)
    dZ = bw["dZ"]
    d_pooled = bw["d_pooled"]  # the gradient of pooled[b, t]: dZ[b, 1 + t] (+ its own, with embeddings)
    key, tab, smp, base = occurrence_keys(rows, B, offsets, indices)
    perm = stable_order(key)
    uniq, seg = segments(key[perm])
    U = len(uniq)
    grad = np.zeros((U, D), dtype=np.float64)
    for u in range(U):
        for q in range(int(seg[u]), int(seg[u + 1])):
            p = int(perm[q])
            grad[u] += d_pooled[smp[p], tab[p]]
    new_rows = np.zeros((U, D), dtype=np.float64)
    new_state = np.zeros(U, dtype=np.float64)
    for u in range(U):
        t = int(tab[perm[int(seg[u])]])
        r = int(uniq[u]) - base[t]
        w = decode(tables[t][r], dtype)
        if optimizer == "sgd":
            new_rows[u] = w - lr * grad[u]
        elif optimizer == "rowwise_adagrad":
            s = (0.0 if state is None else float(state[t][r])) + float(np.mean(grad[u] * grad[u]))
            new_state[u] = s
            new_rows[u] = w - lr * grad[u] / (np.sqrt(s) + eps)
        else:
            raise ValueError(optimizer)
    out = {"d_e0": bw["d_e0"], "dZ": dZ, "perm": perm, "unique_keys": uniq, "seg_offsets": seg,
           "grad": grad, "new_rows": new_rows, "base": np.array(base, dtype=np.int64)}
    if optimizer == "rowwise_adagrad":
        out["new_state"] = new_state
    return out
