"""Pins for the CPU oracle, independent of the oracle's own code.

Each pin checks the oracle against something it does not compute itself:
hand-worked values (tests/golden), a textbook reformulation (bag-count matrix
times table; Z Z^T and its strict lower triangle), a closed form (the
factorization-machine identity, F(F-1)/2 pair count, finite differences of a
quadratic loss), brute force on tiny inputs, and invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import dlrm_oracle as orc


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_example_t2_d2.json")) as f:
        return json.load(f)


def _tables_f32(g):
    return [np.array(t, dtype=np.float32) for t in g["tables"]]


# ---------------------------------------------------------------------------
# Hand-worked example
# ---------------------------------------------------------------------------
def test_golden_forward(golden_dir):
    g = _golden(golden_dir)
    off = orc.lengths_to_offsets(g["lengths_table_major"])
    assert off.tolist() == g["offsets"]
    idx = np.array(g["indices"], dtype=np.int32)
    r = orc.embbag_fwd(_tables_f32(g), "f32", g["B"], off, idx, np.array(g["e0"], np.float32))
    np.testing.assert_array_equal(r["pooled"], np.array(g["pooled"], dtype=np.float64))
    np.testing.assert_array_equal(r["out"], np.array(g["out"], dtype=np.float64))


def test_golden_pair_order(golden_dir):
    with open(os.path.join(golden_dir, "worked_example_pair_order_t3.json")) as f:
        g = json.load(f)
    tabs = [np.array(t, dtype=np.float32) for t in g["tables"]]
    r = orc.embbag_fwd(tabs, "f32", g["B"], np.array(g["offsets"]), np.array(g["indices"], np.int32),
                       np.array(g["e0"], np.float32))
    np.testing.assert_array_equal(r["out"], np.array(g["out"], dtype=np.float64))


def test_golden_backward(golden_dir):
    g = _golden(golden_dir)
    off = np.array(g["offsets"])
    idx = np.array(g["indices"], dtype=np.int32)
    tabs = _tables_f32(g)
    e0 = np.array(g["e0"], np.float32)
    pooled = np.array(g["pooled"], dtype=np.float64)
    r = orc.embbag_bwd_update(tabs, "f32", g["B"], off, idx, e0, pooled,
                              np.array(g["d_out"], np.float32), g["lr"])
    np.testing.assert_array_equal(r["dZ"], np.array(g["dZ"], dtype=np.float64))
    np.testing.assert_array_equal(r["d_e0"], np.array(g["d_e0"], dtype=np.float64))
    key, _, _, _ = orc.occurrence_keys([t.shape[0] for t in tabs], g["B"], off, idx)
    assert key.tolist() == g["keys"]
    assert r["perm"].tolist() == g["perm"]
    assert r["unique_keys"].tolist() == g["unique_keys"]
    assert r["seg_offsets"].tolist() == g["seg_offsets"]
    np.testing.assert_array_equal(r["grad"], np.array(g["grad"], dtype=np.float64))
    np.testing.assert_array_equal(r["new_rows"], np.array(g["new_rows"], dtype=np.float64))


# ---------------------------------------------------------------------------
# Random tiny instances
# ---------------------------------------------------------------------------
def _random_instance(seed, T=3, B=5, D=4, max_len=4, rows=(5, 1, 7), dtype="f32", empty=True):
    rng = np.random.default_rng(seed)
    rows = list(rows)[:T]
    lengths = rng.integers(0 if empty else 1, max_len + 1, size=T * B)
    if empty:
        lengths[1] = 0
    idx = np.concatenate([rng.integers(0, rows[t], size=int(lengths[t * B:(t + 1) * B].sum()))
                          for t in range(T)]).astype(np.int32)
    if dtype == "f64":
        tabs = [rng.standard_normal((n, D)) for n in rows]
    else:
        tabs = [rng.standard_normal((n, D)).astype(np.float32) for n in rows]
    e0 = rng.standard_normal((B, D)).astype(np.float32)
    return tabs, orc.lengths_to_offsets(lengths), idx, e0, lengths


@pytest.mark.parametrize("seed", range(6))
def test_pool_equals_count_matrix_product(seed):
    """EmbeddingBag-sum equals (bag-count matrix) @ table, a textbook identity."""
    tabs, off, idx, _, _ = _random_instance(seed)
    T, B = len(tabs), 5
    pooled = orc.embbag_pool(tabs, "f32", B, off, idx)
    for t in range(T):
        A = np.zeros((B, tabs[t].shape[0]))
        for b in range(B):
            for p in range(off[t * B + b], off[t * B + b + 1]):
                A[b, idx[p]] += 1.0
        np.testing.assert_allclose(pooled[:, t], A @ tabs[t].astype(np.float64), rtol=1e-14, atol=1e-14)


def test_pool_single_index_is_the_row_exactly():
    rng = np.random.default_rng(7)
    tab = rng.standard_normal((50, 8)).astype(np.float16)
    idx = rng.integers(0, 50, size=10).astype(np.int32)
    off = np.arange(11)
    pooled = orc.embbag_pool([tab], "f16", 10, off, idx)
    np.testing.assert_array_equal(pooled[:, 0], tab[idx].astype(np.float64))


@pytest.mark.parametrize("k", [1, 2, 3, 7, 32])
def test_pool_repeated_index_counts_k_times(k):
    tab = np.random.default_rng(k).standard_normal((4, 16)).astype(np.float32)
    idx = np.full(k, 2, dtype=np.int32)
    pooled = orc.embbag_pool([tab], "f32", 1, np.array([0, k]), idx)
    np.testing.assert_array_equal(pooled[0, 0], k * tab[2].astype(np.float64))


def test_pool_empty_bag_is_positive_zero():
    tab = np.ones((3, 4), np.float32)
    pooled = orc.embbag_pool([tab], "f32", 2, np.array([0, 0, 2]), np.array([0, 1], np.int32))
    assert np.all(pooled[0, 0] == 0.0) and not np.any(np.signbit(pooled[0, 0]))
    np.testing.assert_array_equal(pooled[1, 0], [2, 2, 2, 2])


def test_pool_permutation_invariant_exact_integers():
    rng = np.random.default_rng(3)
    tab = rng.integers(-4, 5, size=(20, 8)).astype(np.float32)
    idx = rng.integers(0, 20, size=12).astype(np.int32)
    a = orc.embbag_pool([tab], "f32", 1, np.array([0, 12]), idx)
    b = orc.embbag_pool([tab], "f32", 1, np.array([0, 12]), idx[::-1].copy())
    np.testing.assert_array_equal(a, b)


def test_decode_bf16_and_f16_exact():
    # bf16 bit patterns of 1.0, -2.0, 0.5, 3.140625 (0x4049), smallest normal
    bits = np.array([[0x3F80, 0xC000, 0x3F00, 0x4049, 0x0080]], dtype=np.uint16)
    v = orc.decode(bits, "bf16")
    assert v.tolist() == [[1.0, -2.0, 0.5, 3.140625, 2.0 ** -126]]
    h = np.array([[1.5, -0.25, 65504.0]], dtype=np.float16)
    assert orc.decode(h, "f16").tolist() == [[1.5, -0.25, 65504.0]]


# ---------------------------------------------------------------------------
# Interaction
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("F", [2, 3, 5, 9, 27])
def test_interaction_equals_gram_strict_lower(F):
    """Dots equal the strict lower triangle of Z Z^T in numpy's row-major tril order."""
    rng = np.random.default_rng(F)
    B, D = 4, 6
    e0 = rng.standard_normal((B, D))
    pooled = rng.standard_normal((B, F - 1, D))
    out = orc.interact(e0, pooled)
    assert out.shape == (B, D + F * (F - 1) // 2)
    np.testing.assert_array_equal(out[:, :D], e0)
    ii, jj = np.tril_indices(F, -1)
    for b in range(B):
        Z = np.vstack([e0[b][None], pooled[b]])
        G = Z @ Z.T
        np.testing.assert_allclose(out[b, D:], G[ii, jj], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(G, G.T, rtol=0, atol=1e-13)


@pytest.mark.parametrize("F", range(1, 70))
def test_pair_count_and_order(F):
    pr = list(orc.pairs(F))
    assert len(pr) == F * (F - 1) // 2 == orc.pair_count(F)
    assert [k for k, _, _ in pr] == list(range(len(pr)))
    assert all(k == i * (i - 1) // 2 + j and 0 <= j < i < F for k, i, j in pr)
    assert len({(i, j) for _, i, j in pr}) == len(pr)


@pytest.mark.parametrize("seed", range(4))
def test_interaction_fm_identity(seed):
    """Sum of pairwise dots = 1/2 (|sum_i z_i|^2 - sum_i |z_i|^2) (FM second-order term)."""
    rng = np.random.default_rng(100 + seed)
    B, T, D = 3, 12, 16
    e0 = rng.standard_normal((B, D))
    pooled = rng.standard_normal((B, T, D))
    out = orc.interact(e0, pooled)
    Z = np.concatenate([e0[:, None], pooled], axis=1)
    fm = 0.5 * ((Z.sum(axis=1) ** 2).sum(axis=1) - (Z ** 2).sum(axis=(1, 2)))
    np.testing.assert_allclose(out[:, D:].sum(axis=1), fm, rtol=1e-12)


def test_interaction_orthogonal_and_parallel_vectors():
    F, D = 6, 8
    e0 = np.zeros((2, D))
    e0[0, 0] = 3.0
    e0[1, 0] = 1.0
    pooled = np.zeros((2, F - 1, D))
    for i in range(F - 1):
        pooled[0, i, i + 1] = i + 2.0   # mutually orthogonal rows -> every dot is 0
        pooled[1, i, 0] = 1.0           # identical unit rows -> every dot is 1
    out = orc.interact(e0, pooled)
    assert np.all(out[0, D:] == 0.0)
    assert np.all(out[1, D:] == 1.0)


# ---------------------------------------------------------------------------
# Backward: finite differences of a quadratic loss are exact up to rounding
# ---------------------------------------------------------------------------
def _loss(tabs, B, off, idx, e0, d_out):
    r = orc.embbag_fwd(tabs, "f64", B, off, idx, e0)
    return float((r["out"] * d_out).sum())


@pytest.mark.parametrize("seed", range(3))
def test_backward_matches_finite_differences(seed):
    tabs, off, idx, e0, _ = _random_instance(seed, dtype="f64")
    e0 = e0.astype(np.float64)
    B = 5
    rng = np.random.default_rng(50 + seed)
    F = len(tabs) + 1
    D = tabs[0].shape[1]
    d_out = rng.standard_normal((B, D + F * (F - 1) // 2))
    fwd = orc.embbag_fwd(tabs, "f64", B, off, idx, e0)
    r = orc.embbag_bwd_update(tabs, "f64", B, off, idx, e0, fwd["pooled"], d_out, lr=0.0)
    base = r["base"]
    grad_of = {int(k): r["grad"][u] for u, k in enumerate(r["unique_keys"])}
    h = 1e-3
    for t, tab in enumerate(tabs):
        for row in range(tab.shape[0]):
            for d in range(D):
                tp = [x.copy() for x in tabs]
                tm = [x.copy() for x in tabs]
                tp[t][row, d] += h
                tm[t][row, d] -= h
                fd = (_loss(tp, B, off, idx, e0, d_out) - _loss(tm, B, off, idx, e0, d_out)) / (2 * h)
                want = grad_of.get(int(base[t]) + row, np.zeros(D))[d]
                assert abs(fd - want) <= 1e-8 * (1 + abs(fd)), (t, row, d, fd, want)
    for b in range(B):
        for d in range(D):
            ep = e0.copy()
            em = e0.copy()
            ep[b, d] += h
            em[b, d] -= h
            fd = (_loss(tabs, B, off, idx, ep, d_out) - _loss(tabs, B, off, idx, em, d_out)) / (2 * h)
            assert abs(fd - r["d_e0"][b, d]) <= 1e-8 * (1 + abs(fd))


def test_backward_gradient_conservation():
    tabs, off, idx, e0, _ = _random_instance(11, B=5)
    fwd = orc.embbag_fwd(tabs, "f32", 5, off, idx, e0)
    d_out = np.random.default_rng(1).standard_normal((5, 4 + 6))
    r = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], d_out, lr=0.01)
    _, tab, smp, _ = orc.occurrence_keys([t.shape[0] for t in tabs], 5, off, idx)
    total = sum(r["dZ"][smp[p], 1 + tab[p]] for p in range(len(idx)))
    np.testing.assert_allclose(r["grad"].sum(axis=0), total, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Sort and segments: brute force
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(5))
def test_stable_order_and_segments_brute_force(seed):
    rng = np.random.default_rng(seed)
    keys = rng.integers(0, 9, size=40)
    perm = orc.stable_order(keys)
    assert perm.tolist() == sorted(range(40), key=lambda p: (keys[p], p))
    uniq, seg = orc.segments(keys[perm])
    groups = [(k, len(list(g))) for k, g in itertools.groupby(sorted(keys.tolist()))]
    assert uniq.tolist() == [k for k, _ in groups]
    assert seg[0] == 0 and seg[-1] == 40
    assert np.diff(seg).tolist() == [c for _, c in groups]
    assert np.all(np.diff(uniq) > 0)


def test_sgd_untouched_rows_and_closed_form():
    tabs, off, idx, e0, _ = _random_instance(5, B=5)
    fwd = orc.embbag_fwd(tabs, "f32", 5, off, idx, e0)
    d_out = np.random.default_rng(2).standard_normal((5, 4 + 6))
    lr = 0.01
    r = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], d_out, lr=lr)
    base = r["base"]
    touched = set(int(k) for k in r["unique_keys"])
    used = set(int(base[t]) + int(i) for t in range(3)
               for i in idx[off[t * 5]:off[(t + 1) * 5]])
    assert touched == used
    for u, k in enumerate(r["unique_keys"]):
        t = int(np.searchsorted(base, k, side="right") - 1)
        np.testing.assert_allclose(r["new_rows"][u], tabs[t][k - base[t]] - lr * r["grad"][u], rtol=1e-15)


# ---------------------------------------------------------------------------
# Status bits
# ---------------------------------------------------------------------------
def test_status_bits():
    rows = [4, 2]
    good_off = np.array([0, 1, 2, 3, 4])
    good_idx = np.array([0, 3, 1, 0], np.int32)
    assert orc.bag_status(2, 2, rows, good_off, good_idx) == 0
    assert orc.bag_status(2, 2, rows, good_off, np.array([0, 4, 1, 0], np.int32)) == oracle.STATUS_BAD_INDEX
    assert orc.bag_status(2, 2, rows, good_off, np.array([0, 3, 2, 0], np.int32)) == oracle.STATUS_BAD_INDEX
    assert orc.bag_status(2, 2, rows, good_off, np.array([-1, 3, 1, 0], np.int32)) == oracle.STATUS_BAD_INDEX
    assert orc.bag_status(2, 2, rows, np.array([0, 2, 1, 3, 4]), good_idx) == oracle.STATUS_BAD_OFFSETS
    assert orc.bag_status(2, 2, rows, np.array([0, 1, 2, 3, 3]), good_idx) == oracle.STATUS_BAD_OFFSETS
    assert orc.bag_status(2, 2, rows, np.array([1, 1, 2, 3, 4]), good_idx) == oracle.STATUS_BAD_OFFSETS
    with pytest.raises(oracle.BagError) as ei:
        orc.embbag_pool([np.zeros((4, 4), np.float32), np.zeros((2, 4), np.float32)], "f32", 2,
                        good_off, np.array([0, 4, 1, 0], np.int32))
    assert ei.value.bits == oracle.STATUS_BAD_INDEX


# ---------------------------------------------------------------------------
# Planted mistakes: each pin above must catch a plausible oracle bug
# ---------------------------------------------------------------------------
def test_planted_mistakes_are_caught(monkeypatch, golden_dir):
    g = _golden(golden_dir)
    idx = np.array(g["indices"], dtype=np.int32)
    off = np.array(g["offsets"])
    e0 = np.array(g["e0"], np.float32)
    good = orc.embbag_fwd(_tables_f32(g), "f32", 2, off, idx, e0)["out"]

    # (a) column-major pair order instead of row-major
    def bad_pairs(F, self_pairs=False):
        k = 0
        for j in range(F):
            for i in range(j if self_pairs else j + 1, F):
                yield k, i, j
                k += 1
    with monkeypatch.context() as m:
        m.setattr(orc, "pairs", bad_pairs)
        with pytest.raises(AssertionError):
            test_golden_pair_order(golden_dir)
        with pytest.raises(AssertionError):
            test_interaction_equals_gram_strict_lower(5)

    # (b) backward dropping the dZ_j term
    def bad_bwd(e0_, pooled, d_out, self_pairs=False, with_embeddings=False):
        B, T, D = pooled.shape
        Z = orc.stack_z(np.asarray(e0_, np.float64), pooled)
        dZ = np.zeros_like(Z)
        for k, i, j in orc.pairs(T + 1):
            dZ[:, i] += np.asarray(d_out, np.float64)[:, D + k][:, None] * Z[:, j]
        return {"dZ": dZ, "d_e0": np.asarray(d_out, np.float64)[:, :D] + dZ[:, 0], "d_pooled": dZ[:, 1:]}
    with monkeypatch.context() as m:
        m.setattr(orc, "interact_bwd", bad_bwd)
        r = orc.embbag_bwd_update(_tables_f32(g), "f32", 2, off, idx, e0, np.array(g["pooled"], np.float64),
                                  np.array(g["d_out"], np.float32), g["lr"])
        assert not np.array_equal(r["grad"], np.array(g["grad"], dtype=np.float64))

    # (c) an unstable sort changes the permutation on ties
    with monkeypatch.context() as m:
        m.setattr(orc, "stable_order", lambda k: np.argsort(-np.asarray(k), kind="stable")[::-1])
        r = orc.embbag_bwd_update(_tables_f32(g), "f32", 2, off, idx, e0, np.array(g["pooled"], np.float64),
                                  np.array(g["d_out"], np.float32), g["lr"])
        assert r["perm"].tolist() != g["perm"]
    assert np.array_equal(good, np.array(g["out"], dtype=np.float64))


def test_planted_pool_decode_sgd_segment_mistakes(monkeypatch, golden_dir):
    """More plausible oracle bugs, each caught by a pin that does not use the oracle's code."""
    real_pool = orc.embbag_pool
    real_decode = orc.decode
    real_segments = orc.segments

    # (d) pooling that drops the last row of every bag (off-by-one on the CSR end)
    def short_pool(tables, dtype, B, offsets, indices):
        off = np.asarray(offsets).copy()
        T = len(tables)
        pooled = np.zeros((B, T, tables[0].shape[1]))
        for t in range(T):
            for b in range(B):
                s, e = int(off[t * B + b]), int(off[t * B + b + 1])
                for p in range(s, max(s, e - 1)):
                    pooled[b, t] += real_decode(tables[t][int(indices[p])], dtype)
        return pooled
    with monkeypatch.context() as m:
        m.setattr(orc, "embbag_pool", short_pool)
        with pytest.raises(AssertionError):
            test_pool_equals_count_matrix_product(0)
        with pytest.raises(AssertionError):
            test_golden_forward(golden_dir)

    # (e) bf16 decode with the wrong shift (bits << 15)
    def bad_decode(table, dtype):
        if dtype == "bf16":
            return (table.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        return real_decode(table, dtype)
    with monkeypatch.context() as m:
        m.setattr(orc, "decode", bad_decode)
        with pytest.raises(AssertionError):
            test_decode_bf16_and_f16_exact()

    # (f) SGD with the wrong sign: caught by the hand-worked updated rows
    g = _golden(golden_dir)
    r = orc.embbag_bwd_update(_tables_f32(g), "f32", 2, np.array(g["offsets"]), np.array(g["indices"], np.int32),
                              np.array(g["e0"], np.float32), np.array(g["pooled"], np.float64),
                              np.array(g["d_out"], np.float32), -g["lr"])
    assert not np.array_equal(r["new_rows"], np.array(g["new_rows"], dtype=np.float64))

    # (g) segments that start a new run one position late
    def late_segments(sorted_keys):
        u, s = real_segments(sorted_keys)
        s = s.copy()
        s[1:-1] += 1
        return u, s
    with monkeypatch.context() as m:
        m.setattr(orc, "segments", late_segments)
        with pytest.raises(AssertionError):
            test_golden_backward(golden_dir)
        with pytest.raises(AssertionError):
            test_stable_order_and_segments_brute_force(0)


# ---------------------------------------------------------------------------
# Interaction with self-pairs (i >= j)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("F", [1, 2, 5, 27])
def test_self_pair_interaction_equals_gram_lower_with_diagonal(F):
    """With self-pairs the dots are numpy's lower triangle of Z Z^T, diagonal included,
    in row-major order, F(F+1)/2 of them."""
    rng = np.random.default_rng(F)
    B, D = 3, 8
    e0 = rng.standard_normal((B, D))
    pooled = rng.standard_normal((B, F - 1, D))
    out = orc.interact(e0, pooled, self_pairs=True)
    assert out.shape == (B, D + F * (F + 1) // 2)
    Z = np.concatenate([e0[:, None], pooled], axis=1)
    il, jl = np.tril_indices(F)
    for b in range(B):
        np.testing.assert_allclose(out[b, D:], (Z[b] @ Z[b].T)[il, jl], rtol=1e-13, atol=1e-13)


def test_self_pair_fm_identity_and_hand_example():
    """Sum over i >= j of z_i . z_j = 1/2 (|sum z|^2 + sum |z|^2); and a hand-worked F=3 case:
    z0=(1,0), z1=(2,1), z2=(0,3) -> (0,0)=1, (1,0)=2, (1,1)=5, (2,0)=0, (2,1)=3, (2,2)=9."""
    rng = np.random.default_rng(9)
    e0 = rng.standard_normal((4, 6))
    pooled = rng.standard_normal((4, 5, 6))
    out = orc.interact(e0, pooled, self_pairs=True)
    Z = np.concatenate([e0[:, None], pooled], axis=1)
    s = Z.sum(axis=1)
    np.testing.assert_allclose(out[:, 6:].sum(axis=1), 0.5 * ((s * s).sum(1) + (Z * Z).sum((1, 2))), rtol=1e-12)
    hand = orc.interact(np.array([[1.0, 0.0]]), np.array([[[2.0, 1.0], [0.0, 3.0]]]), self_pairs=True)
    assert hand[0].tolist() == [1.0, 0.0, 1.0, 2.0, 5.0, 0.0, 3.0, 9.0]


@pytest.mark.parametrize("self_pairs", [False, True])
def test_interaction_backward_finite_differences(self_pairs):
    """<d_out, out(Z)> is quadratic in Z: the central difference is exact up to rounding."""
    rng = np.random.default_rng(5 + self_pairs)
    B, T, D = 2, 3, 4
    e0 = rng.standard_normal((B, D))
    pooled = rng.standard_normal((B, T, D))
    P = orc.pair_count(T + 1, self_pairs)
    d_out = rng.standard_normal((B, D + P))
    g = orc.interact_bwd(e0, pooled, d_out, self_pairs=self_pairs)

    def loss(e, p):
        return float((d_out * orc.interact(e, p, self_pairs=self_pairs)).sum())
    h = 1e-3
    for b in range(B):
        for f in range(T + 1):
            for d in range(D):
                ep, pp = e0.copy(), pooled.copy()
                em, pm = e0.copy(), pooled.copy()
                if f == 0:
                    ep[b, d] += h
                    em[b, d] -= h
                    want = g["d_e0"][b, d]
                else:
                    pp[b, f - 1, d] += h
                    pm[b, f - 1, d] -= h
                    want = g["dZ"][b, f, d]
                num = (loss(ep, pp) - loss(em, pm)) / (2 * h)
                assert abs(num - want) < 1e-8 * (1 + abs(want))


# ---------------------------------------------------------------------------
# Row-wise AdaGrad
# ---------------------------------------------------------------------------
def _adagrad_instance(seed, scale=1.0):
    tabs, off, idx, e0, _ = _random_instance(seed, B=5)
    fwd = orc.embbag_fwd(tabs, "f32", 5, off, idx, e0)
    d_out = np.random.default_rng(seed + 1).standard_normal((5, 4 + 6)) * scale
    return tabs, off, idx, e0, fwd, d_out


def test_adagrad_first_step_moves_each_row_by_lr_rms():
    """From a zero state, the first row-wise AdaGrad step divides G by its own RMS:
    every touched row moves by exactly lr in RMS (eps -> 0), whatever the gradient."""
    tabs, off, idx, e0, fwd, d_out = _adagrad_instance(3)
    r = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], d_out, 0.05,
                              optimizer="rowwise_adagrad", eps=1e-30)
    for u, k in enumerate(r["unique_keys"]):
        t = int(np.searchsorted(r["base"], k, side="right") - 1)
        w = tabs[t][k - r["base"][t]].astype(np.float64)
        step = w - r["new_rows"][u]
        assert abs(np.sqrt(np.mean(step * step)) - 0.05) < 1e-12
        assert abs(r["new_state"][u] - np.mean(r["grad"][u] ** 2)) <= 1e-15 * (1 + r["new_state"][u])


def test_adagrad_first_step_is_scale_invariant_and_sgd_is_not():
    tabs, off, idx, e0, fwd, d1 = _adagrad_instance(4)
    a = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], d1, 0.1, optimizer="rowwise_adagrad",
                              eps=1e-30)
    b = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], 37.0 * d1, 0.1,
                              optimizer="rowwise_adagrad", eps=1e-30)
    np.testing.assert_allclose(a["new_rows"], b["new_rows"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b["new_state"], 37.0 ** 2 * a["new_state"], rtol=1e-12)
    s1 = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], d1, 0.1)
    s2 = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], 37.0 * d1, 0.1)
    assert not np.allclose(s1["new_rows"], s2["new_rows"])


def test_adagrad_state_accumulates_and_damps_the_step():
    """With the state of a first step carried into a second identical gradient, the
    second step is the first divided by sqrt(2) (state doubles, eps -> 0)."""
    tabs, off, idx, e0, fwd, d_out = _adagrad_instance(6)
    r1 = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], d_out, 0.1,
                               optimizer="rowwise_adagrad", eps=1e-30)
    state = [np.zeros(t.shape[0]) for t in tabs]
    for u, k in enumerate(r1["unique_keys"]):
        t = int(np.searchsorted(r1["base"], k, side="right") - 1)
        state[t][k - r1["base"][t]] = r1["new_state"][u]
    r2 = orc.embbag_bwd_update(tabs, "f32", 5, off, idx, e0, fwd["pooled"], d_out, 0.1,
                               optimizer="rowwise_adagrad", state=state, eps=1e-30)
    np.testing.assert_allclose(r2["new_state"], 2 * r1["new_state"], rtol=1e-14)
    for u, k in enumerate(r1["unique_keys"]):
        t = int(np.searchsorted(r1["base"], k, side="right") - 1)
        w = tabs[t][k - r1["base"][t]].astype(np.float64)
        np.testing.assert_allclose(w - r2["new_rows"][u], (w - r1["new_rows"][u]) / np.sqrt(2.0), rtol=1e-12)


# ---------------------------------------------------------------------------
# Row-wise 4-bit tables
# ---------------------------------------------------------------------------
def _q4_golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_example_q4_rows.json")) as f:
        return json.load(f)


def test_q4_decode_hand_worked_nibbles(golden_dir):
    """Stored bytes decoded by hand: the low 4 bits of a code byte are the even column."""
    g = _q4_golden(golden_dir)
    tab = orc.Q4Table(np.array(g["stored"], dtype=np.uint8), g["D"])
    for r, want in enumerate(g["rows"]):
        assert orc.decode(tab[r], "q4").tolist() == want
    off = np.array(g["bags"]["offsets"])
    idx = np.array(g["bags"]["indices"], dtype=np.int32)
    got = orc.embbag_pool([tab], "q4", len(off) - 1, off, idx)
    assert got[:, 0].tolist() == g["bags"]["pooled"]


def test_q4_pool_equals_dequantized_f64():
    """Pooling 4-bit rows equals pooling the rows dequantized in fp64 from the unpacked
    codes (the synthetic packer's codes and pairs, not the oracle's decoder)."""
    rng = np.random.default_rng(44)
    D = 16
    codes = rng.integers(0, 16, size=(30, D)).astype(np.uint8)
    sb = np.stack([rng.uniform(1e-3, 1e-1, 30), rng.uniform(-1, 1, 30)], axis=1).astype(np.float32)
    from sparse_embedding_lookup_dlrm_amd import synth
    stored = synth.pack_q4_rows(codes, sb)
    assert stored.shape == (30, synth.q4_row_stride(D))
    deq = codes.astype(np.float64) * sb[:, 0:1].astype(np.float64) + sb[:, 1:2].astype(np.float64)
    idx = rng.integers(0, 30, size=25).astype(np.int32)
    off = np.array([0, 3, 3, 10, 25])
    got = orc.embbag_pool([orc.Q4Table(stored, D)], "q4", 4, off, idx)
    want = orc.embbag_pool([deq], "f64", 4, off, idx)
    np.testing.assert_array_equal(got, want)


def test_q4_planted_nibble_swap_is_caught(monkeypatch, golden_dir):
    """A decoder that reads the high 4 bits as the even column fails the hand-worked pin."""
    def swapped(row, D):
        q = np.zeros(D)
        for k in range(D // 2):
            q[2 * k], q[2 * k + 1] = int(row[k]) >> 4, int(row[k]) & 0xF
        scale = float(np.frombuffer(bytes(row[D // 2:D // 2 + 4]), dtype="<f4")[0])
        bias = float(np.frombuffer(bytes(row[D // 2 + 4:D // 2 + 8]), dtype="<f4")[0])
        return scale * q + bias
    with monkeypatch.context() as m:
        m.setattr(orc, "decode_q4_row", swapped)
        with pytest.raises(AssertionError):
            test_q4_decode_hand_worked_nibbles(golden_dir)


# ---------------------------------------------------------------------------
# Table-wise 8-bit tables
# ---------------------------------------------------------------------------
def test_q8_table_wise_hand_example():
    """One (scale, bias) pair for the table: rows decode with that pair, and a bag of n
    rows pools to scale * (sum of its codes) + n * bias (worked by hand)."""
    codes = np.array([[0, 255, 128], [7, 0, 1], [2, 2, 2]], dtype=np.uint8)
    tab = orc.Q8Table.table_wise(codes, 0.5, -1.0)
    assert orc.decode(tab[1], "q8").tolist() == [2.5, -1.0, -0.5]
    off = np.array([0, 2, 5])
    idx = np.array([0, 1, 1, 2, 2], dtype=np.int32)
    got = orc.embbag_pool([tab], "q8", 2, off, idx)
    assert got[0, 0].tolist() == [0.5 * 7 - 2, 0.5 * 255 - 2, 0.5 * 129 - 2]
    assert got[1, 0].tolist() == [0.5 * 11 - 3, 0.5 * 4 - 3, 0.5 * 5 - 3]



# ---------------------------------------------------------------------------
# Interaction layouts: self-pairs and the embeddings concatenated alongside
# ---------------------------------------------------------------------------
_LAYOUTS = {"strict": (False, False), "self_pairs": (True, False), "with_embeddings": (False, True),
            "self_pairs_with_embeddings": (True, True)}


def test_golden_layouts(golden_dir):
    """The four layouts and the with-embeddings backward against hand-worked values."""
    with open(os.path.join(golden_dir, "worked_example_layouts_f3_d2.json")) as f:
        g = json.load(f)
    e0, pooled = np.array(g["e0"], float), np.array(g["pooled"], float)
    for name, (sp, we) in _LAYOUTS.items():
        assert orc.interact(e0, pooled, self_pairs=sp, with_embeddings=we).tolist() == g["out"][name], name
    bw = g["backward_with_embeddings"]
    r = orc.interact_bwd(e0, pooled, np.array(bw["d_out"], float), with_embeddings=True)
    assert r["d_e0"].tolist() == bw["d_e0"]
    assert r["d_pooled"].tolist() == bw["d_pooled"]


@pytest.mark.parametrize("self_pairs", [False, True])
def test_with_embeddings_output_is_z_then_the_dots_of_the_plain_layout(self_pairs):
    """With the embeddings concatenated the row is Z's F vectors (a copy) followed by exactly
    the dots of the layout without them."""
    rng = np.random.default_rng(17 + self_pairs)
    B, T, D = 3, 5, 6
    e0, pooled = rng.standard_normal((B, D)), rng.standard_normal((B, T, D))
    a = orc.interact(e0, pooled, self_pairs=self_pairs, with_embeddings=True)
    b = orc.interact(e0, pooled, self_pairs=self_pairs)
    F = T + 1
    assert a.shape == (B, F * D + orc.pair_count(F, self_pairs))
    np.testing.assert_array_equal(a[:, :D], e0)
    np.testing.assert_array_equal(a[:, D:F * D].reshape(B, T, D), pooled)
    np.testing.assert_array_equal(a[:, F * D:], b[:, D:])


@pytest.mark.parametrize("self_pairs", [False, True])
def test_with_embeddings_backward_finite_differences(self_pairs):
    """<d_out, out(Z)> stays quadratic in Z with the embeddings concatenated (their part is
    linear): the central difference is exact up to rounding."""
    rng = np.random.default_rng(23 + self_pairs)
    B, T, D = 2, 3, 4
    e0 = rng.standard_normal((B, D))
    pooled = rng.standard_normal((B, T, D))
    d_out = rng.standard_normal((B, (T + 1) * D + orc.pair_count(T + 1, self_pairs)))
    g = orc.interact_bwd(e0, pooled, d_out, self_pairs=self_pairs, with_embeddings=True)

    def loss(e, p):
        return float((d_out * orc.interact(e, p, self_pairs=self_pairs, with_embeddings=True)).sum())
    h = 1e-3
    for b in range(B):
        for f in range(T + 1):
            for d in range(D):
                ep, pp, em, pm = e0.copy(), pooled.copy(), e0.copy(), pooled.copy()
                if f == 0:
                    ep[b, d] += h
                    em[b, d] -= h
                    want = g["d_e0"][b, d]
                else:
                    pp[b, f - 1, d] += h
                    pm[b, f - 1, d] -= h
                    want = g["d_pooled"][b, f - 1, d]
                num = (loss(ep, pp) - loss(em, pm)) / (2 * h)
                assert abs(num - want) <= 1e-8 * (1 + abs(want)), (b, f, d, num, want)


@pytest.mark.parametrize("self_pairs,with_emb", [(True, False), (False, True), (True, True)])
def test_sparse_backward_layouts_match_finite_differences(self_pairs, with_emb):
    """The row gradients of the sparse backward in every interaction layout equal central
    differences of <d_out, forward(tables)> taken through the whole forward (pooling,
    then the layout's output)."""
    tabs, off, idx, e0, _ = _random_instance(7, dtype="f64")
    e0 = e0.astype(np.float64)
    B = 5
    T, D = len(tabs), tabs[0].shape[1]
    W = ((T + 1) * D if with_emb else D) + orc.pair_count(T + 1, self_pairs)
    d_out = np.random.default_rng(71).standard_normal((B, W))

    def loss(tb):
        r = orc.embbag_fwd(tb, "f64", B, off, idx, e0, self_pairs=self_pairs, with_embeddings=with_emb)
        return float((r["out"] * d_out).sum())
    fwd = orc.embbag_fwd(tabs, "f64", B, off, idx, e0, self_pairs=self_pairs, with_embeddings=with_emb)
    r = orc.embbag_bwd_update(tabs, "f64", B, off, idx, e0, fwd["pooled"], d_out, lr=0.0,
                              self_pairs=self_pairs, with_embeddings=with_emb)
    grad_of = {int(k): r["grad"][u] for u, k in enumerate(r["unique_keys"])}
    h = 1e-3
    for t, tab in enumerate(tabs):
        for row in range(tab.shape[0]):
            for d in range(D):
                tp = [x.copy() for x in tabs]
                tm = [x.copy() for x in tabs]
                tp[t][row, d] += h
                tm[t][row, d] -= h
                fd = (loss(tp) - loss(tm)) / (2 * h)
                want = grad_of.get(int(r["base"][t]) + row, np.zeros(D))[d]
                assert abs(fd - want) <= 1e-8 * (1 + abs(fd)), (t, row, d, fd, want)


def test_planted_layout_mistakes_are_caught(monkeypatch, golden_dir):
    """A backward that forgets the direct gradient of the concatenated embeddings, and a
    forward that puts the dots before the embeddings, both fail the pins above."""
    real_bwd = orc.interact_bwd

    def no_direct(e0, pooled, d_out, self_pairs=False, with_embeddings=False):
        r = real_bwd(e0, pooled, d_out, self_pairs=self_pairs, with_embeddings=with_embeddings)
        r["d_pooled"] = r["dZ"][:, 1:].copy()
        return r
    with monkeypatch.context() as m:
        m.setattr(orc, "interact_bwd", no_direct)
        with pytest.raises(AssertionError):
            test_golden_layouts(golden_dir)
        with pytest.raises(AssertionError):
            test_with_embeddings_backward_finite_differences(False)
        with pytest.raises(AssertionError):
            test_sparse_backward_layouts_match_finite_differences(False, True)
    real_fwd = orc.interact

    def dots_first(e0, pooled, self_pairs=False, with_embeddings=False):
        out = real_fwd(e0, pooled, self_pairs=self_pairs, with_embeddings=with_embeddings)
        if not with_embeddings:
            return out
        F, D = pooled.shape[1] + 1, pooled.shape[2]
        return np.concatenate([out[:, F * D:], out[:, :F * D]], axis=1)
    with monkeypatch.context() as m:
        m.setattr(orc, "interact", dots_first)
        with pytest.raises(AssertionError):
            test_golden_layouts(golden_dir)
