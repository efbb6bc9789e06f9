"""Host-side check of the fact the backward's key build relies on: with offsets clamped
into [0, nnz], bag j holding [o_j, max(o_j, o_{j+1})) plus the two gaps [0, o_0) and
[o_last, nnz) cover every position 0..nnz-1 (for any offsets, valid or not)."""
import numpy as np


def _covered(off, nnz):
    c = np.clip(np.asarray(off, dtype=np.int64), 0, nnz)
    cov = np.zeros(nnz, bool)
    for j in range(len(c) - 1):
        cov[c[j]:max(c[j], c[j + 1])] = True
    cov[0:c[0]] = True
    cov[c[-1]:nnz] = True
    return cov


def test_every_position_is_covered_for_arbitrary_offsets():
    rng = np.random.default_rng(0)
    for trial in range(3000):
        nnz = int(rng.integers(0, 60))
        nb = int(rng.integers(1, 12))
        kind = trial % 3
        if kind == 0:  # valid CSR
            cuts = np.sort(rng.integers(0, nnz + 1, size=nb - 1))
            off = np.concatenate([[0], cuts, [nnz]])
        elif kind == 1:  # arbitrary values, in and out of range, any order
            off = rng.integers(-10, nnz + 10, size=nb + 1)
        else:  # a valid CSR with a few entries disturbed
            cuts = np.sort(rng.integers(0, nnz + 1, size=nb - 1))
            off = np.concatenate([[0], cuts, [nnz]])
            k = rng.integers(0, nb + 1, size=2)
            off[k] = rng.integers(-5, nnz + 5, size=2)
        assert _covered(off, nnz).all(), (off, nnz)


def test_valid_offsets_leave_no_gap():
    off = [0, 3, 3, 7, 12]
    c = np.asarray(off)
    assert c[0] == 0 and c[-1] == 12  # both gaps empty: the bags alone cover [0, 12)
    cov = np.zeros(12, bool)
    for j in range(4):
        cov[c[j]:c[j + 1]] = True
    assert cov.all()
