"""GPU parity of the standalone interaction (both pair sets) and of its exported
backward against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import dlrm_oracle as orc
from sparse_embedding_lookup_dlrm_amd import ops

from gpu_util import assert_mag_close, need_gpu

pytestmark = pytest.mark.gpu
RTOL = 1e-5  # fp32 inputs


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _inputs(B, T, D, seed, integer=False):
    rng = np.random.default_rng(seed)
    if integer:
        e0 = rng.integers(-3, 4, size=(B, D)).astype(np.float32)
        pooled = rng.integers(-3, 4, size=(B, T, D)).astype(np.float32)
    else:
        e0 = rng.standard_normal((B, D)).astype(np.float32)
        pooled = (rng.standard_normal((B, T, D)) * 0.1).astype(np.float32)
    return e0, pooled


@pytest.mark.parametrize("self_pairs", [False, True])
@pytest.mark.parametrize("B,T,D", [(1, 1, 4), (7, 3, 16), (130, 26, 128), (33, 64, 128), (5, 100, 32)])
def test_interact_forward(self_pairs, B, T, D):
    e0, pooled = _inputs(B, T, D, seed=B * 1000 + T + D + self_pairs)
    out = ops.interact(torch.from_numpy(e0).cuda(), torch.from_numpy(pooled).cuda(), self_pairs=self_pairs)
    torch.cuda.synchronize()
    ref = orc.interact(e0, pooled, self_pairs=self_pairs)
    mag = orc.interact(np.abs(e0), np.abs(pooled), self_pairs=self_pairs)
    got = out.cpu().numpy()
    assert got.shape == ref.shape
    np.testing.assert_array_equal(got[:, :D], e0)
    assert_mag_close(got[:, D:], ref[:, D:], mag[:, D:], RTOL, "dots")


@pytest.mark.parametrize("self_pairs", [False, True])
def test_interact_forward_exact_integers(self_pairs):
    e0, pooled = _inputs(50, 12, 64, seed=5, integer=True)
    out = ops.interact(torch.from_numpy(e0).cuda(), torch.from_numpy(pooled).cuda(), self_pairs=self_pairs)
    np.testing.assert_array_equal(out.cpu().numpy(), orc.interact(e0, pooled, self_pairs=self_pairs).astype(np.float32))


@pytest.mark.parametrize("self_pairs", [False, True])
@pytest.mark.parametrize("B,T,D", [(1, 1, 4), (9, 5, 16), (64, 26, 128), (17, 64, 64)])
def test_interact_backward(self_pairs, B, T, D):
    e0, pooled = _inputs(B, T, D, seed=B + 7 * T + D + 100 * self_pairs)
    P = orc.pair_count(T + 1, self_pairs)
    d_out = np.random.default_rng(B * T).standard_normal((B, D + P)).astype(np.float32)
    d_e0, d_pooled = ops.interact_bwd(torch.from_numpy(e0).cuda(), torch.from_numpy(pooled).cuda(),
                                      torch.from_numpy(d_out).cuda(), self_pairs=self_pairs)
    torch.cuda.synchronize()
    r = orc.interact_bwd(e0, pooled, d_out, self_pairs=self_pairs)
    m = orc.interact_bwd(np.abs(e0), np.abs(pooled), np.abs(d_out), self_pairs=self_pairs)
    assert_mag_close(d_e0.cpu().numpy(), r["d_e0"], m["d_e0"], RTOL, "d_e0")
    assert_mag_close(d_pooled.cpu().numpy(), r["dZ"][:, 1:], m["dZ"][:, 1:], RTOL, "d_pooled")


@pytest.mark.parametrize("self_pairs", [False, True])
def test_interact_backward_exact_integers_and_no_d_e0(self_pairs):
    e0, pooled = _inputs(20, 9, 32, seed=11, integer=True)
    P = orc.pair_count(10, self_pairs)
    d_out = np.random.default_rng(3).integers(-2, 3, size=(20, 32 + P)).astype(np.float32)
    r = orc.interact_bwd(e0, pooled, d_out, self_pairs=self_pairs)
    d_e0, d_pooled = ops.interact_bwd(torch.from_numpy(e0).cuda(), torch.from_numpy(pooled).cuda(),
                                      torch.from_numpy(d_out).cuda(), self_pairs=self_pairs)
    np.testing.assert_array_equal(d_e0.cpu().numpy(), r["d_e0"].astype(np.float32))
    np.testing.assert_array_equal(d_pooled.cpu().numpy(), r["dZ"][:, 1:].astype(np.float32))
    _, d_pooled2 = ops.interact_bwd(torch.from_numpy(e0).cuda(), torch.from_numpy(pooled).cuda(),
                                    torch.from_numpy(d_out).cuda(), self_pairs=self_pairs, want_d_e0=False)
    assert torch.equal(d_pooled, d_pooled2)


def test_interact_rejects_bad_arguments():
    e0 = torch.zeros((2, 8), device="cuda")
    pooled = torch.zeros((2, 3, 8), device="cuda")
    out = torch.zeros((2, 8 + 10), device="cuda")
    L = ops.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert L.dlrm_interact_ex(3, 2, 8, 4, p(e0), p(pooled), p(out), None) == -1  # layout bits 0..3 only
    assert L.dlrm_interact_ex(3, 2, 8, -1, p(e0), p(pooled), p(out), None) == -1
    assert L.dlrm_interact_bwd(3, 2, 8, 0, p(e0), p(pooled), p(out), None, None, None) == -1  # d_pooled required
    assert L.dlrm_interact_bwd(3, 2, 6, 0, p(e0), p(pooled), p(out), None, p(pooled), None) == -2  # D % 4


@pytest.mark.parametrize("self_pairs", [False, True])
@pytest.mark.parametrize("B,T,D", [(1, 1, 4), (7, 3, 16), (64, 26, 128), (9, 64, 64)])
def test_interact_with_embeddings_forward_and_backward(self_pairs, B, T, D):
    """Layout with the embeddings concatenated alongside the dots: the Z rows come out as bit
    copies, the dots as in the plain layout, and the backward adds each row's own gradient."""
    e0, pooled = _inputs(B, T, D, seed=B * 31 + T + D + self_pairs)
    de, dp = torch.from_numpy(e0).cuda(), torch.from_numpy(pooled).cuda()
    out = ops.interact(de, dp, self_pairs=self_pairs, with_embeddings=True)
    plain = ops.interact(de, dp, self_pairs=self_pairs)
    torch.cuda.synchronize()
    F = T + 1
    got = out.cpu().numpy()
    ref = orc.interact(e0, pooled, self_pairs=self_pairs, with_embeddings=True)
    assert got.shape == ref.shape
    np.testing.assert_array_equal(got[:, :F * D], ref[:, :F * D].astype(np.float32))
    assert torch.equal(out[:, F * D:], plain[:, D:])
    mag = orc.interact(np.abs(e0), np.abs(pooled), self_pairs=self_pairs, with_embeddings=True)
    assert_mag_close(got[:, F * D:], ref[:, F * D:], mag[:, F * D:], RTOL, "dots")
    d_out = np.random.default_rng(B + T).standard_normal((B, ref.shape[1])).astype(np.float32)
    d_e0, d_pooled = ops.interact_bwd(de, dp, torch.from_numpy(d_out).cuda(), self_pairs=self_pairs,
                                      with_embeddings=True)
    torch.cuda.synchronize()
    r = orc.interact_bwd(e0, pooled, d_out, self_pairs=self_pairs, with_embeddings=True)
    m = orc.interact_bwd(np.abs(e0), np.abs(pooled), np.abs(d_out), self_pairs=self_pairs, with_embeddings=True)
    assert_mag_close(d_e0.cpu().numpy(), r["d_e0"], m["d_e0"], RTOL, "d_e0")
    assert_mag_close(d_pooled.cpu().numpy(), r["d_pooled"], m["d_pooled"], RTOL, "d_pooled")


@pytest.mark.parametrize("self_pairs", [False, True])
def test_interact_with_embeddings_exact_integers(self_pairs):
    e0, pooled = _inputs(30, 10, 32, seed=13, integer=True)
    de, dp = torch.from_numpy(e0).cuda(), torch.from_numpy(pooled).cuda()
    out = ops.interact(de, dp, self_pairs=self_pairs, with_embeddings=True)
    ref = orc.interact(e0, pooled, self_pairs=self_pairs, with_embeddings=True)
    np.testing.assert_array_equal(out.cpu().numpy(), ref.astype(np.float32))
    d_out = np.random.default_rng(4).integers(-2, 3, size=ref.shape).astype(np.float32)
    r = orc.interact_bwd(e0, pooled, d_out, self_pairs=self_pairs, with_embeddings=True)
    d_e0, d_pooled = ops.interact_bwd(de, dp, torch.from_numpy(d_out).cuda(), self_pairs=self_pairs,
                                      with_embeddings=True)
    np.testing.assert_array_equal(d_e0.cpu().numpy(), r["d_e0"].astype(np.float32))
    np.testing.assert_array_equal(d_pooled.cpu().numpy(), r["d_pooled"].astype(np.float32))
