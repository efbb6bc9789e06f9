"""Host-side checks of the seeded input generators (no GPU)."""
import numpy as np
import pytest
import torch

from sparse_embedding_lookup_dlrm_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 0.01,
                        np.array([1.0, -0.0, 0.0, 3.0e38, 1.00390625, 1.01171875], np.float32)])
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_workloads_are_deterministic_and_shaped():
    w = synth.WORKLOADS["tiny-4t1k-d16-b128"]
    a = synth.make_batch(w)
    b = synth.make_batch(w)
    np.testing.assert_array_equal(a.indices, b.indices)
    np.testing.assert_array_equal(a.tables[2], b.tables[2])
    assert a.lengths.shape == (w.T * w.B,) and np.all(a.lengths == 1)
    assert a.indices.dtype == np.int32 and a.indices.min() >= 0 and a.indices.max() < 1000
    assert a.e0.shape == (128, 16) and a.e0.dtype == np.float32
    assert w.P == 10 and w.out_width == 26


def test_loguniform_rows_and_zipf_head():
    w = synth.WORKLOADS["zipf-26t-d128-b2048"]
    rows = synth.table_rows(w)
    assert len(rows) == 26 and min(rows) >= 1000 and max(rows) <= 1_000_000
    lengths = synth.gen_lengths(w)
    idx = synth.gen_indices(w, rows, lengths)
    assert len(idx) == 26 * 2048
    # Row 0 is the hottest: its frequency is close to 1 / H(n, alpha).
    t0 = idx[:2048]
    n = rows[0]
    h = (np.arange(1, n + 1, dtype=np.float64) ** -1.05).sum()
    p0 = 1.0 / h
    assert abs((t0 == 0).mean() - p0) < 5 * np.sqrt(p0 * (1 - p0) / 2048) + 1e-3
    assert t0.max() < n


def test_multihot_lengths_and_capacity_lengths():
    w = synth.WORKLOADS["multihot-8t4m-d64-fp16-b4096"].replace(B=512)
    L = synth.gen_lengths(w)
    assert L.min() >= 0 and L.max() <= 100 and abs(L.mean() - 20) < 1.0
    c = synth.WORKLOADS[synth.CAPACITY].replace(B=256)
    L = synth.gen_lengths(c)
    assert L.min() >= 1 and L.max() <= 32 and abs(L.mean() - 16.5) < 0.5


def test_zipf_sampler_law_small_support():
    rng = np.random.default_rng(9)
    s = synth.sample_zipf(rng, 5, 1.1, 200000)
    w = np.arange(1, 6, dtype=np.float64) ** -1.1
    np.testing.assert_allclose(np.bincount(s, minlength=5) / 200000, w / w.sum(), atol=4e-3)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_host_table_dtypes(dtype):
    w = synth.Workload("t", T=2, rows=10, D=8, dtype=dtype, B=4, bag=("fixed", 1), dist=("uniform",), seed=3)
    tabs = synth.gen_tables_host(w)
    want = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    assert all(t.dtype == want and t.shape == (10, 8) for t in tabs)


def test_quantize_table_q8_round_trip_within_half_step():
    """Table-wise codes reproduce every value within half a step (scale / 2), use the
    full code range, and give a constant table scale 1 and exact values."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((200, 16)) * 0.05).astype(np.float32)
    codes, sb = synth.quantize_table_q8(x)
    back = codes.astype(np.float64) * float(sb[0]) + float(sb[1])
    assert np.max(np.abs(back - x.astype(np.float64))) <= 0.5 * float(sb[0]) * (1 + 1e-5)
    assert codes.min() == 0 and codes.max() == 255
    c1, sb1 = synth.quantize_table_q8(np.full((3, 4), 0.75, np.float32))
    assert sb1.tolist() == [1.0, 0.75] and not c1.any()


def test_quantize_rows_q4_round_trip_and_packing():
    """Row-wise 4-bit codes reconstruct each row within half a step, and the stored form
    puts column 2k in the low 4 bits of byte k with the scale and bias right after."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((20, 128)) * 0.01).astype(np.float32)
    codes, sb = synth.quantize_rows_q4(x)
    assert codes.max() <= 15
    rec = codes.astype(np.float64) * sb[:, :1] + sb[:, 1:]
    assert np.all(np.abs(rec - x) <= 0.5 * sb[:, :1] * (1 + 1e-5) + 1e-9)
    stored = synth.pack_q4_rows(codes, sb)
    assert stored.shape == (20, 128) and synth.q4_row_stride(128) == 128
    assert synth.q4_row_stride(256) == 256 and synth.q4_row_stride(512) == 512
    np.testing.assert_array_equal(stored[:, :64] & 0xF, codes[:, 0::2])
    np.testing.assert_array_equal(stored[:, :64] >> 4, codes[:, 1::2])
    np.testing.assert_array_equal(stored[:, 64:72].copy().view(np.float32), sb)
    assert not stored[:, 72:].any()
