"""Shared helpers for the GPU parity tests: moving seeded batches to the device,
and magnitude-relative comparisons.

Tolerances: a float result is compared as |got - ref| <= rtol * M, where M is
the same expression evaluated on absolute values (for a dot: sum_d |z_i||z_j|;
for a pooled sum: sum_p |w_p|), computed by the oracle on |inputs|. Plain
|ref|-relative checks fail under cancellation even for exact-rounding fp32
arithmetic. rtol is 1e-5 for fp32 tables and 2e-3 for fp16/bf16 tables.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import dlrm_oracle as orc
from sparse_embedding_lookup_dlrm_amd import ops, synth

RTOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()  # raises if the HIP library is missing: no fallback


def dev_tables(tables, dtype, device="cuda"):
    out = []
    for t in tables:
        if dtype == "bf16":
            out.append(torch.from_numpy(t.view(np.int16)).to(device).view(torch.bfloat16))
        else:
            out.append(torch.from_numpy(t).to(device))
    return out


def host_tables(dtables, dtype):
    """Device tables -> host storage form (float32 / float16 / uint16 bits)."""
    if dtype == "bf16":
        return [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in dtables]
    return [t.cpu().numpy() for t in dtables]


def abs_tables(tables, dtype):
    if dtype == "bf16":
        return [t & np.uint16(0x7FFF) for t in tables]
    return [np.abs(t) for t in tables]


def assert_mag_close(got, ref, mag, rtol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    lim = rtol * mag
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} mag {mag[tuple(i)]!r} rtol {rtol}")


class DeviceBatch:
    """A seeded batch on the device: tables, lengths -> offsets (by the library), indices, e0."""

    def __init__(self, b: synth.Batch, device="cuda"):
        self.b = b
        w = b.w
        self.tables = dev_tables(b.tables, w.dtype, device)
        self.lengths = torch.from_numpy(b.lengths).to(device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.offsets = ops.lengths_to_offsets(self.lengths, status=self.status)
        self.indices = torch.from_numpy(b.indices).to(device)
        self.e0 = torch.from_numpy(b.e0).to(device)

    def fwd(self, **kw):
        return ops.embbag_fwd(self.tables, self.offsets, self.indices, self.b.w.B, self.e0, status=self.status, **kw)


def oracle_fwd(b: synth.Batch):
    w = b.w
    off = orc.lengths_to_offsets(b.lengths)
    r = orc.embbag_fwd(b.tables, w.dtype, w.B, off, b.indices, b.e0)
    at = abs_tables(b.tables, w.dtype)
    pooled_mag = orc.embbag_pool(at, w.dtype, w.B, off, b.indices)
    dots_mag = orc.interact(np.abs(b.e0), pooled_mag)
    return off, r, pooled_mag, dots_mag


def check_fwd(db: DeviceBatch, pooled, inter, exact=False):
    b = db.b
    w = b.w
    off, r, pooled_mag, dots_mag = oracle_fwd(b)
    np.testing.assert_array_equal(db.offsets.cpu().numpy(), off.astype(np.int32))
    rtol = 0.0 if exact else RTOL[w.dtype]
    if pooled is not None:
        assert_mag_close(pooled.cpu().numpy(), r["pooled"], pooled_mag, rtol, f"{w.name} pooled")
    if inter is not None:
        got = inter.cpu().numpy()
        np.testing.assert_array_equal(got[:, :w.D], b.e0)  # e0 block is a bit copy
        assert_mag_close(got[:, w.D:], r["out"][:, w.D:], dots_mag[:, w.D:], rtol, f"{w.name} dots")
    return r
