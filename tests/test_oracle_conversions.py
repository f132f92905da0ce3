"""Pins of the oracle's IEEE conversions against independent library routines.

The oracle writes its fp16/bf16 conversions from the IEEE 754 format
definitions; numpy's float16 cast and torch's bfloat16 cast are independent
round-to-nearest-even implementations of the same definitions.
"""
import numpy as np
import pytest
import torch


def _f32_probe_set(rng):
    """Every binary16 value, every exact midpoint between neighbours, and the
    binary32 values one ulp either side of each midpoint, plus random bits."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)          # all finite non-negative halves
    v = h.astype(np.uint16).view(np.float16).astype(np.float32)
    nxt = np.append(v[1:], np.float32(65536.0))
    mid = ((v.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)  # exact
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    rnd = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    special = np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30, np.inf, -np.inf,
                        2.0 ** -24, 2.0 ** -25, 1.5 * 2 ** -25, 2.0 ** -26, 2.0 ** -14,
                        2.0 ** -14 - 2.0 ** -25, 1e-45, 3e-8], np.float32)
    allv = np.concatenate([v, mid, up, dn, rnd, special])
    return np.concatenate([allv, -allv])


def test_f32_to_f16_matches_numpy(ref):
    x = _f32_probe_set(np.random.default_rng(1))
    got = ref.f32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    fin = np.isfinite(x)
    assert np.array_equal(got[fin], want[fin])
    nan = np.isnan(x)
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f16_to_f32_exhaustive(ref):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = ref.f16_bits_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))


def test_f32_to_bf16_matches_torch(ref):
    rng = np.random.default_rng(2)
    x = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    # exact ties: low 16 bits 0x8000 with even and odd kept halves
    ties = (rng.integers(0, 2 ** 16, size=20000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x[np.isfinite(x)], ties[np.isfinite(ties)],
                        np.array([3.3895e38, 3.4028235e38, -0.0, 0.0], np.float32)])
    got = ref.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_bf16_to_f32_exhaustive(ref):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = np.array([ref.lib().kvq_ref_bf16_to_f32(int(v)) for v in h[::97]], np.float32)
    want = torch.from_numpy(h[::97].view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
