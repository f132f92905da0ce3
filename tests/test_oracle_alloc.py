"""Pins of the width allocator's two parts (Coordinated Mixed-Precision KV
Cache Quantization, arXiv 2611.10096, Abstract: sensitivity from a local
attention-error bound, then a budgeted choice of widths).

The sensitivity bound must cover the measured error of attention restricted
to the block after quantizing it at each width, and its first-order part
c(b) S must approach the bound as b grows; the greedy allocation must stay
within one step's gain of the brute-force optimum, use its budget
monotonically and order widths by sensitivity."""
import itertools

import numpy as np
import pytest

import kvq_synth as syn
import oracle


def _block(H, D, seed, outliers=0):
    k = syn.bf16_to_f32(syn.random_normal_bf16((64, H, D), seed)).copy()
    if outliers:
        k[:, :, np.random.default_rng(seed).choice(D, outliers, replace=False)] *= 8.0
    return syn.bf16_bits(k), syn.random_normal_bf16((64, H, D), seed + 1)


def _local_attention(K, V, q, scale):
    z = scale * K @ q
    p = np.exp(z - z.max())
    p /= p.sum()
    return p @ V


@pytest.mark.parametrize("seed,outliers", [(1, 0), (2, 4), (3, 2)])
def test_bound_covers_measured_error(seed, outliers):
    H, D, Hq = 2, 128, 8
    k, v = _block(H, D, seed, outliers)
    q = syn.random_normal_bf16((Hq, D), seed + 10)
    scale = D ** -0.5
    kf, vf, qf = (syn.bf16_to_f32(x).astype(np.float64) for x in (k, v, q))
    for b in (2, 3, 4, 8):
        bits = np.array([b], np.uint8)
        off, tot = oracle.packed_offsets(bits, H, D)
        pk, pv = np.zeros(tot, np.uint8), np.zeros(tot, np.uint8)
        oracle.quantize_seq(k, H, D, bits, off, pk)
        oracle.quantize_seq(v, H, D, bits, off, pv)
        kr = oracle.restore_seq(pk, bits, off, None, H, D).astype(np.float64)
        vr = oracle.restore_seq(pv, bits, off, None, H, D).astype(np.float64)
        for h in range(Hq):
            g = h // (Hq // H)
            err = np.linalg.norm(_local_attention(kr[:, g], vr[:, g], qf[h], scale) -
                                 _local_attention(kf[:, g], vf[:, g], qf[h], scale))
            bound = oracle.block_error_bound(k, v, H, D, q, h, scale, b)
            # the reconstruction bound's fp16-scale slack (2^-10 relative) on top
            assert err <= bound * (1 + 2.0 ** -9) + 1e-9, (b, h, err, bound)


def test_first_order_part_is_the_bounds_coefficient():
    H, D, Hq = 2, 64, 4
    k, v = _block(H, D, 7, outliers=3)
    q = syn.random_normal_bf16((Hq, D), 17)
    scale = 0.125
    S = oracle.block_sensitivity(k, v, H, D, q, scale)
    # S is the coefficient of c(b) in the bound as c(b) -> 0 (a 20-bit factor,
    # evaluated only as mathematics: the codes themselves stop at 8 bits)
    exact = sum(oracle.block_error_bound(k, v, H, D, q, h, scale, 20) for h in range(Hq))
    assert abs(oracle.width_cost(20) * S - exact) <= 1e-3 * exact
    # and the exact bound is convex in the error factor: first order underestimates it
    for b in (2, 3, 4):
        assert oracle.width_cost(b) * S <= sum(oracle.block_error_bound(k, v, H, D, q, h, scale, b)
                                               for h in range(Hq)) + 1e-12


def _bytes(b, H=8, D=128):
    return H * D * (8 * b + 4)


def _error(S, w):
    return sum(s * oracle.width_cost(b) for s, b in zip(S, w))


@pytest.mark.parametrize("seed", range(6))
def test_greedy_near_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 4
    S = rng.lognormal(0, 1.5, size=n)
    lo, hi = n * _bytes(2), n * _bytes(8)
    for frac in (0.1, 0.3, 0.5, 0.8):
        budget = lo + frac * (hi - lo)
        w = oracle.allocate_widths(S, _bytes, budget)
        assert sum(_bytes(int(b)) for b in w) <= budget
        best = min(_error(S, c) for c in itertools.product(oracle.WIDTHS, repeat=n)
                   if sum(_bytes(b) for b in c) <= budget)
        step = max(s * (oracle.width_cost(a) - oracle.width_cost(b)) for s in S
                   for a, b in zip(oracle.WIDTHS, oracle.WIDTHS[1:]))
        assert best - 1e-12 <= _error(S, w) <= best + step


def test_budget_extremes_and_monotone():
    rng = np.random.default_rng(9)
    S = rng.lognormal(0, 1, size=30)
    lo, hi = 30 * _bytes(2), 30 * _bytes(8)
    assert np.all(oracle.allocate_widths(S, _bytes, lo) == 2)
    assert np.all(oracle.allocate_widths(S, _bytes, hi) == 8)
    with pytest.raises(ValueError):
        oracle.allocate_widths(S, _bytes, lo - 1)
    prev = None
    for frac in np.linspace(0, 1, 11):
        e = _error(S, oracle.allocate_widths(S, _bytes, lo + frac * (hi - lo)))
        assert prev is None or e <= prev + 1e-12
        prev = e


def test_widths_follow_sensitivity():
    S = np.array([0.1, 5.0, 1.0, 5.0, 0.01, 2.0])
    for frac in (0.2, 0.5, 0.7):
        lo, hi = S.size * _bytes(2), S.size * _bytes(8)
        w = oracle.allocate_widths(S, _bytes, lo + frac * (hi - lo))
        for i in range(S.size):
            for j in range(S.size):
                if S[i] > S[j]:
                    assert w[i] >= w[j]
