"""The library's budgeted width allocator (host code, no GPU) against the
oracle's greedy: identical widths for identical sensitivities and budgets,
and its argument checks."""
import os

import numpy as np
import pytest

import oracle
import quantized_kv_cache_group_amd as kvq

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")


@pytest.mark.parametrize("H,D", [(8, 128), (8, 256), (1, 512)])
@pytest.mark.parametrize("seed", range(4))
def test_allocator_matches_oracle(H, D, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 120))
    S = rng.lognormal(0, 2, size=n).astype(np.float32)
    S[rng.integers(0, n, size=n // 5)] = S[0]                # equal sensitivities: ties by index
    bb = lambda b: kvq.block_bytes(b, H, D)
    lo, hi = n * bb(2), n * bb(8)
    for frac in (0.0, 0.05, 0.33, 0.5, 0.9, 1.0, 1.5):
        budget = int(lo + frac * (hi - lo))
        got = kvq.allocate_widths(S, H, D, budget)
        want = oracle.allocate_widths(S.astype(np.float64), bb, budget)
        assert np.array_equal(got, want), (n, frac)
        assert sum(bb(int(b)) for b in got) <= budget


def test_allocator_mean_three_bits():
    """A budget of the mean-3-bit size (the mixed-width workload's average)."""
    rng = np.random.default_rng(7)
    S = rng.lognormal(0, 1, size=1000).astype(np.float32)
    H, D = 8, 256
    w = kvq.allocate_widths(S, H, D, 1000 * kvq.block_bytes(3, H, D))
    assert set(np.unique(w)) <= {2, 3, 4, 8}
    assert sum(kvq.block_bytes(int(b), H, D) for b in w) <= 1000 * kvq.block_bytes(3, H, D)
    order = np.argsort(S)
    assert np.all(np.diff(w[order].astype(int)) >= 0)       # widths follow sensitivity


def test_allocator_rejects():
    S = np.ones(4, np.float32)
    with pytest.raises(kvq.KVQError):
        kvq.allocate_widths(S, 8, 128, 4 * kvq.block_bytes(2, 8, 128) - 1)
    with pytest.raises(kvq.KVQError):
        kvq.allocate_widths(np.array([1.0, np.nan], np.float32), 8, 128, 1 << 30)
    with pytest.raises(kvq.KVQError):
        kvq.allocate_widths(np.array([-1.0], np.float32), 8, 128, 1 << 30)
    with pytest.raises(kvq.KVQError):
        kvq.allocate_widths(S, 8, 96, 1 << 30)
    assert kvq.allocate_widths(np.zeros(0, np.float32), 8, 128, 0).size == 0
