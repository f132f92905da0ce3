"""Seeded sweep of decode, top-K and chunk shapes against the oracle (2e-3
max-abs, 1e-3 relative L2), through the C ABI: every path the planner picks
(the G <= 4 and G 5-16 decodes, the latent decode, the generic kernel for
other head_dims and for latent caches with several heads, both top-K scoring
kernels, the chunk kernels) over
random sequence counts, block counts (0 included), bf16 windows, mixed
widths and query scales.  Each case's draw is fixed by its index."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
from parity import build, close, ref_decode, to_dev_bf16

pytestmark = pytest.mark.gpu

WIDTHS = np.array([2, 3, 4, 8], np.uint8)


def _shape(rng, max_blocks, max_window):
    A = int(rng.integers(1, 6))
    nb = [int(v) for v in rng.integers(0, max_blocks + 1, size=A)]
    win = [int(v) for v in rng.integers(0, max_window + 1, size=A)]
    bits = [rng.choice(WIDTHS, size=n) for n in nb]
    return A, nb, win, bits


@pytest.mark.parametrize("case", range(40))
def test_sweep_decode(case):
    rng = np.random.default_rng(7000 + case)
    H = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    D = int(rng.choice([64, 128, 192, 256, 320]))
    A, nb, win, bits = _shape(rng, 12, 140)
    lengths = [64 * n + w for n, w in zip(nb, win)]
    b = build(H, D, lengths, bits=bits, window=win, seed=7100 + case)
    qs = float(rng.choice([0.5, 1.0, 3.0]))
    q = syn.random_normal_bf16((A, G * H, D), 7200 + case, scale=qs)
    scale = D ** -0.5
    out = b.cache.attend_decode(to_dev_bf16(q), scale)
    torch.cuda.synchronize()
    close(out.cpu().numpy(), ref_decode(b, q, scale), what=f"decode case {case}: H {H} G {G} D {D} nb {nb} win {win}")


@pytest.mark.parametrize("case", range(12))
def test_sweep_latent(case):
    rng = np.random.default_rng(7300 + case)
    H = 1 if case < 8 else 2                      # two latent heads: the generic kernel
    D = 512 if case < 8 else 128
    R = int(rng.choice([0, 64]))
    Hq = H * int(rng.integers(1, 17 if H == 1 else 5))
    A, nb, win, bits = _shape(rng, 20, 100)
    lengths = [64 * n + w for n, w in zip(nb, win)]
    b = build(H, D, lengths, bits=bits, window=win, latent=True, rope_dim=R, seed=7400 + case)
    q = syn.random_normal_bf16((A, Hq, D + R), 7500 + case, scale=2.0)
    scale = (D + R) ** -0.5
    out = b.cache.attend_decode(to_dev_bf16(q), scale)
    torch.cuda.synchronize()
    close(out.cpu().numpy(), ref_decode(b, q, scale), what=f"latent case {case}: H {H} Hq {Hq} D {D} R {R} nb {nb}")


@pytest.mark.parametrize("case", range(20))
def test_sweep_chunk(case):
    rng = np.random.default_rng(7600 + case)
    H = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128, 256]))
    n_new = int(rng.integers(1, 101))
    A, nb, win, bits = _shape(rng, 8, 100)
    A = min(A, 3)
    nb, win, bits = nb[:A], win[:A], bits[:A]
    lengths = [64 * n + w for n, w in zip(nb, win)]
    b = build(H, D, lengths, bits=bits, window=win, seed=7700 + case)
    qn = syn.random_normal_bf16((A, n_new, G * H, D), 7800 + case)
    kn = syn.random_normal_bf16((A, n_new, H, D), 7900 + case)
    vn = syn.random_normal_bf16((A, n_new, H, D), 8000 + case)
    scale = D ** -0.5
    out = b.cache.attend_chunk(to_dev_bf16(qn), to_dev_bf16(kn), to_dev_bf16(vn), scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    c = b.cache
    for a in range(A):
        s = b.seq(a)
        want = oracle.attend_chunk_seq(b.ref_pool, s["bits"], s["koff"], s["voff"], s["kw"], s["vw"],
                                       c.H, c.D, qn[a], kn[a], vn[a], scale, 0, n_new)
        close(got[a], want, what=f"chunk case {case} seq {a}: H {H} G {G} D {D} n_new {n_new} nb {nb} win {win}")


@pytest.mark.parametrize("case", range(12))
def test_sweep_topk(case):
    """Top-K over seeded shapes: a valid selection within the scores'
    rounding allowance, then the oracle's decode over exactly the kept set."""
    from test_gpu_topk import _check_selection, _ref_sparse, _run
    rng = np.random.default_rng(8100 + case)
    latent = case >= 9
    H = 1 if latent else int(rng.choice([1, 2, 4]))
    D = 512 if latent else int(rng.choice([64, 128, 256]))
    R = 64 if latent else 0
    G = int(rng.choice([2, 8, 16])) if latent else int(rng.choice([1, 2, 4, 8, 16]))
    A, nb, win, bits = _shape(rng, 40, 100)
    lengths = [64 * n + w for n, w in zip(nb, win)]
    b = build(H, D, lengths, bits=bits, window=win, latent=latent, rope_dim=R, seed=8200 + case)
    q = syn.random_normal_bf16((A, G * H, D + R), 8300 + case, scale=2.0)
    scale = (D + R) ** -0.5
    K = int(rng.integers(1, 24))
    got, sel = _run(b, q, scale, K)
    _check_selection(b, q, scale, K, sel)
    close(got, _ref_sparse(b, q, scale, sel), what=f"topk case {case}: H {H} G {G} D {D} K {K} nb {nb}")
