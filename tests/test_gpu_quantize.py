"""GPU parity of quantize and restore: bit-exact against the oracle on
codes, scales, biases and restored values, through the C ABI."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
from parity import build, gpu_pool_matches, to_dev_bf16

pytestmark = pytest.mark.gpu


def _hard_values(L, H, D, seed):
    """bf16 rows mixing the distributions that exercise every branch: normal,
    outlier channels, tiny values (fp16-subnormal steps), values near the fp16
    limit, constant groups and signed zeros."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((L, H, D)).astype(np.float32)
    kind = r.integers(0, 7, size=(L, H, D // 64))
    for t in range(L):
        for h in range(H):
            for g in range(D // 64):
                sl = x[t, h, g * 64:(g + 1) * 64]
                k = kind[t, h, g]
                if k == 1:
                    sl[r.integers(0, 64, 2)] *= 10.0
                elif k == 2:
                    sl *= np.float32(10.0 ** r.uniform(-9, -4))
                elif k == 3:
                    sl *= np.float32(r.uniform(1e3, 2e4))
                    sl[0] = np.float32(65280.0 * np.sign(sl[0] or 1.0))
                elif k == 4:
                    sl[:] = np.float32(r.standard_normal())
                elif k == 5:
                    sl[:] = 0.0
                    sl[r.integers(0, 64, 5)] = -0.0
                    sl[r.integers(0, 64, 1)] = 1.0
    return syn.bf16_bits(x)


@pytest.mark.parametrize("D,H", [(64, 2), (128, 8), (256, 4), (512, 1), (192, 3)])
def test_quantize_bit_exact_mixed_widths(D, H):
    rng = np.random.default_rng(D + H)
    lengths = [64 * 5, 64 * 3 + 17, 0, 64, 64 * 9]
    window = [0, 17, 0, 0, 0]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    k_src = [_hard_values(L, H, D, 10 * a + D) for a, L in enumerate(lengths)]
    v_src = [syn.random_normal_bf16((L, H, D), 99 + a) for a, L in enumerate(lengths)]
    b = build(H, D, lengths, bits=bits, window=window, k_src=k_src, v_src=v_src)
    gpu_pool_matches(b)


@pytest.mark.parametrize("D,H,latent", [(128, 8, False), (64, 2, False), (192, 3, False), (512, 1, True)])
def test_quantize_kv_one_launch_bit_exact(D, H, latent):
    """kvq_quantize_kv (K and V in one launch) against the oracle, with mixed
    widths, ragged and empty sequences."""
    rng = np.random.default_rng(7 * D + H)
    lengths = [64 * 7, 64 * 2 + 5, 0, 64 * 4, 64]
    window = [0, 5, 0, 0, 0]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    k_src = [_hard_values(L, H, D, 31 * a + D) for a, L in enumerate(lengths)]
    v_src = None if latent else [syn.random_normal_bf16((L, H, D), 7 + a) for a, L in enumerate(lengths)]
    b = build(H, D, lengths, bits=bits, window=window, latent=latent, k_src=k_src, v_src=v_src, fused=True)
    gpu_pool_matches(b)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_quantize_single_width_tiny(bits):
    w = syn.workload(0)
    k = w.kv(0, 0, syn.TAG_K)
    v = w.kv(0, 0, syn.TAG_V)
    b = build(2, 64, [256], bits=[np.full(4, bits, np.uint8)], k_src=[k], v_src=[v])
    gpu_pool_matches(b)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_restore_bit_exact(out_dtype):
    H, D = 4, 128
    rng = np.random.default_rng(5)
    lengths = [64 * 4 + 30, 64 * 2, 5]
    window = [30, 0, 5]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    k_src = [_hard_values(L, H, D, a) for a, L in enumerate(lengths)]
    b = build(H, D, lengths, bits=bits, window=window, k_src=k_src)
    c = b.cache
    S = 64 * c.max_blocks + c.window_cap
    sentinel = torch.full((c.A, S + 3, H, D), 7.0, dtype=out_dtype, device="cuda")
    c.dequantize("k", sentinel)
    got = sentinel.cpu()
    for a in range(c.A):
        s = b.seq(a)
        want = oracle.restore_seq(b.ref_pool, s["bits"], s["koff"], s["kw"], H, D)
        L = lengths[a]
        if out_dtype == torch.float32:
            g = got[a, :L].numpy()
            assert np.array_equal(g.view(np.uint32), want.view(np.uint32))
        else:
            g = got[a, :L].view(torch.int16).numpy().view(np.uint16)
            wb = oracle.f32_to_bf16_bits(want.ravel()).reshape(want.shape)
            assert np.array_equal(g, wb)
        # rows past the sequence are untouched
        assert torch.all(got[a, L:] == 7.0)


def test_quantize_llama_shape_full():
    """All 10 agents x 4096 tokens of the Llama-3.1-8B layer, K with outliers."""
    w = syn.workload(1)
    k_src = [w.kv(a, 0, syn.TAG_K) for a in range(w.n_agents)]
    v_src = [w.kv(a, 0, syn.TAG_V) for a in range(w.n_agents)]
    b = build(w.n_kv_heads, w.head_dim, w.lengths, k_src=k_src, v_src=v_src)
    gpu_pool_matches(b)


def test_quantize_mla_latent_full():
    """4 agents x 32768 tokens of a 512-dim latent (one KV head)."""
    w = syn.workload(4)
    k_src = [w.kv(a, 0, syn.TAG_K) for a in range(w.n_agents)]
    b = build(1, 512, w.lengths, k_src=k_src, latent=True)
    gpu_pool_matches(b)


def test_quantize_deterministic():
    H, D = 8, 128
    b = build(H, D, [64 * 16] * 3, seed=3)
    p1 = b.cache.k_pool.clone()
    buf = np.zeros((3, 64 * 16, H, D), np.uint16)
    for a in range(3):
        buf[a] = b.k_src[a]
    b.cache.quantize("k", to_dev_bf16(buf))
    torch.cuda.synchronize()
    assert torch.equal(p1, b.cache.k_pool)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_quantize_scale_sweep(bits):
    """Groups whose ranges sweep every binade from fp16-subnormal steps to
    the fp16 limit, with random offsets: scales, biases and codes bit-exact."""
    r = np.random.default_rng(1000 + bits)
    n_blocks, H, D = 48, 2, 128
    L = 64 * n_blocks
    x = r.standard_normal((L, H, D)).astype(np.float32)
    e = r.uniform(-30, 15, size=(L, H, D // 64, 1)).astype(np.float32)
    off = r.uniform(-1, 1, size=(L, H, D // 64, 1)).astype(np.float32)
    g = x.reshape(L, H, D // 64, 64)
    g = (g * np.exp2(e) + off * np.exp2(e + r.uniform(0, 4))).astype(np.float32)
    g = np.clip(g, -60000, 60000)
    k = syn.bf16_bits(g.reshape(L, H, D))
    b = build(H, D, [L], bits=[np.full(n_blocks, bits, np.uint8)], k_src=[k], v_src=[k])
    gpu_pool_matches(b)


def test_quantize_restore_past_grid_limit():
    """One sequence of 65 600 blocks (4.2M tokens, one 64-dim head): more
    blocks than one grid dimension holds, so quantize and restore stride over
    the blocks.  The whole pool is compared byte for byte; restored rows are
    compared on the first blocks and on every block past the 65 535th."""
    H, D, nblk = 1, 64, 65600
    rng = np.random.default_rng(65600)
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=nblk)]
    b = build(H, D, [64 * nblk], bits=bits, window=[0], latent=True, seed=11)
    gpu_pool_matches(b)
    c = b.cache
    out = torch.full((1, 64 * nblk, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    c.dequantize("k", out)
    s = b.seq(0)
    for j0, j1 in ((0, 8), (65530, nblk)):
        want = oracle.restore_seq(b.ref_pool, s["bits"][j0:j1], s["koff"][j0:j1], None, H, D)
        got = out[0, 64 * j0:64 * j1].cpu().view(torch.int16).numpy().view(np.uint16)
        wb = oracle.f32_to_bf16_bits(want.ravel()).reshape(want.shape)
        assert np.array_equal(got, wb), (j0, j1)


def test_restore_window_tiles_in_second_launch():
    """65 530 blocks plus a 600-token window: the restore's work items (blocks,
    then 64-token window tiles) number 65 540, so the last window tiles fall
    in the second launch.  Restored rows of the last blocks and of the whole
    window are compared with the oracle, in fp32 and bf16."""
    H, D, nblk, nw = 1, 64, 65530, 600
    rng = np.random.default_rng(65530)
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=nblk)]
    b = build(H, D, [64 * nblk + nw], bits=bits, window=[nw], latent=True, seed=12)
    c = b.cache
    s = b.seq(0)
    j0 = nblk - 3
    want = oracle.restore_seq(b.ref_pool, s["bits"][j0:], s["koff"][j0:], s["kw"], H, D)
    for dt in (torch.float32, torch.bfloat16):
        out = torch.full((1, 64 * nblk + c.window_cap, H, D), 7.0, dtype=dt, device="cuda")
        c.dequantize("k", out)
        tail = out[0, 64 * j0:64 * nblk + nw].cpu()
        if dt == torch.float32:
            assert np.array_equal(tail.numpy().view(np.uint32), want.view(np.uint32))
        else:
            wb = oracle.f32_to_bf16_bits(want.ravel()).reshape(want.shape)
            assert np.array_equal(tail.view(torch.int16).numpy().view(np.uint16), wb)
