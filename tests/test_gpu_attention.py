"""GPU parity of decode and chunk attention against the oracle: within
2e-3 max-abs and 1e-3 relative L2 (fp32 outputs against fp64 attention over
the oracle's own restored rows), through the C ABI."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
from parity import build, close, gpu_pool_matches, ref_decode, to_dev_bf16

pytestmark = pytest.mark.gpu


def _decode(b, q_bits, scale):
    q = to_dev_bf16(q_bits)
    out = b.cache.attend_decode(q, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_decode_tiny_workload():
    w = syn.workload(0)
    k, v = w.kv(0, 0, syn.TAG_K), w.kv(0, 0, syn.TAG_V)
    b = build(w.n_kv_heads, w.head_dim, w.lengths, k_src=[k], v_src=[v])
    q = w.q(0)
    close(_decode(b, q, w.scale), ref_decode(b, q, w.scale), what="tiny")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_decode_gqa_groups(G):
    H, D = 2, 128
    lengths = [64 * 7 + 3, 64 * 2, 1000]
    b = build(H, D, lengths, keep_recent=40, seed=G)
    q = syn.random_normal_bf16((3, G * H, D), 11 + G)
    close(_decode(b, q, D ** -0.5), ref_decode(b, q, D ** -0.5), what=f"G={G}")


def test_decode_edge_lengths():
    """Empty sequence, one window token, exactly one block, block + 1."""
    H, D = 2, 64
    lengths = [0, 1, 64, 65, 63, 128]
    window = [0, 1, 0, 1, 63, 0]
    b = build(H, D, lengths, window=window, seed=4)
    q = syn.random_normal_bf16((6, 8, D), 12)
    got = _decode(b, q, 0.125)
    want = ref_decode(b, q, 0.125)
    assert np.all(got[0] == 0.0)
    close(got, want, what="edges")


def test_decode_more_sequences_than_a_wave():
    """70 sequences (the split plan scans them 64 at a time), many empty or
    window-only, windows of 0..200 tokens, mixed widths."""
    rng = np.random.default_rng(70)
    H, D, G, A = 2, 64, 2, 70
    nb = [int(v) for v in rng.integers(0, 12, size=A)]
    window = [int(v) for v in rng.integers(0, 201, size=A)]
    for a in range(0, A, 9):
        nb[a], window[a] = 0, 0
    lengths = [64 * n + w for n, w in zip(nb, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    b = build(H, D, lengths, bits=bits, window=window, seed=70)
    q = syn.random_normal_bf16((A, G * H, D), 17)
    got = _decode(b, q, 0.125)
    for a in range(0, A, 9):
        assert np.all(got[a] == 0.0)
    close(got, ref_decode(b, q, 0.125), what="70 sequences")


def test_decode_many_sequences_one_split_each():
    """300 sequences x 16 KV heads of 0..4 blocks with windows: more splits
    than resident workgroups, so the balanced split plan gives each sequence
    one block split and one window split; the plan's scans over sequences
    run in five chunks of 64."""
    rng = np.random.default_rng(300)
    H, D, G, A = 16, 64, 2, 300
    nb = [int(v) for v in rng.integers(0, 5, size=A)]
    window = [int(v) for v in rng.integers(1, 64, size=A)]
    lengths = [64 * n + w for n, w in zip(nb, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    b = build(H, D, lengths, bits=bits, window=window, seed=300)
    q = syn.random_normal_bf16((A, G * H, D), 19)
    close(_decode(b, q, 0.125), ref_decode(b, q, 0.125), what="300 sequences")


def test_decode_long_sequence_among_short():
    """One 1 200-block sequence among 30 of 0..3 blocks, one KV head: the
    balanced plan's splits are a few blocks long, at least ceil(1200 / 511)
    so that no row has more than 512 splits to merge."""
    rng = np.random.default_rng(1200)
    H, D, G = 1, 128, 4
    nb = [1200] + [int(v) for v in rng.integers(0, 4, size=30)]
    window = [17] + [int(v) for v in rng.integers(0, 80, size=30)]
    lengths = [64 * n + w for n, w in zip(nb, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    b = build(H, D, lengths, bits=bits, window=window, seed=1200)
    q = syn.random_normal_bf16((len(nb), G * H, D), 20)
    close(_decode(b, q, D ** -0.5), ref_decode(b, q, D ** -0.5), what="long among short")


def test_decode_long_window():
    """A 9 000-token bf16 window: more than 128 rounds of 64 tokens, so each
    window split takes 128 tokens."""
    H, D, G = 1, 128, 4
    lengths = [9000 + 64 * 3, 500]
    window = [9000, 500 - 64 * 7]
    b = build(H, D, lengths, window=window, seed=71)
    q = syn.random_normal_bf16((2, G * H, D), 18)
    close(_decode(b, q, D ** -0.5), ref_decode(b, q, D ** -0.5), what="long window")


@pytest.mark.parametrize("D", [64, 256, 512])
def test_decode_mixed_widths_window(D):
    rng = np.random.default_rng(D)
    H, G = 4, 2
    lengths = [int(v) for v in rng.integers(200, 2000, size=4)]
    window = [128 + (L % 64) for L in lengths]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n, p=[0.4, 0.4, 0.15, 0.05]) for n in nb]
    b = build(H, D, lengths, bits=bits, window=window, seed=D)
    q = syn.random_normal_bf16((4, G * H, D), 13)
    close(_decode(b, q, D ** -0.5), ref_decode(b, q, D ** -0.5), what=f"mixed D={D}")


def test_decode_latent_with_rope():
    H, D, R, Hq = 1, 512, 64, 16
    lengths = [64 * 20, 64 * 3 + 9]
    b = build(H, D, lengths, latent=True, rope_dim=R, keep_recent=0, window=[0, 9], seed=5)
    q = syn.random_normal_bf16((2, Hq, D + R), 14)
    s = 576 ** -0.5
    close(_decode(b, q, s), ref_decode(b, q, s), what="latent+rope")


def test_decode_llama_10_agents_full():
    w = syn.workload(1)
    k_src = [w.kv(a, 0, syn.TAG_K) for a in range(w.n_agents)]
    v_src = [w.kv(a, 0, syn.TAG_V) for a in range(w.n_agents)]
    b = build(w.n_kv_heads, w.head_dim, w.lengths, k_src=k_src, v_src=v_src)
    q = w.q(0)
    close(_decode(b, q, w.scale), ref_decode(b, q, w.scale), what="llama-10")


def test_decode_gemma_mixed_full_layer():
    """One sampled layer of the Gemma-3-12B mixed-width workload, all 8 agents."""
    w = syn.workload(2)
    layer = w.layers[0]
    k_src = [w.kv(a, layer, syn.TAG_K) for a in range(w.n_agents)]
    v_src = [w.kv(a, layer, syn.TAG_V) for a in range(w.n_agents)]
    bits = [w.bits(a, layer) for a in range(w.n_agents)]
    b = build(w.n_kv_heads, w.head_dim, w.lengths, bits=bits, window=w.n_window,
              k_src=k_src, v_src=v_src)
    gpu_pool_matches(b)
    q = w.q(layer)
    close(_decode(b, q, w.scale), ref_decode(b, q, w.scale), what="gemma-mixed")


def test_decode_mla_4_agents_full():
    w = syn.workload(4)
    k_src = [w.kv(a, 0, syn.TAG_K) for a in range(w.n_agents)]
    rope = [w.rope(a, 0) for a in range(w.n_agents)]
    b = build(1, 512, w.lengths, latent=True, rope_dim=64, k_src=k_src, rope=rope)
    q = w.q(0)
    close(_decode(b, q, w.scale), ref_decode(b, q, w.scale), what="mla")


def test_decode_deterministic():
    b = build(8, 128, [4096, 3000], keep_recent=128, seed=9)
    q = syn.random_normal_bf16((2, 32, 128), 15)
    a1 = _decode(b, q, 0.1)
    a2 = _decode(b, q, 0.1)
    assert np.array_equal(a1, a2)


# ---- chunk -------------------------------------------------------------------
def _chunk(b, qn, kn, vn, scale):
    out = b.cache.attend_chunk(to_dev_bf16(qn), to_dev_bf16(kn), to_dev_bf16(vn), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref_chunk(b, a, qn, kn, vn, scale, rows=None):
    s = b.seq(a)
    c = b.cache
    r0, r1 = (0, qn.shape[0]) if rows is None else rows
    return oracle.attend_chunk_seq(b.ref_pool, s["bits"], s["koff"], s["voff"], s["kw"], s["vw"],
                                   c.H, c.D, qn, kn, vn, scale, r0, r1)


@pytest.mark.parametrize("G,n_new", [(4, 37), (1, 5), (2, 64), (16, 3)])
def test_chunk_small(G, n_new):
    H, D = 2, 128
    lengths = [64 * 5 + 20, 64 * 2]
    b = build(H, D, lengths, window=[20, 0], seed=G)
    A = 2
    qn = syn.random_normal_bf16((A, n_new, G * H, D), 21)
    kn = syn.random_normal_bf16((A, n_new, H, D), 22)
    vn = syn.random_normal_bf16((A, n_new, H, D), 23)
    got = _chunk(b, qn, kn, vn, D ** -0.5)
    for a in range(A):
        want = _ref_chunk(b, a, qn[a], kn[a], vn[a], D ** -0.5)
        close(got[a], want, what=f"chunk a={a}")


def test_chunk_empty_cache():
    H, D = 1, 64
    b = build(H, D, [0], seed=1)
    qn = syn.random_normal_bf16((1, 9, 4, D), 31)
    kn = syn.random_normal_bf16((1, 9, H, D), 32)
    vn = syn.random_normal_bf16((1, 9, H, D), 33)
    got = _chunk(b, qn, kn, vn, 0.125)
    close(got[0], _ref_chunk(b, 0, qn[0], kn[0], vn[0], 0.125), what="chunk-empty")
    # the first new token sees only itself: output equals its value
    v0 = syn.bf16_to_f32(vn[0, 0, 0])
    assert np.allclose(got[0, 0], v0[None, :], atol=1e-6)


def test_chunk_one_token_equals_decode():
    H, D = 8, 128
    b = build(H, D, [64 * 10 + 5], window=[5], seed=2)
    qn = syn.random_normal_bf16((1, 1, 32, D), 41)
    kn = syn.random_normal_bf16((1, 1, H, D), 42)
    vn = syn.random_normal_bf16((1, 1, H, D), 43)
    got = _chunk(b, qn, kn, vn, D ** -0.5)
    close(got[0], _ref_chunk(b, 0, qn[0], kn[0], vn[0], D ** -0.5), what="chunk-1")


@pytest.mark.parametrize("D,G", [(64, 4), (256, 2), (128, 8)])
def test_chunk_mixed_widths_window(D, G):
    """Chunk over a cache with 2/3/4/8-bit blocks and a bf16 window, causal
    new tokens spanning several 64-key tiles and a ragged tail."""
    rng = np.random.default_rng(D + G)
    H = 2
    lengths = [64 * 7 + 45, 64 * 3 + 130]
    window = [45, 130]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    b = build(H, D, lengths, bits=bits, window=window, seed=D)
    A, n_new = 2, 150
    qn = syn.random_normal_bf16((A, n_new, G * H, D), 51)
    kn = syn.random_normal_bf16((A, n_new, H, D), 52)
    vn = syn.random_normal_bf16((A, n_new, H, D), 53)
    got = _chunk(b, qn, kn, vn, D ** -0.5)
    for a in range(A):
        close(got[a], _ref_chunk(b, a, qn[a], kn[a], vn[a], D ** -0.5), what=f"chunk D={D} a={a}")


def test_decode_workspace_reuse():
    """One workspace serves several decode and top-K calls in a row (the top-K
    call's selection tables sit after the decode's partials): every decode
    gives the same output as the first."""
    H, D, G = 8, 128, 4
    lengths = [64 * 30 + 50, 64 * 9, 300]
    b = build(H, D, lengths, keep_recent=60, seed=33)
    c = b.cache
    q = to_dev_bf16(syn.random_normal_bf16((3, G * H, D), 34))
    nb = max(c.topk_workspace_bytes(G * H, 4), c.decode_workspace_bytes(G * H))
    ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
    first = c.attend_decode(q, D ** -0.5, workspace=ws).cpu().numpy()
    for i in range(3):
        c.attend_decode_topk(q, D ** -0.5, 4, workspace=ws)
        again = c.attend_decode(q, D ** -0.5, workspace=ws).cpu().numpy()
        assert np.array_equal(first, again)
    close(first, ref_decode(b, syn.random_normal_bf16((3, G * H, D), 34), D ** -0.5), what="reuse")
