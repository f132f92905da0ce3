"""Pins of the oracle's top-K sparse decode pieces: block scores in closed
form, the top-K rule, that keeping every block is the full decode, and the
error bound of the discarded attention mass (Reasoning-Aware Error-Bounded
KV-Cache Compression and Sparse Attention for Long-Context LLMs, section
2B): for any kept set, |o - o'|_2 <= 2 V_max delta, delta the full
attention's mass on the dropped tokens, V_max the largest value norm."""
import numpy as np
import pytest

import kvq_synth as syn
import oracle


def _cache(H, D, nb, nw, seed, bits=None, scale_k=1.0):
    bits = np.full(nb, 4, np.uint8) if bits is None else np.asarray(bits, np.uint8)
    T = 64 * nb + nw
    k = syn.random_normal_bf16((T, H, D), seed, scale=scale_k)
    v = syn.random_normal_bf16((T, H, D), seed + 1)
    koff, tot = oracle.packed_offsets(bits, H, D)
    pool = np.zeros(2 * max(tot, 256), np.uint8)
    voff = koff + np.uint64(max(tot, 256))
    oracle.quantize_seq(k, H, D, bits, koff, pool)
    oracle.quantize_seq(v, H, D, bits, voff, pool)
    return dict(pool=pool, bits=bits, koff=koff, voff=voff, k=k, v=v, nb=nb, nw=nw, H=H, D=D)


def _sparse(c, sel, q, scale):
    nb, nw = c["nb"], c["nw"]
    kw = c["k"][64 * nb:] if nw else None
    vw = c["v"][64 * nb:] if nw else None
    return oracle.attend_decode_seq(c["pool"], c["bits"][sel], c["koff"][sel], c["voff"][sel], kw, vw, None,
                                    c["H"], c["D"], q, scale)


def test_block_scores_closed_form():
    """Keys on the quantization grid round-trip exactly; a query that is a
    unit vector on dim d scores a block by scale * max_t k_t[d]."""
    H, D, nb = 1, 64, 3
    rng = np.random.default_rng(0)
    k = np.zeros((64 * nb, H, D), np.float32)
    for t in range(64 * nb):
        codes = rng.integers(0, 16, size=D)
        codes[0], codes[1] = 0, 15                        # both endpoints: min/max fix the grid
        k[t, 0] = -1.0 + codes * 0.125                    # bias -1, scale 1/8: exact in bf16 and fp16
    kb = syn.bf16_bits(k)
    bits = np.full(nb, 4, np.uint8)
    koff, tot = oracle.packed_offsets(bits, H, D)
    pool = np.zeros(tot, np.uint8)
    oracle.quantize_seq(kb, H, D, bits, koff, pool)
    r = oracle.restore_seq(pool, bits, koff, None, H, D)
    assert np.array_equal(r, k)                           # the grid round-trips
    for d in (2, 17, 63):
        q = np.zeros((1, D), np.float32)
        q[0, d] = 1.0
        s = oracle.block_scores_seq(pool, bits, koff, None, H, D, syn.bf16_bits(q), 0.5)
        want = [0.5 * k[64 * j:64 * j + 64, 0, d].max() for j in range(nb)]
        assert np.array_equal(s, np.asarray(want, np.float64))
    # a negative query picks the block minimum instead
    q = np.zeros((1, D), np.float32)
    q[0, 5] = -2.0
    s = oracle.block_scores_seq(pool, bits, koff, None, H, D, syn.bf16_bits(q), 1.0)
    assert np.array_equal(s, [-2.0 * k[64 * j:64 * j + 64, 0, 5].min() for j in range(nb)])


def test_topk_rule_and_nesting():
    s = np.array([0.5, 2.0, 2.0, -1.0, 3.0, 0.5])
    assert list(oracle.topk_blocks(s, 1)) == [4]
    assert list(oracle.topk_blocks(s, 2)) == [1, 4]
    assert list(oracle.topk_blocks(s, 3)) == [1, 2, 4]
    assert list(oracle.topk_blocks(s, 4)) == [0, 1, 2, 4]          # tie 0.5: index 0 first
    assert list(oracle.topk_blocks(s, 10)) == [0, 1, 2, 3, 4, 5]
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50)
    prev = set()
    for k in range(1, 51):
        cur = set(oracle.topk_blocks(x, k))
        assert prev < cur and len(cur) == k
        prev = cur


def test_all_blocks_is_full_decode():
    c = _cache(2, 128, 6, 70, seed=3)
    q = syn.random_normal_bf16((8, 128), 4)
    full = oracle.attend_decode_seq(c["pool"], c["bits"], c["koff"], c["voff"], c["k"][64 * 6:], c["v"][64 * 6:],
                                    None, 2, 128, q, 0.1)
    assert np.array_equal(_sparse(c, np.arange(6), q, 0.1), full)


def test_planted_block_is_selected():
    H, D, nb = 2, 64, 8
    c = _cache(H, D, nb, 0, seed=5, scale_k=0.3)
    q = syn.random_normal_bf16((4 * H, D), 6)
    qf = syn.bf16_to_f32(q)
    k = syn.bf16_to_f32(c["k"]).copy()
    k[64 * 5 + 7, 0] = 4.0 * qf[0] / np.linalg.norm(qf[0])          # one token aligned with head 0
    c2 = _cache(H, D, nb, 0, seed=5, scale_k=0.3)
    kb = syn.bf16_bits(k)
    oracle.quantize_seq(kb, H, D, c2["bits"], c2["koff"], c2["pool"])
    s = oracle.block_scores_seq(c2["pool"], c2["bits"], c2["koff"], None, H, D, q, 0.125)
    assert list(oracle.topk_blocks(s, 1)) == [5]


@pytest.mark.parametrize("seed,K", [(7, 1), (8, 3), (9, 6), (10, 10)])
def test_discarded_mass_bound(seed, K):
    H, D, nb, nw = 2, 64, 12, 40
    c = _cache(H, D, nb, nw, seed, bits=np.random.default_rng(seed).choice([2, 3, 4, 8], size=nb))
    Hq, scale = 8, 64 ** -0.5
    q = syn.random_normal_bf16((Hq, D), seed + 100, scale=2.0)
    s = oracle.block_scores_seq(c["pool"], c["bits"], c["koff"], None, H, D, q, scale)
    sel = oracle.topk_blocks(s, K)
    full = oracle.attend_decode_seq(c["pool"], c["bits"], c["koff"], c["voff"], c["k"][64 * nb:], c["v"][64 * nb:],
                                    None, H, D, q, scale)
    sp = _sparse(c, sel, q, scale)
    # delta and V_max from the restored rows, in numpy fp64
    Kr = oracle.restore_seq(c["pool"], c["bits"], c["koff"], c["k"][64 * nb:], H, D).astype(np.float64)
    Vr = oracle.restore_seq(c["pool"], c["bits"], c["voff"], c["v"][64 * nb:], H, D).astype(np.float64)
    keep = np.zeros(64 * nb + nw, bool)
    for j in sel:
        keep[64 * j:64 * j + 64] = True
    keep[64 * nb:] = True
    qf = syn.bf16_to_f32(q).astype(np.float64)
    G = Hq // H
    for h in range(Hq):
        g = h // G
        z = scale * Kr[:, g] @ qf[h]
        p = np.exp(z - z.max())
        p /= p.sum()
        delta = p[~keep].sum()
        vmax = np.linalg.norm(Vr[:, g], axis=1).max()
        err = np.linalg.norm(full[h].astype(np.float64) - sp[h].astype(np.float64))
        assert err <= 2 * vmax * delta + 1e-5, (h, err, 2 * vmax * delta)
