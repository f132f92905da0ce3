"""Pins of the oracle's attention over a restored cache.

The pages fix the semantics: the receiving agent rebuilds 16-bit key/value
rows from the quantized cache and runs ordinary attention (QKVShare,
Metodologia, injection path).  So the oracle's attention must equal softmax
attention over its own dequantized rows.  Pinned here by closed forms and
invariants that a dropped term, a wrong sign, a wrong GQA index, a missing
window token or a transposed operand would break, and by a brute-force fp64
evaluation written with numpy's exp and matmul on tiny shapes.
"""
import numpy as np
import pytest

import kvq_synth as syn


def _q(shape, seed, scale=1.0):
    return syn.random_normal_bf16(shape, seed, scale)


def _f(h):
    return syn.bf16_to_f32(h).astype(np.float64)


def _cache(ref, T_blocks, H, D, bits=4, seed=0, scale=1.0, window=0):
    """Quantized cache of one sequence; returns pieces + restored fp32 rows."""
    bits_arr = np.full(T_blocks, bits, np.uint8) if np.isscalar(bits) else np.asarray(bits, np.uint8)
    koff, tot = ref.packed_offsets(bits_arr, H, D)
    voff = koff + np.uint64(tot)
    pool = np.zeros(2 * tot, np.uint8)
    k = syn.random_normal_bf16((T_blocks * 64, H, D), seed, scale)
    v = syn.random_normal_bf16((T_blocks * 64, H, D), seed + 1, scale)
    ref.quantize_seq(k, H, D, bits_arr, koff, pool)
    ref.quantize_seq(v, H, D, bits_arr, voff, pool)
    kw = syn.random_normal_bf16((window, H, D), seed + 2, scale) if window else None
    vw = syn.random_normal_bf16((window, H, D), seed + 3, scale) if window else None
    K = ref.restore_seq(pool, bits_arr, koff, kw, H, D)
    V = ref.restore_seq(pool, bits_arr, voff, vw, H, D)
    return dict(pool=pool, bits=bits_arr, koff=koff, voff=voff, kw=kw, vw=vw, K=K, V=V)


def _brute(K, V, q, scale):
    """numpy fp64 softmax attention, query head h on KV head h // G."""
    T, H, _ = K.shape
    Hq = q.shape[0]
    G = Hq // H
    out = np.zeros((Hq, V.shape[2]))
    for h in range(Hq):
        s = scale * (K[:, h // G, :].astype(np.float64) @ _f(q[h]))
        p = np.exp(s - s.max())
        out[h] = (p[:, None] * V[:, h // G, :].astype(np.float64)).sum(0) / p.sum()
    return out


def test_single_token_returns_its_value(ref):
    H, D = 2, 64
    K = syn.bf16_to_f32(syn.random_normal_bf16((1, H, D), 1)).reshape(1, H, D)
    V = syn.bf16_to_f32(syn.random_normal_bf16((1, H, D), 2)).reshape(1, H, D)
    q = _q((8, D), 3)
    out = ref.attention(K, V, q, 0.125)
    for h in range(8):
        assert np.array_equal(out[h], V[0, h // 4])


def test_equal_keys_give_mean_value(ref):
    T, H, D = 37, 1, 64
    K = np.repeat(syn.bf16_to_f32(syn.random_normal_bf16((1, H, D), 1)).reshape(1, H, D), T, 0)
    V = syn.bf16_to_f32(syn.random_normal_bf16((T, H, D), 2)).reshape(T, H, D)
    out = ref.attention(K, V, _q((2, D), 3), 0.3)
    want = V.astype(np.float64).mean(0)[0]
    assert np.allclose(out[0], want, rtol=0, atol=1e-6)
    assert np.allclose(out[1], want, rtol=0, atol=1e-6)


def test_two_token_closed_form(ref):
    H, D = 1, 64
    rng = np.random.default_rng(4)
    for _ in range(20):
        K = syn.bf16_to_f32(syn.random_normal_bf16((2, H, D), int(rng.integers(1 << 30)))).reshape(2, H, D)
        V = syn.bf16_to_f32(syn.random_normal_bf16((2, H, D), int(rng.integers(1 << 30)))).reshape(2, H, D)
        q = _q((1, D), int(rng.integers(1 << 30)))
        scale = float(rng.uniform(0.05, 0.5))
        qd = _f(q[0])
        delta = scale * (K[1, 0].astype(np.float64) @ qd - K[0, 0].astype(np.float64) @ qd)
        w1 = 1.0 / (1.0 + np.exp(-delta))
        want = (1 - w1) * V[0, 0] + w1 * V[1, 0]
        out = ref.attention(K, V, q, scale)
        assert np.allclose(out[0], want, rtol=1e-6, atol=1e-7)


def test_dominant_key_and_large_scores(ref):
    """A key aligned with the query and huge scores: no overflow (the row
    maximum is subtracted) and the output is that key's value."""
    T, H, D = 50, 1, 64
    K = np.zeros((T, H, D), np.float32)
    V = syn.bf16_to_f32(syn.random_normal_bf16((T, H, D), 9)).reshape(T, H, D)
    q = syn.bf16_bits(np.full((1, D), 100.0, np.float32))
    K[17, 0, :] = 100.0
    K[3, 0, :] = 99.0
    out = ref.attention(K, V, q, 1.0)
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0], V[17, 0], atol=1e-6)


def test_permutation_invariance(ref):
    T, H, D = 70, 2, 64
    K = syn.bf16_to_f32(syn.random_normal_bf16((T, H, D), 1)).reshape(T, H, D)
    V = syn.bf16_to_f32(syn.random_normal_bf16((T, H, D), 2)).reshape(T, H, D)
    q = _q((4, D), 3)
    perm = np.random.default_rng(0).permutation(T)
    a = ref.attention(K, V, q, 0.2)
    b = ref.attention(K[perm], V[perm], q, 0.2)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)


def test_gqa_head_mapping(ref):
    """Query head h reads KV head h // G: make each KV head's keys point at a
    different token and check every query head follows its own group."""
    T, H, D, Hq = 16, 4, 64, 8
    K = np.zeros((T, H, D), np.float32)
    V = np.zeros((T, H, D), np.float32)
    for g in range(H):
        K[3 * g + 1, g, :] = 1.0
        V[:, g, :] = np.arange(T, dtype=np.float32)[:, None]
    q = syn.bf16_bits(np.full((Hq, D), 1.0, np.float32))
    out = ref.attention(K, V, q, 10.0)
    for h in range(Hq):
        assert np.allclose(out[h], 3 * (h // 2) + 1, atol=1e-3)


def test_brute_force_tiny(ref):
    """Decode over a quantized cache (blocks and window) against numpy fp64
    softmax over the same restored rows, on the tiny workload shape."""
    for nb, win in [(4, 0), (1, 0), (0, 1), (0, 63), (1, 1), (2, 44)]:
        H, D, Hq = 2, 64, 8
        c = _cache(ref, nb, H, D, seed=nb * 10 + win, window=win)
        q = _q((Hq, D), 5)
        out = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], c["voff"], c["kw"], c["vw"],
                                    None, H, D, q, 0.125)
        want = _brute(c["K"], c["V"], q, 0.125)
        assert np.allclose(out, want, rtol=1e-6, atol=1e-7), (nb, win)


def test_decode_empty_cache_is_zero(ref):
    H, D = 1, 64
    bits = np.zeros(0, np.uint8)
    off = np.zeros(0, np.uint64)
    pool = np.zeros(256, np.uint8)
    out = ref.attend_decode_seq(pool, bits, off, off, None, None, None, H, D, _q((2, D), 1), 0.1)
    assert np.all(out == 0)


def test_decode_mixed_widths_equals_restore_then_attend(ref):
    H, D, Hq = 2, 256, 4
    bits = np.array([2, 3, 4, 8, 3], np.uint8)
    c = _cache(ref, 5, H, D, bits=bits, seed=3, window=130)
    q = _q((Hq, D), 6)
    out = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], c["voff"], c["kw"], c["vw"],
                                None, H, D, q, 1 / 16)
    assert np.allclose(out, _brute(c["K"], c["V"], q, 1 / 16), rtol=1e-6, atol=1e-7)


def test_latent_values_alias_keys(ref):
    """Latent attention with no rope part equals GQA with one KV head whose
    values are the same restored rows as the keys."""
    H, D, Hq = 1, 512, 16
    c = _cache(ref, 2, H, D, seed=8)
    q = _q((Hq, D), 7)
    mla = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], None, None, None, None, H, D, q,
                                576 ** -0.5)
    gqa = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], c["koff"], None, None, None, H, D,
                                q, 576 ** -0.5)
    assert np.array_equal(mla, gqa)
    assert np.allclose(mla, _brute(c["K"], c["K"], q, 576 ** -0.5), rtol=1e-6, atol=1e-7)


def test_rope_part_adds_to_scores(ref):
    """Rope dims extend the keys: equal rope rows shift every score by the
    same amount (output unchanged); distinct rope rows enter the dot product."""
    H, D, R, Hq = 1, 512, 64, 16
    c = _cache(ref, 2, H, D, seed=11)
    T = 128
    q = _q((Hq, D + R), 12)
    rope_same = np.repeat(syn.random_normal_bf16((1, H, R), 13), T, 0)
    a = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], None, None, None, rope_same, H, D, q,
                              0.05)
    b = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], None, None, None, None, H, D,
                              q[:, :D].copy(), 0.05)
    assert np.allclose(a, b, rtol=1e-5, atol=1e-6)
    rope = syn.random_normal_bf16((T, H, R), 14)
    out = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], None, None, None, rope, H, D, q, 0.05)
    Kfull = np.concatenate([c["K"], syn.bf16_to_f32(rope).reshape(T, H, R)], axis=2)
    assert np.allclose(out, _brute(Kfull, c["K"], q, 0.05), rtol=1e-6, atol=1e-7)


def test_chunk_single_token_equals_decode(ref):
    """A one-token chunk equals decode over the cache with that token appended
    to the bf16 window."""
    H, D, Hq = 2, 64, 8
    c = _cache(ref, 3, H, D, seed=21, window=10)
    qn = _q((1, Hq, D), 22)
    kn = syn.random_normal_bf16((1, H, D), 23)
    vn = syn.random_normal_bf16((1, H, D), 24)
    ch = ref.attend_chunk_seq(c["pool"], c["bits"], c["koff"], c["voff"], c["kw"], c["vw"], H, D,
                              qn, kn, vn, 0.125)
    kw = np.concatenate([c["kw"], kn])
    vw = np.concatenate([c["vw"], vn])
    dec = ref.attend_decode_seq(c["pool"], c["bits"], c["koff"], c["voff"], kw, vw, None, H, D,
                                qn[0], 0.125)
    assert np.array_equal(ch[0], dec)


def test_chunk_causal_and_brute(ref):
    H, D, Hq, n = 2, 64, 4, 9
    c = _cache(ref, 2, H, D, seed=31)
    qn = _q((n, Hq, D), 32)
    kn = syn.random_normal_bf16((n, H, D), 33)
    vn = syn.random_normal_bf16((n, H, D), 34)
    out = ref.attend_chunk_seq(c["pool"], c["bits"], c["koff"], c["voff"], None, None, H, D,
                               qn, kn, vn, 0.125)
    Kn = syn.bf16_to_f32(kn).reshape(n, H, D)
    Vn = syn.bf16_to_f32(vn).reshape(n, H, D)
    for i in range(n):
        K = np.concatenate([c["K"], Kn[: i + 1]])
        V = np.concatenate([c["V"], Vn[: i + 1]])
        assert np.allclose(out[i], _brute(K, V, qn[i], 0.125), rtol=1e-6, atol=1e-7)
    # future tokens do not leak into earlier rows
    kn2 = kn.copy()
    kn2[5:] = syn.random_normal_bf16((n - 5, H, D), 99)
    out2 = ref.attend_chunk_seq(c["pool"], c["bits"], c["koff"], c["voff"], None, None, H, D,
                                qn, kn2, vn, 0.125)
    assert np.array_equal(out[:5], out2[:5])
    assert not np.array_equal(out[5:], out2[5:])
    # a row range computes the same rows
    part = ref.attend_chunk_seq(c["pool"], c["bits"], c["koff"], c["voff"], None, None, H, D,
                                qn, kn, vn, 0.125, 3, 6)
    assert np.array_equal(part[3:6], out[3:6])
