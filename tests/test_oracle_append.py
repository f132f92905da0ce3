"""Pins of the oracle's window roll (quantize on append).

The roll is defined by the token stream alone: whatever the chunking of the
appended tokens, the final cache must be the one obtained by cutting the
whole stream at once, i.e. quantizing its first 64k tokens as blocks
(kvq_ref_quantize_seq, itself pinned in test_oracle_quantize.py) and keeping
the rest as the window.  These tests check that, the counts, the keep-recent
rule, latent + rope caches, and the refusal of results that do not fit.
"""
import numpy as np
import pytest

import kvq_synth as syn
import oracle


class Seq:
    """One sequence's storage in host arrays (oracle layout)."""

    def __init__(self, H, D, bits, cap, latent=False, rope_dim=0):
        self.H, self.D, self.cap = H, D, cap
        self.bits = np.asarray(bits, np.uint8)
        self.koff, tot = oracle.packed_offsets(self.bits, H, D)
        self.voff = None if latent else self.koff.copy()
        self.kp = np.zeros(max(tot, 256), np.uint8)
        self.vp = None if latent else np.zeros(max(tot, 256), np.uint8)
        self.kw = np.zeros((cap, H, D), np.uint16)
        self.vw = None if latent else np.zeros((cap, H, D), np.uint16)
        self.rope = None
        if rope_dim:
            self.rope = np.zeros((64 * self.bits.size + cap, H, rope_dim), np.uint16)
        self.nb, self.nw = 0, 0

    def append(self, k, v, keep, rope_new=None):
        self.nb, self.nw = oracle.append_seq(self.kp, self.vp, self.bits, self.koff, self.voff, self.nb,
                                             self.kw, self.vw, self.nw, self.H, self.D, k, v, keep,
                                             self.rope, rope_new)


def _stream(T, H, D, seed):
    return syn.random_normal_bf16((T, H, D), seed)


@pytest.mark.parametrize("T,keep", [(300, 128), (191, 128), (192, 128), (64, 0), (1000, 128), (50, 128)])
def test_append_all_at_once_cuts_the_stream(T, keep):
    H, D = 2, 128
    rng = np.random.default_rng(T)
    bits = rng.choice(np.array([2, 3, 4, 8], np.uint8), size=20)
    x, y = _stream(T, H, D, 1), _stream(T, H, D, 2)
    s = Seq(H, D, bits, cap=keep + 63 if keep else 63)
    s.append(x, y, keep)
    k = (T - keep) // 64 if T > keep else 0
    assert (s.nb, s.nw) == (k, T - 64 * k)
    if k:
        assert keep <= s.nw <= keep + 63
    # blocks: the oracle's sequence quantizer on the stream's first 64k tokens
    want_k = np.zeros_like(s.kp)
    want_v = np.zeros_like(s.vp)
    oracle.quantize_seq(x, H, D, bits[:k], s.koff[:k], want_k)
    oracle.quantize_seq(y, H, D, bits[:k], s.koff[:k], want_v)
    assert np.array_equal(s.kp, want_k) and np.array_equal(s.vp, want_v)
    assert np.array_equal(s.kw[:s.nw], x[64 * k:]) and np.array_equal(s.vw[:s.nw], y[64 * k:])


@pytest.mark.parametrize("chunks", [[1] * 300, [5, 64, 1, 63, 100, 67], [200, 0, 1, 129], [64] * 5])
def test_append_chunking_does_not_matter(chunks):
    H, D, keep = 2, 64, 128
    T = sum(chunks)
    bits = np.array([4, 3, 2, 8, 4, 3, 2, 8], np.uint8)
    x, y = _stream(T, H, D, 3), _stream(T, H, D, 4)
    one = Seq(H, D, bits, cap=191)
    one.append(x, y, keep)
    inc = Seq(H, D, bits, cap=191)
    t = 0
    for c in chunks:
        inc.append(x[t:t + c], y[t:t + c], keep)
        t += c
        assert 64 * inc.nb + inc.nw == t                    # no token lost or duplicated
        assert inc.nw <= 191
    assert (inc.nb, inc.nw) == (one.nb, one.nw)
    assert np.array_equal(inc.kp, one.kp) and np.array_equal(inc.vp, one.vp)
    assert np.array_equal(inc.kw[:inc.nw], one.kw[:one.nw])
    assert np.array_equal(inc.vw[:inc.nw], one.vw[:one.nw])


def test_append_restores_to_the_stream():
    """Restoring after rolls gives the stream rows back: exact for the
    window, within the pinned reconstruction bound for the blocks."""
    H, D, keep = 1, 64, 128
    T = 777
    x = _stream(T, H, D, 5)
    s = Seq(H, D, np.full(12, 8, np.uint8), cap=191)
    for c in (100, 300, 1, 376):
        t0 = 64 * s.nb + s.nw
        s.append(x[t0:t0 + c], x[t0:t0 + c], keep)
    r = oracle.restore_seq(s.kp, s.bits[:s.nb], s.koff[:s.nb], s.kw[:s.nw], H, D)
    assert r.shape[0] == T
    xf = syn.bf16_to_f32(x)
    assert np.array_equal(r[64 * s.nb:], xf[64 * s.nb:])
    assert np.max(np.abs(r[:64 * s.nb] - xf[:64 * s.nb])) < 0.05     # 8-bit codes of N(0,1) rows


def test_append_latent_with_rope():
    H, D, R, keep = 1, 512, 64, 128
    T = 400
    x = _stream(T, H, D, 6)
    rp = syn.random_normal_bf16((T, H, R), 7)
    s = Seq(H, D, np.full(6, 4, np.uint8), cap=191, latent=True, rope_dim=R)
    for c in (150, 150, 100):
        t0 = 64 * s.nb + s.nw
        s.append(x[t0:t0 + c], None, keep, rope_new=rp[t0:t0 + c])
    k = (T - keep) // 64
    assert (s.nb, s.nw) == (k, T - 64 * k)
    assert np.array_equal(s.rope[:T], rp)            # one row per token position, none moved
    assert not s.rope[T:].any()
    want = np.zeros_like(s.kp)
    oracle.quantize_seq(x, H, D, s.bits[:k], s.koff[:k], want)
    assert np.array_equal(s.kp, want)


def test_append_refuses_what_does_not_fit():
    H, D = 1, 64
    s = Seq(H, D, np.full(2, 4, np.uint8), cap=191)
    x = _stream(400, H, D, 8)
    before = s.kp.copy()
    with pytest.raises(ValueError):
        s.append(x, x, 128)                                 # needs 4 blocks, 2 exist
    assert np.array_equal(s.kp, before) and (s.nb, s.nw) == (0, 0)
    t = Seq(H, D, np.full(4, 4, np.uint8), cap=100)
    with pytest.raises(ValueError):
        t.append(x[:150], x[:150], 128)                     # window of 150 > 100


def test_append_nothing_is_identity():
    H, D = 2, 64
    s = Seq(H, D, np.full(3, 3, np.uint8), cap=191)
    x = _stream(150, H, D, 9)
    s.append(x, x, 128)
    kp, kw, st = s.kp.copy(), s.kw.copy(), (s.nb, s.nw)
    s.append(x[:0], x[:0], 128)
    assert (s.nb, s.nw) == st and np.array_equal(s.kp, kp) and np.array_equal(s.kw, kw)
