"""GPU parity of the window roll (kvq_append) against the oracle: counts,
block payloads, window rows and rope rows bit-exact after every call, for
ragged initial states, mixed widths, call sizes from 0 to several blocks, a
latent cache with rope, and a cache without a window; then decode over the
rolled cache against the oracle's decode of the oracle's own state."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
import quantized_kv_cache_group_amd as kvq
from parity import close, to_dev_bf16

pytestmark = pytest.mark.gpu


class Twin:
    """The same caches on the GPU (LayerCache) and in oracle host arrays."""

    def __init__(self, H, D, nb0, nw0, max_blocks, cap, seed, latent=False, rope_dim=0):
        A = len(nb0)
        rng = np.random.default_rng(seed)
        widths = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=max_blocks) for _ in range(A)]
        self.H, self.D, self.A, self.cap, self.latent, self.R = H, D, A, cap, latent, rope_dim
        self.c = kvq.LayerCache(H, D, nb0, nw0, [w[:n] for w, n in zip(widths, nb0)], max_blocks=max_blocks,
                                window_cap=cap, latent=latent, rope_dim=rope_dim,
                                future_bits=[w[n:] for w, n in zip(widths, nb0)])
        self.widths = widths
        self.seqs = []
        T0 = [64 * n + w for n, w in zip(nb0, nw0)]
        k0 = [syn.random_normal_bf16((T, H, D), seed * 100 + a) for a, T in enumerate(T0)]
        v0 = None if latent else [syn.random_normal_bf16((T, H, D), seed * 100 + 50 + a) for a, T in enumerate(T0)]
        r0 = [syn.random_normal_bf16((T, H, rope_dim), seed * 100 + 80 + a) for a, T in enumerate(T0)] if rope_dim else None
        # GPU: quantize the initial blocks, copy the windows and rope rows
        S = max(64 * max_blocks, 64)
        for which, src in (("k", k0), ("v", v0)):
            if src is None:
                continue
            buf = np.zeros((A, S, H, D), np.uint16)
            for a in range(A):
                buf[a, :64 * nb0[a]] = src[a][:64 * nb0[a]]
            self.c.quantize(which, to_dev_bf16(buf))
            win = self.c.k_window if which == "k" else self.c.v_window
            for a in range(A):
                if nw0[a]:
                    win[a, :nw0[a]] = to_dev_bf16(src[a][64 * nb0[a]:])
        if rope_dim:
            for a in range(A):
                if T0[a]:
                    self.c.rope[a, :T0[a]] = to_dev_bf16(r0[a])
        # oracle: the same state in host arrays
        for a in range(A):
            koff, tot = oracle.packed_offsets(widths[a], H, D)
            s = dict(koff=koff, voff=None if latent else koff.copy(), kp=np.zeros(max(tot, 256), np.uint8),
                     vp=None if latent else np.zeros(max(tot, 256), np.uint8),
                     kw=np.zeros((max(cap, 1), H, D), np.uint16),
                     vw=None if latent else np.zeros((max(cap, 1), H, D), np.uint16),
                     rope=np.zeros((64 * max_blocks + cap, H, rope_dim), np.uint16) if rope_dim else None,
                     nb=nb0[a], nw=nw0[a])
            oracle.quantize_seq(k0[a], H, D, widths[a][:nb0[a]], koff[:nb0[a]], s["kp"])
            if not latent:
                oracle.quantize_seq(v0[a], H, D, widths[a][:nb0[a]], koff[:nb0[a]], s["vp"])
            if nw0[a]:
                s["kw"][:nw0[a]] = k0[a][64 * nb0[a]:]
                if not latent:
                    s["vw"][:nw0[a]] = v0[a][64 * nb0[a]:]
            if rope_dim:
                s["rope"][:T0[a]] = r0[a]
            self.seqs.append(s)
        torch.cuda.synchronize()

    def append(self, n, keep, seed, in_place=False):
        A, H, D = self.A, self.H, self.D
        kn = syn.random_normal_bf16((A, n, H, D), seed)
        vn = None if self.latent else syn.random_normal_bf16((A, n, H, D), seed + 1)
        rn = syn.random_normal_bf16((A, n, H, self.R), seed + 2) if self.R else None
        self.c.append(to_dev_bf16(kn), None if vn is None else to_dev_bf16(vn), keep,
                      None if rn is None else to_dev_bf16(rn), in_place=in_place)
        for a, s in enumerate(self.seqs):
            s["nb"], s["nw"] = oracle.append_seq(s["kp"], s["vp"], self.widths[a], s["koff"], s["voff"], s["nb"],
                                                 s["kw"] if self.cap else None,
                                                 s["vw"] if self.cap else None, s["nw"], H, D, kn[a],
                                                 None if vn is None else vn[a], keep, s["rope"],
                                                 None if rn is None else rn[a])
        torch.cuda.synchronize()

    def check(self, what):
        c = self.c
        nb = c.n_blocks.cpu().numpy()
        nw = c.n_window.cpu().numpy()
        assert list(nb) == [s["nb"] for s in self.seqs], f"{what}: n_blocks"
        assert list(nb) == c.n_blocks_host, f"{what}: host mirror of n_blocks"
        if self.cap:
            assert list(nw) == [s["nw"] for s in self.seqs], f"{what}: n_window"
            assert list(nw) == c.n_window_host, f"{what}: host mirror of n_window"
        kp = c.k_pool.cpu().numpy()
        vp = None if self.latent else c.v_pool.cpu().numpy()
        kw = c.k_window.cpu().view(torch.int16).numpy().view(np.uint16)
        vw = None if self.latent else c.v_window.cpu().view(torch.int16).numpy().view(np.uint16)
        for a, s in enumerate(self.seqs):
            for j in range(s["nb"]):
                n = oracle.block_bytes(int(self.widths[a][j]), self.H, self.D)
                g0, r0 = int(c.offset_host[a, j]), int(s["koff"][j])
                assert np.array_equal(kp[g0:g0 + n], s["kp"][r0:r0 + n]), f"{what}: K block {a},{j}"
                if vp is not None:
                    assert np.array_equal(vp[g0:g0 + n], s["vp"][r0:r0 + n]), f"{what}: V block {a},{j}"
            w = s["nw"]
            if self.cap:
                assert np.array_equal(kw[a, :w], s["kw"][:w]), f"{what}: K window {a}"
                if vw is not None:
                    assert np.array_equal(vw[a, :w], s["vw"][:w]), f"{what}: V window {a}"
            if self.R:
                rp = c.rope[a].cpu().view(torch.int16).numpy().view(np.uint16)
                T = 64 * s["nb"] + w
                assert np.array_equal(rp[:T], s["rope"][:T]), f"{what}: rope rows {a}"

    def ref_decode(self, q, scale):
        out = np.zeros((self.A, q.shape[1], self.D), np.float32)
        for a, s in enumerate(self.seqs):
            nb, nw = s["nb"], s["nw"]
            rope = s["rope"][:64 * nb + nw] if self.R else None
            pool = s["kp"] if self.latent else np.concatenate([s["kp"], s["vp"]])
            voff = None if self.latent else s["voff"][:nb] + np.uint64(s["kp"].size)
            out[a] = oracle.attend_decode_seq(pool, self.widths[a][:nb], s["koff"][:nb], voff,
                                              s["kw"][:nw] if nw else None,
                                              None if (self.latent or not nw) else s["vw"][:nw], rope,
                                              self.H, self.D, q[a], scale)
        return out


@pytest.mark.parametrize("D,in_place", [(64, False), (128, False), (256, False), (128, True)])
def test_append_rolls_match_oracle(D, in_place):
    """Counts written to the other count buffer by the window launch, or
    (in_place) over the counts the kernels read, by a launch of their own."""
    H = 2
    t = Twin(H, D, nb0=[0, 2, 1], nw0=[0, 100, 191], max_blocks=14, cap=191, seed=D)
    t.check("initial")
    for i, n in enumerate([1, 63, 64, 65, 0, 200, 1, 130]):
        t.append(n, 128, seed=1000 + 10 * i, in_place=in_place)
        t.check(f"D={D} call {i} (n_new={n})")
    q = syn.random_normal_bf16((3, 4 * H, D), 77)
    got = t.c.attend_decode(to_dev_bf16(q), D ** -0.5)
    torch.cuda.synchronize()
    close(got.cpu().numpy(), t.ref_decode(q, D ** -0.5), what=f"decode after rolls D={D}")


def test_append_latent_rope_matches_oracle():
    t = Twin(1, 512, nb0=[3, 0], nw0=[150, 20], max_blocks=12, cap=191, seed=5, latent=True, rope_dim=64)
    t.check("initial")
    for i, n in enumerate([1, 41, 64, 300]):
        t.append(n, 128, seed=2000 + 10 * i, in_place=(i == 2))
        t.check(f"latent call {i}")
    q = syn.random_normal_bf16((2, 16, 576), 78)
    got = t.c.attend_decode(to_dev_bf16(q), 576 ** -0.5)
    torch.cuda.synchronize()
    close(got.cpu().numpy(), t.ref_decode(q, 576 ** -0.5), what="latent decode after rolls")


def test_append_without_window():
    t = Twin(4, 128, nb0=[1, 0], nw0=[0, 0], max_blocks=6, cap=0, seed=9)
    for i, n in enumerate([64, 128, 0, 64]):
        t.append(n, 0, seed=3000 + 10 * i, in_place=(i % 2 == 1))
        t.check(f"no-window call {i}")


def test_append_keep_zero_and_small_keep():
    t = Twin(2, 64, nb0=[0, 0, 0], nw0=[0, 10, 63], max_blocks=8, cap=70, seed=11)
    for i, n in enumerate([1, 54, 1, 128]):
        t.append(n, 7, seed=4000 + 10 * i)
        t.check(f"keep=7 call {i}")


def test_append_window_move_cases():
    """Every way the window can move, each checked against the oracle: old
    rows moved to the front with no overlap (64k < W, 64k >= W2: chunks in
    parallel), overlapping moves (ordered rounds), new rows only (k == 0),
    and a window made entirely of new rows (64k >= W)."""
    t = Twin(2, 128, nb0=[0, 1, 0], nw0=[150, 140, 40], max_blocks=12, cap=200, seed=13)
    t.check("initial")
    # (keep, n_new) per call; the comments give sequence 0's (W, k, W2)
    calls = [(0, 10),      # W=150, T=160: k=2, 64k=128 < W, W2=32 <= 128: disjoint move of old rows
             (0, 5),       # W=32, T=37: k=0: new rows appended in place
             (20, 150),    # W=37, T=187: k=2, 64k=128 >= W: new rows only
             (100, 120),   # W=59, T=179: k=1, 64k=64 >= W
             (137, 90),    # W=115, T=205: k=1, 64k=64 < W, W2=141 > 64: overlapping, ordered rounds
             (137, 30)]    # W=141, T=171: k=0 (keep + 63 <= window_cap bounds keep)
    for i, (keep, n) in enumerate(calls):
        t.append(n, keep, seed=5000 + 10 * i)
        t.check(f"move case {i} (keep={keep}, n_new={n})")
