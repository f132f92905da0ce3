"""Shared helpers of the GPU parity tests: build a quantized cache on the GPU
from seeded bf16 sources, build the oracle's copy from the same sources on the
CPU, and compare to the stated tolerances.

Every expected value here comes from ``oracle`` on inputs from ``kvq_synth``;
nothing the GPU computes is fed back to the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import kvq_synth as syn
import oracle
import quantized_kv_cache_group_amd as kvq

ATOL = 2e-3     # max-abs on attention outputs
RTOL_L2 = 1e-3  # relative L2 on attention outputs


def close(got, want, atol=ATOL, rl2=RTOL_L2, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(got - want) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    assert mx <= atol, f"{what}: max-abs {mx:.3e} > {atol}"
    assert rel <= rl2, f"{what}: rel-L2 {rel:.3e} > {rl2}"
    return mx, rel


def to_dev_bf16(bits_u16: np.ndarray, dev="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16))
    return t.to(dev).view(torch.bfloat16)


@dataclass
class Built:
    cache: kvq.LayerCache
    k_src: list            # per seq bf16 bits [L][H][D]
    v_src: list | None
    rope: list | None      # per seq bf16 bits [L][H][R]
    ref_pool: np.ndarray   # oracle pool: K blocks then V blocks
    k_off: np.ndarray      # [A][max_blocks] offsets into ref_pool
    v_off: np.ndarray | None

    def seq(self, a):
        c = self.cache
        nb, nw = c.n_blocks_host[a], c.n_window_host[a]
        kw = self.k_src[a][64 * nb:64 * nb + nw] if nw else None
        vw = self.v_src[a][64 * nb:64 * nb + nw] if (nw and self.v_src is not None) else None
        return dict(bits=c.bits_host[a, :nb], koff=self.k_off[a, :nb],
                    voff=None if self.v_off is None else self.v_off[a, :nb], kw=kw, vw=vw,
                    rope=None if self.rope is None else self.rope[a])


def build(H, D, lengths, bits=None, window=None, latent=False, rope_dim=0, k_src=None,
          v_src=None, rope=None, seed=0, keep_recent=0, quantize_on_gpu=True, fused=False) -> Built:
    """lengths: tokens per sequence.  Full blocks are quantized, keeping at
    least ``keep_recent`` newest tokens (or ``window[a]`` tokens) in bf16."""
    A = len(lengths)
    if window is None:
        window = [L - 64 * (max(L - keep_recent, 0) // 64) for L in lengths]
    n_blocks = [(L - w) // 64 for L, w in zip(lengths, window)]
    assert all(64 * b + w == L for b, w, L in zip(n_blocks, window, lengths))
    if bits is None:
        bits = [np.full(b, 4, np.uint8) for b in n_blocks]
    if k_src is None:
        k_src = [syn.random_normal_bf16((L, H, D), seed * 1000 + 2 * a) for a, L in enumerate(lengths)]
    if v_src is None and not latent:
        v_src = [syn.random_normal_bf16((L, H, D), seed * 1000 + 2 * a + 1) for a, L in enumerate(lengths)]
    if rope_dim and rope is None:
        rope = [syn.random_normal_bf16((L, H, rope_dim), seed * 1000 + 500 + a) for a, L in enumerate(lengths)]
    cache = kvq.LayerCache(H, D, n_blocks, window, bits, latent=latent, rope_dim=rope_dim)

    # Oracle copy, offsets from the oracle's own block size.
    maxb = cache.max_blocks
    k_off = np.zeros((A, max(maxb, 1)), np.uint64)
    pos = 0
    for a in range(A):
        for j in range(n_blocks[a]):
            k_off[a, j] = pos
            pos += (oracle.block_bytes(int(bits[a][j]), H, D) + 255) // 256 * 256
    assert np.array_equal(k_off[:, :maxb], cache.offset_host[:, :maxb]), "layout offsets differ"
    ktot = max(pos, 256)
    v_off = None if latent else k_off + np.uint64(ktot)
    ref_pool = np.zeros(ktot * (1 if latent else 2), np.uint8)
    for a in range(A):
        nb = n_blocks[a]
        oracle.quantize_seq(k_src[a], H, D, bits[a], k_off[a, :nb], ref_pool)
        if not latent:
            oracle.quantize_seq(v_src[a], H, D, bits[a], v_off[a, :nb], ref_pool)

    # GPU copy: quantize the same sources, copy windows and rope as storage.
    S = max(64 * maxb, 64)
    if quantize_on_gpu:
        dev = {}
        for which, src in (("k", k_src), ("v", v_src)):
            if src is None:
                continue
            buf = np.zeros((A, S, H, D), np.uint16)
            for a in range(A):
                nq = 64 * n_blocks[a]
                buf[a, :nq] = src[a][:nq]
            dev[which] = to_dev_bf16(buf)
        if fused:
            cache.quantize_kv(dev["k"], dev.get("v"))
        else:
            for which, t in dev.items():
                cache.quantize(which, t)
    for which, src in (("k", k_src), ("v", v_src)):
        if src is None:
            continue
        win = cache.k_window if which == "k" else cache.v_window
        for a in range(A):
            nq, w = 64 * n_blocks[a], window[a]
            if w:
                win[a, :w] = to_dev_bf16(src[a][nq:nq + w])
    if rope_dim:
        for a in range(A):
            cache.rope[a, :lengths[a]] = to_dev_bf16(rope[a])
    torch.cuda.synchronize()
    return Built(cache, k_src, v_src, rope, ref_pool, k_off, v_off)


def gpu_pool_matches(b: Built):
    """Block payloads of the GPU pools equal the oracle's byte for byte."""
    kp = b.cache.k_pool.cpu().numpy()
    ktot = kp.size
    assert np.array_equal(kp, b.ref_pool[:ktot][:kp.size]), "K pool differs"
    if b.cache.v_pool is not None:
        vp = b.cache.v_pool.cpu().numpy()
        assert np.array_equal(vp, b.ref_pool[b.ref_pool.size // 2:][:vp.size]), "V pool differs"


def ref_decode(b: Built, q_bits: np.ndarray, scale: float, seqs=None):
    """Oracle decode for each sequence: q_bits [A][Hq][Dk] -> [A][Hq][D]."""
    c = b.cache
    out = np.zeros((c.A, q_bits.shape[1], c.D), np.float32)
    for a in (range(c.A) if seqs is None else seqs):
        s = b.seq(a)
        out[a] = oracle.attend_decode_seq(b.ref_pool, s["bits"], s["koff"], s["voff"], s["kw"],
                                          s["vw"], s["rope"], c.H, c.D, q_bits[a], scale)
    return out
