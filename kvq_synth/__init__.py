"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.

This module holds none of the quantization or attention arithmetic: it only
draws random numbers and rounds them to bfloat16, so that the CPU oracle and
the HIP library receive bit-identical inputs.

Recipe (the pages' workloads, as synthetic stand-ins; no dataset is used):
  * every random stream is numpy's Philox counter-based generator, keyed by
    (1000 + workload id, tag, agent, layer) through numpy's SeedSequence;
  * values are drawn fp32 N(0,1), outlier key channels are multiplied in fp32,
    and the result is rounded to bf16 (nearest, ties to even);
  * tags: K=1, V=2, Q=3, K_new=4, V_new=5, outlier channels=6, lengths=7,
    widths=8, layer pick=9, rope=10.

Shapes follow the model geometries named by the pages (Llama-3.1-8B and
Gemma-3-12B grouped-query attention, DeepSeek-V2-Lite latent attention;
Agent Memory Below the Prompt, arXiv 2603.04428, Abstract) and their context
range (1K-32K tokens, up to 10 agents).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TAG_K, TAG_V, TAG_Q, TAG_KNEW, TAG_VNEW, TAG_OUTLIER, TAG_LEN, TAG_BITS, TAG_LAYER, TAG_ROPE = range(1, 11)


def rng(workload: int, tag: int, agent: int = 0, layer: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([1000 + int(workload), int(tag), int(agent), int(layer)])
    return np.random.Generator(np.random.Philox(key=ss.generate_state(2, np.uint64)))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, workload: int, tag: int, agent: int = 0, layer: int = 0,
                outlier_channels=None, outlier_gain: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0,1) fp32 draws of ``shape`` (last two axes [H][D] when
    outliers are requested: channel indices per head are multiplied by gain)."""
    x = rng(workload, tag, agent, layer).standard_normal(size=shape, dtype=np.float32)
    if outlier_channels is not None:
        g = np.float32(outlier_gain)
        for h, chans in enumerate(outlier_channels):
            x[..., h, chans] *= g
    return bf16_bits(x)


def outlier_channels(workload: int, n_heads: int, head_dim: int, count: int, layer: int = 0):
    """Distinct channel indices per KV head, drawn uniformly from [0, D)."""
    r = rng(workload, TAG_OUTLIER, 0, layer)
    return [np.sort(r.choice(head_dim, size=count, replace=False)) for _ in range(n_heads)]


def uniform_bf16(shape, lo: float, hi: float, seed: int) -> np.ndarray:
    x = np.random.Generator(np.random.Philox(key=[seed, 77])).uniform(lo, hi, size=shape)
    return bf16_bits(x.astype(np.float32))


def random_normal_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    x = np.random.Generator(np.random.Philox(key=[seed, 5])).standard_normal(size=shape,
                                                                             dtype=np.float32)
    return bf16_bits(x * np.float32(scale))


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------
@dataclass
class Workload:
    wid: int
    name: str
    n_agents: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    lengths: list            # cached tokens per agent
    n_blocks: list           # quantized 64-token blocks per agent
    n_window: list           # bf16 tail tokens per agent
    layers: list = field(default_factory=lambda: [0])
    rope_dim: int = 0
    n_new: int = 0           # chunk queries
    outliers: int = 0        # outlier K channels per KV head
    outlier_gain: float = 1.0
    scale: float = 0.0       # softmax scale

    def bits(self, agent: int, layer: int) -> np.ndarray:
        """Per-block widths of one (agent, layer)."""
        nb = self.n_blocks[agent]
        if self.wid != 2:
            return np.full(nb, 4, np.uint8)
        r = rng(self.wid, TAG_BITS, agent, layer)
        return r.choice(np.array([2, 3, 4, 8], np.uint8), size=nb, p=[0.40, 0.40, 0.15, 0.05])

    def kv(self, agent: int, layer: int, tag: int) -> np.ndarray:
        """bf16 bits [L][Hkv][D] of one agent's K (tag 1) or V (tag 2)."""
        L = self.lengths[agent]
        chans = None
        if tag == TAG_K and self.outliers:
            chans = outlier_channels(self.wid, self.n_kv_heads, self.head_dim, self.outliers, layer)
        return normal_bf16((L, self.n_kv_heads, self.head_dim), self.wid, tag, agent, layer,
                           chans, self.outlier_gain)

    def rope(self, agent: int, layer: int) -> np.ndarray:
        L = self.lengths[agent]
        return normal_bf16((L, self.n_kv_heads, self.rope_dim), self.wid, TAG_ROPE, agent, layer)

    def q(self, layer: int) -> np.ndarray:
        """Decode queries [A][Hq][D + rope]."""
        return normal_bf16((self.n_agents, self.n_q_heads, self.head_dim + self.rope_dim),
                           self.wid, TAG_Q, 0, layer)

    def chunk_new(self):
        """(q_new [n][Hq][D], k_new [n][Hkv][D], v_new [n][Hkv][D])."""
        n = self.n_new
        return (normal_bf16((n, self.n_q_heads, self.head_dim), self.wid, TAG_Q),
                normal_bf16((n, self.n_kv_heads, self.head_dim), self.wid, TAG_KNEW),
                normal_bf16((n, self.n_kv_heads, self.head_dim), self.wid, TAG_VNEW))


def _split_window(L: int, keep_recent: int):
    """Full blocks are quantized; at least ``keep_recent`` newest tokens stay bf16."""
    nq = 64 * (max(L - keep_recent, 0) // 64)
    return nq // 64, L - nq


def workload(wid: int) -> Workload:
    if wid == 0:   # tiny: 1 agent, 8/2 heads, D 64, 256 tokens, Q4, 2 K outliers x10
        return Workload(0, "tiny-q4-decode", 1, 8, 2, 64, [256], [4], [0], outliers=2,
                        outlier_gain=10.0, scale=1.0 / 8.0)
    if wid == 1:   # Llama-3.1-8B layer, 10 agents x 4096 tokens, Q4, 4 K outliers x8
        return Workload(1, "llama8b-10agent-q4-decode", 10, 32, 8, 128, [4096] * 10, [64] * 10,
                        [0] * 10, outliers=4, outlier_gain=8.0, scale=128 ** -0.5)
    if wid == 2:   # Gemma-3-12B, 8 agents, L ~ U{1024..16384}, widths {2,3,4,8}, 128 bf16 recent
        r = rng(2, TAG_LEN)
        lengths = [int(v) for v in r.integers(1024, 16384, size=8, endpoint=True)]
        nbw = [_split_window(L, 128) for L in lengths]
        layers = sorted(int(v) for v in rng(2, TAG_LAYER).choice(48, size=8, replace=False))
        return Workload(2, "gemma12b-8agent-mixed-decode", 8, 16, 8, 256, lengths,
                        [b for b, _ in nbw], [w for _, w in nbw], layers=layers,
                        scale=1.0 / 16.0)
    if wid == 3:   # Llama-3.1-8B restore of 32768 tokens + 512-token causal chunk
        return Workload(3, "llama8b-32k-restore-512-chunk", 1, 32, 8, 128, [32768], [512], [0],
                        n_new=512, scale=128 ** -0.5)
    if wid == 4:   # DeepSeek-V2-Lite latent: 4 agents x 32768, latent 512 Q4 + rope 64 bf16
        return Workload(4, "deepseek-v2-lite-mla-4agent-32k-decode", 4, 16, 1, 512, [32768] * 4,
                        [512] * 4, [0] * 4, rope_dim=64, scale=576 ** -0.5)
    raise ValueError(wid)
