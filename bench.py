#!/usr/bin/env python3
"""Benchmark of the quantized KV-cache hot path on one MI355X.

One step = one batched decode step over packed caches written beforehand:
the attention call (kvq_attend_decode: split + merge launches) of every
layer of the workload over all agents, or one chunk call (kvq_attend_chunk)
for the restore + chunk workload.  Cache copies rotate so that at least
2 x 256 MB of other copies pass between two reads of one (the Infinity
Cache holds nothing a call can use); every copy is visited once, then the
step runs untimed for ~100 ms (the GPU's clocks rise over the first few ms
of sustained work), then the W warmup steps.  The K timed steps run back to
back between one pair of HIP events on the launch stream (eager launches,
or with --graph one replay of their captured HIP graph, checked against an
eager step).

Prints one JSON line.  `value` is the step's algorithmic attention bytes
(codes and scale/bias of the blocks, bf16 windows, rope rows, queries and
outputs) divided by the step time, in GB/s; `roofline` is for that call.
The quantize launch that builds a layer's K and V caches (kvq_quantize_kv)
is timed the same way on its own and reported as `quantize_GBps` with
`roofline_quantize`.  `cpu_baseline` times the C oracle on a bounded sample
of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--graph]
Side modes (one JSON line each): --restore, --append N, --card, --topk K,
--alloc, --copy-calibration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-KV decode attn effective HBM GB/s + tokens/s; quantize GB/s"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time the K steps as one replay of their HIP graph instead of eager launches")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (the reference for the HBM byte counters)")
    p.add_argument("--topk", type=int, default=0, metavar="K",
                   help="time top-K sparse decode (K of the T/64 blocks per agent, T = --topk-tokens) "
                        "on Llama 10-agent caches, beside the full decode, instead of the workload step")
    p.add_argument("--topk-tokens", type=int, default=0, metavar="T",
                   help="cached tokens per agent for --topk (a multiple of 64; default 4096, 32768 with --topk-mla)")
    p.add_argument("--topk-mla", action="store_true",
                   help="--topk on the DeepSeek-V2-Lite latent shape (4 agents, 512-dim latent + 64 rope dims)")
    p.add_argument("--restore", action="store_true",
                   help="time the restore (dequantize to bf16) of the 32 768-token Q4 cache, K then V")
    p.add_argument("--alloc", action="store_true",
                   help="time block sensitivity (GPU) and the budgeted width allocation (host) on the "
                        "Gemma mixed-width shape instead of the workload step")
    p.add_argument("--card", action="store_true",
                   help="time CacheCard gather and scatter of the Llama 10-agent caches "
                        "(device image <-> cache) instead of the workload step")
    p.add_argument("--append", type=int, default=0, metavar="N_NEW",
                   help="time kvq_append of N_NEW tokens per agent on the Llama 10-agent shape "
                        "(windows of 128..191 tokens, keep 128) instead of the workload step")
    return p.parse_args()


COPY_BYTES = 1 << 30

# HBM bytes per launch of the dominant kernel from rocprofv3 --pmc passes
# (FETCH_SIZE and WRITE_SIZE, KiB per dispatch), scaled by the factors a
# plain 1 GiB device copy gives (bench.py --copy-calibration: FETCH_SIZE
# reads 524300 KiB for 1 GiB read -> x2.0; WRITE_SIZE 1048576 KiB -> x1.0).
# Each entry holds the SHA-256 prefix of the kernel's source at measurement
# time; a changed source reports null until measured again.
COUNTER_FACTOR = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
TRAFFIC = {
    # (workload, call): (source files, sha256 prefix of their contents in that
    # order, FETCH_SIZE KiB, WRITE_SIZE KiB), summed over the call's kernels
    (1, "kvq quantize"): (("quantize.hip",), "7dbb68a3958abdc3", 82011.6, 46080.1),
    (2, "kvq quantize"): (("quantize.hip",), "7dbb68a3958abdc3", 268019.0, 119946.0),
    (3, "kvq dequantize"): (("quantize.hip",), "7dbb68a3958abdc3", 9271.5, 65561.8),
    (3, "kvq quantize"): (("quantize.hip",), "7dbb68a3958abdc3", 65619.1, 36864.1),
    (3, "kvq attend_chunk"): (("chunk.hip",), "f1f82d8b56dc9dce", 47171.2 + 16694.0, 35002.1 + 8192.0),
    (1, "kvq attend_decode"): (("decode_g4.hip", "decode_gqa.hip"), "a496b36197a8d745",
                               23481.7 + 2656.4, 5440.0 + 160.0),
    (2, "kvq attend_decode"): (("decode_g4.hip", "decode_gqa.hip"), "a496b36197a8d745",
                               64375.4 + 2256.5, 4488.0 + 128.0),
    (4, "kvq quantize"): (("quantize.hip",), "7dbb68a3958abdc3", 65779.2, 36881.8),
    (4, "kvq attend_decode"): (("mla.hip", "decode_gqa.hip"), "5116f3d8b60628e6",
                               27102.6 + 4169.1, 10746.6 + 128.0),
    ("alloc", "kvq block_sensitivity"): (("alloc.hip",), "daa276e1c505e00b", 430498.4, 62.0),
}


def traffic_bytes(workload, kernel: str):
    import hashlib
    e = TRAFFIC.get((workload, kernel))
    if e is None:
        return None
    srcs, sha, fetch_kib, write_kib = e
    m = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(ROOT, "quantized_kv_cache_group_amd", "csrc", src), "rb") as f:
            m.update(f.read())
    if m.hexdigest()[:16] != sha:
        return None
    return (fetch_kib * COUNTER_FACTOR["FETCH_SIZE"] + write_kib * COUNTER_FACTOR["WRITE_SIZE"]) * 1024


def copy_calibration():
    """A plain copy of known size: under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    it gives the counter-to-bytes factors used for `traffic`."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": 5}))



SETTLE_MS = 100.0


def settle(torch, fn, ms: float = SETTLE_MS) -> int:
    """Untimed calls fn(0), fn(1), ... until `ms` of wall time has passed
    (synchronizing every 8 calls); returns the number of calls.  For the
    first few ms of sustained work the GPU's clocks are still rising (the
    chunk call of workload 3 measured 353 us per call after 5 warmup steps,
    317 us after ~35 ms of the same work; the Gemma decode 46.6 against 45.4
    us, the latent decode 29.7 against 27.4 us), so every timed region starts
    from the clocks a continuous serving loop runs at.  Runs before the W
    warmup steps, which stay exactly W."""
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return n


def timing_events(torch, stream, n: int = 2):
    """n timing events, each recorded once on `stream` and waited for before
    it opens a timed region: a timed region opened by a never-recorded event
    has at times shown a gap of ~0.9 ms before its first launch."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    return evs

# ---------------------------------------------------------------------------
def gpu_inputs(w, torch, seed: int):
    """bf16 sources [A][Lmax][H][D] for K and V (and rope) of every layer,
    N(0,1) with the workload's outlier channels, drawn on the GPU."""
    import kvq_synth as syn
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    A, H, D = w.n_agents, w.n_kv_heads, w.head_dim
    S = max(64 * b for b in w.n_blocks)
    chans = syn.outlier_channels(w.wid, H, D, w.outliers) if w.outliers else None

    def draw(shape, outl):
        x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        if outl is not None:
            for h, c in enumerate(outl):
                x[..., h, torch.as_tensor(c, device="cuda")] *= w.outlier_gain
        return x.to(torch.bfloat16).contiguous()

    k = draw((A, S, H, D), chans)
    v = None if w.rope_dim else draw((A, S, H, D), None)
    return k, v


def algorithmic_bytes(w, cache, n_q_heads):
    """(quantize bytes for K+V, attention bytes) of one layer."""
    import quantized_kv_cache_group_amd as kvq
    H, D = w.n_kv_heads, w.head_dim
    blocks = 0
    qelems = 0
    for a in range(w.n_agents):
        for j in range(w.n_blocks[a]):
            blocks += kvq.block_bytes(int(cache.bits_host[a, j]), H, D)
        qelems += 64 * w.n_blocks[a] * H * D
    n_t = 1 if w.rope_dim else 2                       # K and V, or the latent only
    quant = n_t * (qelems * 2 + blocks)
    attn = n_t * blocks
    attn += n_t * sum(w.n_window) * H * D * 2           # bf16 window
    attn += sum(w.lengths) * H * w.rope_dim * 2         # bf16 rope
    if w.n_new:
        Hq = n_q_heads
        attn += w.n_new * (Hq + 2 * H) * D * 2 + w.n_new * Hq * D * 4
    else:
        attn += w.n_agents * n_q_heads * (D + w.rope_dim) * 2 + w.n_agents * n_q_heads * D * 4
    return quant, attn


def chunk_flops(w):
    P = w.lengths[0]
    visits = sum(P + i + 1 for i in range(w.n_new))
    return visits * w.n_q_heads * 4 * w.head_dim


# ---------------------------------------------------------------------------
def cpu_baseline(w, layer_ids):
    """Time the oracle on a bounded sample of the bench's own call, as GB/s of
    the same algorithmic attention bytes the GPU figure counts: whole passes
    of the decode over the agents of one layer (pools quantized beforehand,
    untimed), repeated to about 10 s of host time; for the chunk workload, a
    few query rows scaled to all rows.  Also times the oracle's decode (and
    quantize) of the tiny and the Llama 10-agent workloads on one thread."""
    import oracle
    oracle.lib()
    H, D = w.n_kv_heads, w.head_dim
    layer = layer_ids[0]
    prep = [_cpu_prep(w, layer, a) for a in range(w.n_agents if not w.n_new else 1)]
    t_used, bytes_done, passes, note = 0.0, 0.0, 0, ""
    while t_used < 10.0:
        passes += 1
        dt, b, note = _cpu_attend_pass(w, layer, H, D, prep)
        t_used += dt
        bytes_done += b
        if note:
            break
    res = {"value": round(bytes_done / t_used / 1e9, 4), "unit": "GB/s",
           "cores": oracle.max_threads(), "kind": "oracle",
           "sample": f"{passes} pass(es) of the attention over {len(prep)} of {w.n_agents} agents of "
                     f"layer {layer}: {bytes_done / 1e6:.1f} MB of algorithmic attention bytes in "
                     f"{t_used:.2f} s{note}"}
    res["single_thread"] = _cpu_single_thread()
    return res


def _cpu_prep(w, layer, a):
    import kvq_synth as syn
    import oracle
    H, D = w.n_kv_heads, w.head_dim
    k = w.kv(a, layer, syn.TAG_K)
    v = None if w.rope_dim else w.kv(a, layer, syn.TAG_V)
    nb, nw = w.n_blocks[a], w.n_window[a]
    bits = w.bits(a, layer)
    off, tot = oracle.packed_offsets(bits, H, D)
    pool = np.zeros(2 * tot if v is not None else tot, np.uint8)
    voff = off + np.uint64(tot) if v is not None else None
    oracle.quantize_seq(k, H, D, bits, off, pool)
    if v is not None:
        oracle.quantize_seq(v, H, D, bits, voff, pool)
    kw = k[64 * nb:64 * nb + nw] if nw else None
    vw = v[64 * nb:64 * nb + nw] if (nw and v is not None) else None
    rope = w.rope(a, layer) if w.rope_dim else None
    return dict(a=a, bits=bits, off=off, voff=voff, pool=pool, kw=kw, vw=vw, rope=rope)


def _cpu_attend_pass(w, layer, H, D, prep):
    import oracle
    dt, b, note = 0.0, 0.0, ""
    q_all = None if w.n_new else w.q(layer)
    for pr in prep:
        a = pr["a"]
        if w.n_new:
            qn, kn, vn = w.chunk_new()
            rows = 4
            t1 = time.perf_counter()
            oracle.attend_chunk_seq(pr["pool"], pr["bits"], pr["off"], pr["voff"], pr["kw"], pr["vw"], H, D,
                                    qn, kn, vn, w.scale, w.n_new - rows, w.n_new)
            dt += (time.perf_counter() - t1) * (w.n_new / rows)
            _, b_a = algorithmic_bytes(w, _FakeCache(w, [pr["bits"]]), w.n_q_heads)
            b += b_a
            note = (f"; timed on the last {rows} of {w.n_new} query rows and scaled by {w.n_new // rows}")
            break
        t1 = time.perf_counter()
        oracle.attend_decode_seq(pr["pool"], pr["bits"], pr["off"], pr["voff"], pr["kw"], pr["vw"], pr["rope"],
                                 H, D, q_all[a], w.scale)
        dt += time.perf_counter() - t1
        n_t = 1 if w.rope_dim else 2
        blk = sum(oracle.block_bytes(int(x), H, D) for x in pr["bits"])
        b += (n_t * blk + n_t * w.n_window[a] * H * D * 2 + w.lengths[a] * H * w.rope_dim * 2 +
              w.n_q_heads * (D + w.rope_dim) * 2 + w.n_q_heads * D * 4)
    return dt, b, note


def _cpu_single_thread():
    """The oracle on one thread: decode GB/s of the tiny and the Llama
    10-agent workloads (one pass over their agents), and quantize GB/s of
    the tiny one."""
    import ctypes
    import kvq_synth as syn
    import oracle
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    n0 = oracle.max_threads()
    gomp.omp_set_num_threads(1)
    out = {"cores": 1}
    try:
        for wid in (0, 1):
            w = syn.workload(wid)
            H, D = w.n_kv_heads, w.head_dim
            prep = [_cpu_prep(w, 0, a) for a in range(w.n_agents)]
            dt, b, _ = _cpu_attend_pass(w, 0, H, D, prep)
            out[f"{w.name}_decode_GBps"] = round(b / dt / 1e9, 4)
            out[f"{w.name}_decode_s"] = round(dt, 4)
            if wid == 0:
                k = w.kv(0, 0, syn.TAG_K)
                bits = w.bits(0, 0)
                off, tot = oracle.packed_offsets(bits, H, D)
                pool = np.zeros(tot, np.uint8)
                reps, t0 = 0, time.perf_counter()
                while time.perf_counter() - t0 < 1.0:
                    oracle.quantize_seq(k, H, D, bits, off, pool)
                    reps += 1
                dq = (time.perf_counter() - t0) / reps
                blk = sum(oracle.block_bytes(int(x), H, D) for x in bits)
                out[f"{w.name}_quantize_GBps"] = round((k.size * 2 + blk) / dq / 1e9, 4)
    finally:
        gomp.omp_set_num_threads(n0)
    return out


class _FakeCache:
    def __init__(self, w, bits_list):
        mb = max(w.n_blocks)
        self.bits_host = np.full((w.n_agents, max(mb, 1)), 4, np.uint8)
        for a, b in enumerate(bits_list):
            self.bits_host[a, :b.size] = b


# ---------------------------------------------------------------------------
def append_bench(args):
    """kvq_append (window roll) on the Llama-3.1-8B layer shape, 10 agents:
    windows start at 128..191 bf16 tokens (keep 128) over 64 Q4 blocks, and
    each call appends N_NEW tokens of K and V per agent, back to back on one
    cache whose blocks advance through the pool (as in a decode or prefill
    loop).  Algorithmic bytes per call: the new rows read, the old window
    rows moved or cut (read, when a block is cut), the window rows written
    and the block payloads written, for K and V, from the host copy of the
    counts before each call.  New-row buffers rotate past the 256 MB
    last-level cache."""
    import torch
    import kvq_synth as syn
    import quantized_kv_cache_group_amd as kvq

    kvq.lib()
    torch.cuda.set_device(0)
    w = syn.workload(1)
    A, H, D, n = w.n_agents, w.n_kv_heads, w.head_dim, args.append
    keep, cap = 128, 191
    r = syn.rng(1, syn.TAG_LEN)
    win0 = [int(v) for v in r.integers(keep, cap, size=A, endpoint=True)]
    nb0 = [64] * A
    calls = args.warmup + args.steps
    mb = 64 + (cap + n * calls) // 64 + 1
    blk = kvq.block_bytes(4, H, D)
    row = H * D * 2
    c = kvq.LayerCache(H, D, nb0, win0, None, max_blocks=mb, window_cap=cap, future_bits=4)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    c.k_window.normal_(generator=g)
    c.v_window.normal_(generator=g)
    R = min(16, max(2, int(np.ceil(2 * MALL_BYTES / max(2 * A * n * row, 1))) + 1))
    news = [(torch.randn((A, n, H, D), generator=g, device="cuda").to(torch.bfloat16),
             torch.randn((A, n, H, D), generator=g, device="cuda").to(torch.bfloat16)) for _ in range(R)]

    def call_bytes():
        b = 0
        for a in range(A):
            W = c.n_window_host[a]
            T = W + n
            k = (T - keep) // 64 if T > keep else 0
            moved, written = (W, T - 64 * k) if k else (0, n)
            b += 2 * ((n + moved + written) * row + k * blk)
        return b

    for i in range(args.warmup):
        c.append(*news[i % R], keep_recent=keep)
    torch.cuda.synchronize()
    total = 0
    stream = torch.cuda.current_stream()
    e0, e1 = timing_events(torch, torch.cuda.current_stream())
    e0.record(stream)
    for i in range(args.steps):
        total += call_bytes()
        c.append(*news[(args.warmup + i) % R], keep_recent=keep)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    gbs = total / args.steps / (us * 1e-6) / 1e9
    res = {"metric": "kvq_append (quantize on append) GB/s", "value": round(gbs, 2), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "us_per_call": round(us, 3),
           "higher_is_better": True, "dtype": "bf16->u4", "data": "synthetic",
           "config": {"workload": f"llama8b-10agent-append-{n}", "agents": A, "kv_heads": H, "head_dim": D,
                      "window_start": win0, "keep_recent": keep, "window_cap": cap, "n_new": n,
                      "bits": 4, "rotated_inputs": R},
           "bytes_per_call": round(total / args.steps),
           "roofline": {"kernel": "kvq append", "bound": "hbm", "achieved": round(gbs, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": None}}
    print(json.dumps(res), flush=True)


def topk_bench(args):
    """Top-K sparse decode, timed beside the full decode of the same caches.
    Default shape: the Llama-3.1-8B layer, 10 agents x T Q4 tokens (T/64
    blocks each, T = --topk-tokens, 4096 by default), K and V caches.  With
    --topk-mla: the DeepSeek-V2-Lite latent shape, 4 agents x T tokens (T
    defaults to 32768 there), one 512-dim Q4 latent head plus 64 bf16 rope
    dims, 16 query heads (the block scores then run the generic scoring
    kernel over latent and rope dims).  Algorithmic bytes per call: every
    block's codes (and rope rows) for the scores, the kept blocks' codes (and
    rope rows) again for the decode, q and out.  Cache copies rotate past the
    256 MB cache."""
    import torch
    import kvq_synth as syn
    import quantized_kv_cache_group_amd as kvq

    kvq.lib()
    torch.cuda.set_device(0)
    mla = args.topk_mla
    w = syn.workload(4 if mla else 1)
    A, H, D, Hq, K, R_ = w.n_agents, w.n_kv_heads, w.head_dim, w.n_q_heads, args.topk, w.rope_dim
    T = args.topk_tokens if args.topk_tokens else (32768 if mla else 4096)
    if T < 64 or T % 64:
        print("--topk-tokens must be a positive multiple of 64", file=sys.stderr)
        sys.exit(2)
    nblk = T // 64
    blk = kvq.block_bytes(4, H, D)
    n_t = 1 if mla else 2
    rope_tok = H * R_ * 2                            # rope bytes per token
    one = A * nblk * (n_t * blk + 64 * rope_tok)
    R = min(12, max(2, int(np.ceil(2 * MALL_BYTES / one)) + 1))
    caches = [kvq.LayerCache(H, D, [nblk] * A, [0] * A, None, latent=mla, rope_dim=R_) for _ in range(R)]
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    src = [torch.randn((A, T, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(2)]
    for i, c in enumerate(caches):
        c.quantize("k", src[i % 2])
        if not mla:
            c.quantize("v", src[(i + 1) % 2])
        if c.rope is not None:
            c.rope.normal_(generator=g)
    q = torch.randn((A, Hq, D + R_), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((A, Hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(caches[0].topk_workspace_bytes(Hq, K), caches[0].decode_workspace_bytes(Hq)),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def one(sparse, i):
        c = caches[i % R]
        if sparse:
            c.attend_decode_topk(q, w.scale, K, out=out, workspace=ws)
        else:
            c.attend_decode(q, w.scale, out=out, workspace=ws)

    def run(sparse, steps):
        e0, e1 = timing_events(torch, torch.cuda.current_stream())
        e0.record(stream)
        for i in range(steps):
            one(sparse, i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps
    settle(torch, lambda i: one(True, i))
    run(True, args.warmup)
    sp_us = run(True, args.steps)
    settle(torch, lambda i: one(False, i))
    run(False, args.warmup)
    full_us = run(False, args.steps)
    kb = min(K, nblk)
    algo = (A * nblk * (blk + 64 * rope_tok)                   # scores: every block's K codes and rope rows
            + A * kb * (n_t * blk + 64 * rope_tok)              # decode over the kept blocks
            + A * Hq * (D + R_) * 2 + A * Hq * D * 4)
    gbs = algo / (sp_us * 1e-6) / 1e9
    name = (f"deepseek-v2-lite-mla-4agent-{T}tok-q4-top{K}" if mla else f"llama8b-10agent-{T}tok-q4-top{K}")
    res = {"metric": "top-K sparse decode GB/s", "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_ms": SETTLE_MS, "higher_is_better": True, "dtype": "fp16 mfma, fp32 acc",
           "data": "synthetic",
           "config": {"workload": name, "agents": A, "q_heads": Hq, "kv_heads": H, "head_dim": D,
                      "rope_dim": R_, "blocks": nblk, "top_k": K, "bits": 4, "rotated_copies": R},
           "sparse_us": round(sp_us, 3), "full_decode_us": round(full_us, 3),
           "speedup_vs_full": round(full_us / sp_us, 3), "bytes_per_call": algo,
           "roofline": {"kernel": "kvq attend_decode_topk", "bound": "hbm", "achieved": round(gbs, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": None}}
    print(json.dumps(res), flush=True)


def alloc_bench(args):
    """Width allocation on the Gemma-3-12B mixed-width shape (8 agents, L ~
    U{1024..16384}, Hq 16 / Hkv 8, D 256): block sensitivity of every block's
    bf16 K and V rows for the layer's query (GPU; bytes = the rows read), then
    the greedy widths of all blocks of the 8 sampled layers at a mean-3-bit
    budget (host C++)."""
    import torch
    import kvq_synth as syn
    import quantized_kv_cache_group_amd as kvq

    kvq.lib()
    torch.cuda.set_device(0)
    w = syn.workload(2)
    A, H, D, Hq = w.n_agents, w.n_kv_heads, w.head_dim, w.n_q_heads
    S_tok = 64 * max(w.n_blocks)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    R = 2
    ks = [torch.randn((A, S_tok, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(R)]
    vs = [torch.randn((A, S_tok, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(R)]
    q = torch.randn((A, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((A, max(w.n_blocks)), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: kvq.block_sensitivity(ks[i % R], vs[i % R], q, w.scale, out=out))
    for i in range(args.warmup):
        kvq.block_sensitivity(ks[i % R], vs[i % R], q, w.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = timing_events(torch, torch.cuda.current_stream())
    e0.record(stream)
    for i in range(args.steps):
        kvq.block_sensitivity(ks[i % R], vs[i % R], q, w.scale, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    rows = A * S_tok * H * D * 2 * 2
    gbs = rows / (us * 1e-6) / 1e9
    S = out.cpu().numpy()
    allS = np.concatenate([np.tile(S[a, :w.n_blocks[a]], len(w.layers)) for a in range(A)]).astype(np.float32)
    budget = allS.size * kvq.block_bytes(3, H, D)
    t0 = time.perf_counter()
    widths = kvq.allocate_widths(allS, H, D, budget)
    t_alloc = time.perf_counter() - t0
    res = {"metric": "block sensitivity GB/s", "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_ms": SETTLE_MS, "higher_is_better": True, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "gemma12b-8agent-width-allocation", "agents": A, "q_heads": Hq, "kv_heads": H,
                      "head_dim": D, "rows_per_agent": S_tok, "layers": len(w.layers)},
           "sensitivity_us": round(us, 3), "blocks_allocated": int(allS.size),
           "allocate_ms_host": round(t_alloc * 1e3, 3),
           "mean_bits": round(float(np.mean(widths)), 4),
           "width_counts": {str(b): int((widths == b).sum()) for b in (2, 3, 4, 8)},
           "roofline": {"kernel": "kvq block_sensitivity", "bound": "hbm", "achieved": round(gbs, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": traffic_bytes("alloc", "kvq block_sensitivity")}}
    print(json.dumps(res), flush=True)


def restore_bench(args):
    """Restore (dequantize) of the restore + chunk workload's cache: one
    sequence of 32 768 Q4 tokens, 8 KV heads of 128 dims, K then V restored
    to bf16 rows.  Algorithmic bytes per (K, V) pair: codes and metadata read
    (2 x 18 MiB) + bf16 rows written (2 x 64 MiB).  Caches and outputs rotate
    past the 256 MB last-level cache."""
    import torch
    import kvq_synth as syn
    import quantized_kv_cache_group_amd as kvq

    kvq.lib()
    torch.cuda.set_device(0)
    w = syn.workload(3)
    A, H, D = w.n_agents, w.n_kv_heads, w.head_dim
    S = 64 * max(w.n_blocks)
    R = 3
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    caches = []
    for r in range(R):
        c = kvq.LayerCache(H, D, w.n_blocks, w.n_window, None)
        k = torch.randn((A, S, H, D), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((A, S, H, D), generator=g, device="cuda").to(torch.bfloat16)
        c.quantize_kv(k, v)
        caches.append(c)
        del k, v
    outs = [[torch.empty((A, S, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)] for _ in range(R)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def one(i):
        c, o = caches[i % R], outs[i % R]
        c.dequantize("k", o[0])
        c.dequantize("v", o[1])

    def run(steps):
        e0, e1 = timing_events(torch, torch.cuda.current_stream())
        e0.record(stream)
        for i in range(steps):
            one(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps
    settle(torch, one)
    run(args.warmup)
    us = run(args.steps)
    blk = kvq.block_bytes(4, H, D)
    algo = 2 * (A * w.n_blocks[0] * blk + A * S * H * D * 2)
    gbs = algo / (us * 1e-6) / 1e9
    res = {"metric": "kvq_dequantize (restore) GB/s", "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_ms": SETTLE_MS, "higher_is_better": True, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "llama8b-32k-restore-kv-bf16", "agents": A, "kv_heads": H, "head_dim": D,
                      "cache_tokens": S, "bits": 4, "rotated_copies": R},
           "us_per_kv_pair": round(us, 3), "bytes_per_kv_pair": algo,
           # one launch restores one tensor: half the pair's bytes in half its time
           "roofline": {"kernel": "kvq dequantize", "bound": "hbm", "achieved": round(gbs, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "algo_bytes_per_launch": algo // 2,
                        "traffic": traffic_bytes(3, "kvq dequantize")}}
    print(json.dumps(res), flush=True)


def card_bench(args):
    """CacheCard gather (cache -> contiguous device image) and scatter (image
    -> cache) for each of the 10 agents of the Llama-3.1-8B layer shape (4096
    tokens, 64 Q4 blocks, K and V).  Bytes moved per call: the image read plus
    written.  Copies rotate past the 256 MB last-level cache.  Host file
    framing is timed separately (host I/O, not a GPU figure)."""
    import tempfile
    import torch
    import kvq_synth as syn
    import quantized_kv_cache_group_amd as kvq
    from quantized_kv_cache_group_amd import card

    kvq.lib()
    torch.cuda.set_device(0)
    w = syn.workload(1)
    A, H, D = w.n_agents, w.n_kv_heads, w.head_dim
    one = A * 2 * w.n_blocks[0] * kvq.block_bytes(4, H, D)
    R = min(8, max(2, int(np.ceil(2 * MALL_BYTES / (2 * one))) + 1))
    caches = [kvq.LayerCache(H, D, w.n_blocks, w.n_window, None) for _ in range(R)]
    for c in caches:
        c.k_pool.random_(0, 256)
        c.v_pool.random_(0, 256)
    n = caches[0].card_bytes(0)
    imgs = [[torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(A)] for _ in range(R)]
    stream = torch.cuda.current_stream()
    strm = kvq._stream()
    stores = [(c.store("k"), c.store("v")) for c in caches]

    def one(kind, i):
        c = caches[i % R]
        for a in range(A):
            # C ABI directly (sizes precomputed; for scatter the tables already
            # hold the card's counts and widths)
            fn = kvq.lib().kvq_card_gather if kind == "gather" else kvq.lib().kvq_card_scatter
            kvq._check(fn(kvq.ctypes.byref(c.layout()), kvq.ctypes.byref(stores[i % R][0]),
                          kvq.ctypes.byref(stores[i % R][1]), None, 0, a, kvq._ptr(imgs[i % R][a]), n,
                          strm), kind)

    def run(kind, steps):
        e0, e1 = timing_events(torch, torch.cuda.current_stream())
        e0.record(stream)
        for i in range(steps):
            one(kind, i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (steps * A)
    settle(torch, lambda i: one("gather", i))
    run("gather", args.warmup)
    g_us = run("gather", args.steps)
    run("scatter", args.warmup)
    s_us = run("scatter", args.steps)
    t0 = time.perf_counter()
    with tempfile.TemporaryDirectory() as d:
        for a in range(A):
            card.save_card(caches[0], a, f"{d}/{a}.kvqcard")
        t1 = time.perf_counter()
        c2, _ = card.cache_from_cards([f"{d}/{a}.kvqcard" for a in range(A)])
        torch.cuda.synchronize()
        t2 = time.perf_counter()
    g_gbs = 2 * n / (g_us * 1e-6) / 1e9
    s_gbs = 2 * n / (s_us * 1e-6) / 1e9
    res = {"metric": "CacheCard gather GB/s", "value": round(g_gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_ms": SETTLE_MS, "higher_is_better": True, "dtype": "u8",
           "data": "synthetic",
           "config": {"workload": "llama8b-10agent-q4-cachecard", "agents": A, "kv_heads": H, "head_dim": D,
                      "tokens": w.lengths[0], "bits": 4, "image_bytes": n, "rotated_copies": R},
           "gather_us_per_agent": round(g_us, 3), "scatter_us_per_agent": round(s_us, 3),
           "scatter_GBps": round(s_gbs, 2),
           "host_file_save_s_10_agents": round(t1 - t0, 4), "host_file_load_s_10_agents": round(t2 - t1, 4),
           "roofline": {"kernel": "kvq card gather", "bound": "hbm", "achieved": round(g_gbs, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                        "traffic": None}}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.restore:
        restore_bench(args)
        return
    if args.card:
        card_bench(args)
        return
    if args.alloc:
        alloc_bench(args)
        return
    if args.topk:
        topk_bench(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.append:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        append_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    import kvq_synth as syn
    import quantized_kv_cache_group_amd as kvq

    kvq.lib()
    torch.cuda.set_device(0)
    w = syn.workload(args.workload)
    H, D, A, Hq = w.n_kv_heads, w.head_dim, w.n_agents, w.n_q_heads
    layers = w.layers if args.workload == 2 else [0]
    L = len(layers)
    latent = w.rope_dim > 0
    bits_per_layer = [[w.bits(a, layer) for a in range(A)] for layer in layers]
    per_layer = [algorithmic_bytes(w, _FakeCache(w, bits), Hq) for bits in bits_per_layer]
    q_bytes = sum(qb for qb, _ in per_layer)         # quantize: bf16 read + codes/meta written, all layers
    a_bytes = sum(ab for _, ab in per_layer)         # attention: all layers

    # Cache copies: one pass over all copies of all layers reads at least
    # 2 x 256 MB of distinct attention bytes, so no call finds its cache in
    # the Infinity Cache (the Gemma workload's 8 layers already pass 1 GB).
    C = max(1, int(np.ceil(2 * MALL_BYTES / max(a_bytes, 1))) + (0 if a_bytes >= 2 * MALL_BYTES else 1))
    sets = [[kvq.LayerCache(H, D, w.n_blocks, w.n_window, bits, latent=latent, rope_dim=w.rope_dim)
             for bits in bits_per_layer] for _ in range(C)]
    # Quantize sources: enough copies that 2 x 256 MB of other sources pass
    # between two reads of one (the bf16 rows of all layers count).
    src_bytes = sum(2 * (1 if latent else 2) * sum(64 * n for n in w.n_blocks) * H * D for _ in layers)
    n_src = max(1, int(np.ceil(2 * MALL_BYTES / max(src_bytes, 1))) + (0 if src_bytes >= 2 * MALL_BYTES else 1))
    srcs = [[gpu_inputs(w, torch, 1000 * r + li) for li in range(L)] for r in range(n_src)]
    gq = torch.Generator(device="cuda")
    gq.manual_seed(7)
    if w.n_new:
        qn = torch.randn((A, w.n_new, Hq, D), generator=gq, device="cuda").to(torch.bfloat16)
        kn = torch.randn((A, w.n_new, H, D), generator=gq, device="cuda").to(torch.bfloat16)
        vn = torch.randn((A, w.n_new, H, D), generator=gq, device="cuda").to(torch.bfloat16)
        out = torch.empty((A, w.n_new, Hq, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(sets[0][0].chunk_workspace_bytes(Hq, w.n_new), dtype=torch.uint8, device="cuda")
    else:
        qs = [torch.randn((A, Hq, D + w.rope_dim), generator=gq, device="cuda").to(torch.bfloat16)
              for _ in layers]
        out = torch.empty((A, Hq, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(sets[0][0].decode_workspace_bytes(Hq), 256), dtype=torch.uint8, device="cuda")
    # Every copy is quantized once from the sources; windows and rope are
    # bf16 storage, filled with N(0,1).
    for r, cs in enumerate(sets):
        for li, c in enumerate(cs):
            k, v = srcs[r % n_src][li]
            c.quantize_kv(k, v)
            for t in (c.k_window, c.v_window, c.rope):
                if t is not None:
                    t.normal_(generator=gq)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def attend(c, li):
        if w.n_new:
            c.attend_chunk(qn, kn, vn, w.scale, out=out, workspace=ws)
        else:
            c.attend_decode(qs[li], w.scale, out=out, workspace=ws)

    def step(i):
        # one batched decode step: every layer's attention call over the
        # agents' packed caches (copy i mod C)
        cs = sets[i % C]
        for li in range(L):
            attend(cs[li], li)

    # One untimed visit of every cache copy first: the timed steps then see
    # each copy as it is in steady rotation (its first visit alone pays for
    # page-table walks: up to ~2x the call time of a visited copy).
    for i in range(C):
        step(i)
    torch.cuda.synchronize()
    n_settle = settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # With --graph the K timed steps are captured once as a HIP graph (the split and
    # merge launches of every layer's call, over preallocated outputs and
    # workspace; nothing is allocated or cleared inside) and replayed, so a
    # call's host-side launch cost does not pad the GPU time of short
    # calls.  An untimed replay first; its last output must equal an eager
    # run of the same step.  The timed region carries no events inside: the
    # call duration is the timed region divided by its calls.
    graph = None
    graph_check = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
        graph.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        step(args.warmup + args.steps - 1)
        torch.cuda.synchronize()
        graph_check = float((replayed - out).abs().max())
        if graph_check != 0.0:
            raise SystemExit(f"graph replay differs from the eager step (max |diff| {graph_check})")
    t_start, t_end = timing_events(torch, stream)
    t_start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = ms_step / L                             # one attention call (split + merge launches)
    value = a_bytes / (ms_step * 1e-3) / 1e9

    # Quantize (building the caches): every layer's K and V in one launch
    # per layer, rotating sources and destination copies, timed the same way.
    QREPS = max(2 * L, 8)

    def quant(i):
        li = i % L
        k, v = srcs[(i // L) % n_src][li]
        sets[(i // L) % C][li].quantize_kv(k, v)

    for i in range(L):
        quant(i)
    torch.cuda.synchronize()
    e_a, e_b = timing_events(torch, stream)
    e_a.record(stream)
    for i in range(QREPS):
        quant(i)
    e_b.record(stream)
    torch.cuda.synchronize()
    quant_launch_ms = e_a.elapsed_time(e_b) / QREPS
    quant_gbs = (q_bytes / L) / (quant_launch_ms * 1e-3) / 1e9
    attn_gbs = (a_bytes / L) / (attn_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 mfma, fp32 acc",
        "data": "synthetic",
        "config": {"workload": w.name, "agents": A, "layers": L, "q_heads": Hq,
                   "kv_heads": H, "head_dim": D, "cache_tokens": w.lengths if A <= 10 else None,
                   "bits": "2/3/4/8 mixed, mean 3" if args.workload == 2 else 4, "group": 64,
                   "rope_dim": w.rope_dim, "new_tokens": w.n_new,
                   "step": ("one batched decode step: the attention call of every layer"
                            if not w.n_new else "one chunk attention call"),
                   "rotated_cache_copies": C, "rotated_sources": n_src},
        "timing": "eager launches" if graph is None else "one HIP graph replay of the K steps (checked against eager)",
        "settle": {"steps": n_settle, "ms": SETTLE_MS,
                   "what": "untimed steps before the W warmup steps, until the GPU's clocks have risen"},
        "attn_bytes_per_step": int(a_bytes),
        "attn_us_per_call": round(attn_ms * 1e3, 3),
        "quantize_GBps": round(quant_gbs, 2),
        "quantize_us_per_launch": round(quant_launch_ms * 1e3, 3),
        "quantize_bytes_per_launch": int(q_bytes / L),
    }
    if w.n_new:
        fl = chunk_flops(w)
        tfl = fl / (attn_ms * 1e-3) / 1e12
        res["chunk_TFLOPs"] = round(tfl, 2)
        res["prefill_tokens_per_s"] = round(w.n_new / (attn_ms * 1e-3), 1)
        res["roofline"] = {"kernel": "kvq attend_chunk", "bound": "mfma", "achieved": round(tfl, 2),
                           "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
                           "traffic": traffic_bytes(args.workload, "kvq attend_chunk")}
    else:
        res["decode_tokens_per_s"] = round(A / (ms_step * 1e-3), 1)
        res["roofline"] = {"kernel": "kvq attend_decode", "bound": "hbm",
                           "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                           "traffic": traffic_bytes(args.workload, "kvq attend_decode")}
    tr = traffic_bytes(args.workload, "kvq quantize")
    res["roofline_quantize"] = {"kernel": "kvq quantize", "bound": "hbm", "achieved": round(quant_gbs, 2),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(quant_gbs / HBM_PEAK_GBS, 4),
                                "traffic": None if tr is None else round(tr)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, layers)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
