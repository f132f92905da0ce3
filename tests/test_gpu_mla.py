"""GPU latent (MLA) decode against the oracle at 2e-3 max-abs and 1e-3
relative L2: one 512-dim latent KV head quantized per 64-token block, an
optional 64-dim bf16 rope part, up to 16 query heads, values = the latent
(DeepSeek-V2-Lite absorbed attention, as Agent Memory Below the Prompt,
Abstract, restores it; QKVShare, Metodologia: restore, then ordinary
attention).

Cases: every code width (2, 3, 4 and 8 bits, mixed within a sequence),
without rope, fewer than 16 heads, bf16 windows of more than one 64-token
tile, a window-only sequence, a split longer than 64 blocks, and latents
scaled so that fp16 products of probabilities and group scales would
overflow if probabilities were allowed to exceed 1."""
import ctypes

import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
from parity import build, close, ref_decode, to_dev_bf16

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _decode(b, q_bits, scale):
    out = b.cache.attend_decode(to_dev_bf16(q_bits), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _mixed_bits(n_blocks, seed):
    rng = np.random.default_rng(seed)
    return [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in n_blocks]


@pytest.mark.parametrize("R,Hq", [(64, 16), (0, 16), (64, 5), (0, 1)])
def test_mla_mixed_widths(R, Hq):
    H, D = 1, 512
    window = [20, 100, 0, 50]
    n_blocks = [37, 11, 5, 0]
    lengths = [64 * n + w for n, w in zip(n_blocks, window)]
    b = build(H, D, lengths, bits=_mixed_bits(n_blocks, 7 + R + Hq), latent=True, rope_dim=R, window=window,
              seed=30 + Hq)
    q = syn.random_normal_bf16((4, Hq, D + R), 31 + R, scale=2.0)
    s = (D + R) ** -0.5
    close(_decode(b, q, s), ref_decode(b, q, s), what=f"mla mixed R={R} Hq={Hq}")


def test_mla_split_longer_than_block_table():
    """200 blocks under a layout of 20 000 blocks per sequence: the plan gives
    128 blocks per split, past the 64 table entries a split loads at once."""
    H, D, R, Hq = 1, 512, 64, 16
    nb, nw = 200, 30
    b = build(H, D, [64 * nb + nw], bits=_mixed_bits([nb], 41), latent=True, rope_dim=R, window=[nw], seed=40)
    c = b.cache
    MB = 20000
    bits = torch.zeros((1, MB), dtype=torch.uint8, device="cuda")
    offs = torch.zeros((1, MB), dtype=torch.int64, device="cuda")
    bits[0, :nb] = torch.from_numpy(c.bits_host[0, :nb]).cuda()
    offs[0, :nb] = torch.from_numpy(c.offset_host[0, :nb].astype(np.int64)).cuda()
    import quantized_kv_cache_group_amd as kvq
    L = kvq.Layout(n_seqs=1, n_heads=H, head_dim=D, max_blocks=MB, window_cap=c.window_cap,
                   n_blocks=c.n_blocks.data_ptr(), n_window=c.n_window.data_ptr(), bits=bits.data_ptr())
    K = kvq.Store(offset=offs.data_ptr(), pool=c.k_pool.data_ptr(), window=c.k_window.data_ptr())
    n = ctypes.c_size_t(0)
    lib = kvq.lib()
    assert lib.kvq_decode_workspace(ctypes.byref(L), Hq, R, ctypes.byref(n)) == 0
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    q = syn.random_normal_bf16((1, Hq, D + R), 42, scale=2.0)
    qd = to_dev_bf16(q)
    out = torch.full((1, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    s = (D + R) ** -0.5
    st = lib.kvq_attend_decode(ctypes.byref(L), ctypes.byref(K), None, c.rope.data_ptr(), R, qd.data_ptr(), Hq,
                               ctypes.c_float(s), out.data_ptr(), ws.data_ptr(), n.value, None)
    assert st == 0, lib.kvq_strerror(st)
    torch.cuda.synchronize()
    close(out.cpu().numpy(), ref_decode(b, q, s), what="mla 128-block split")


def test_mla_large_scales_in_slack_rises():
    """2-bit latents scaled by 8192 (group scales above 1024) with queries
    scaled by 1/8192, so the scores are those of the unscaled cache.  Every
    64-token tile is planted along the query direction with a maximum score
    of 10 or 17 log2 units, alternating in pairs of tiles: a later tile sits 7
    log2 units above an earlier one, within an 8-unit slack, where a
    probability of 2^7 times a group scale above 1024 would overflow fp16.
    Outputs compare after dividing by 8192."""
    H, D, R, Hq = 1, 512, 64, 16
    nb, lam = 40, 8192.0
    sigma, gain = (D + R) ** -0.5, 3.0
    rng = np.random.Generator(np.random.Philox(key=[77, 5]))
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    lat = rng.standard_normal((64 * nb, D)) * 0.05
    targets = []
    for j in range(nb):
        target = 10.0 + 7.0 * ((j // 2) % 2)                 # log2 units
        targets.append(target)
        beta = target / (sigma * gain * np.sqrt(D) * LOG2E)
        lat[64 * j:64 * j + 64] += beta * u
    k_src = [syn.bf16_bits((lat * lam).astype(np.float32)).reshape(64 * nb, 1, D)]
    rope = [syn.bf16_bits((rng.standard_normal((64 * nb, 1, R)) * 0.05).astype(np.float32))]
    b = build(H, D, [64 * nb], bits=[np.full(nb, 2, np.uint8)], latent=True, rope_dim=R, window=[0],
              k_src=k_src, rope=rope, seed=0)
    qz = gain * np.sqrt(D) * u[None, :] + rng.standard_normal((Hq, D)) * 0.01
    qr = rng.standard_normal((Hq, R)) * 0.01
    q = syn.bf16_bits((np.concatenate([qz, qr], axis=1) / lam).astype(np.float32))[None]
    # the planted structure, from the oracle's restored keys: group scales
    # above 1024 and tile maxima rising 6..8 log2 units over the tile before
    s = b.seq(0)
    kr = oracle.restore_seq(b.ref_pool, s["bits"], s["koff"], None, H, D).astype(np.float64).reshape(-1, D)
    qf = syn.bf16_to_f32(q[0]).astype(np.float64)
    sc = (qf[:, :D] @ kr.T + qf[:, D:] @ syn.bf16_to_f32(rope[0]).astype(np.float64).reshape(-1, R).T)
    tmax = (sc * sigma * LOG2E).reshape(Hq, nb, 64).max(axis=2)
    rises = tmax[:, 2::4] - tmax[:, 1::4]
    assert rises.min() > 6.0 and rises.max() < 8.0, (rises.min(), rises.max())
    # (scale, bias) fp16 pairs follow the 64 x 512 x 2 bits of codes
    scales = np.concatenate([b.ref_pool[int(o) + 8192:int(o) + 8192 + 2048].view(np.float16)[0::2]
                             for o in s["koff"]]).astype(np.float32)
    assert np.median(scales) > 1024.0, np.median(scales)
    got = _decode(b, q, sigma) / lam
    want = ref_decode(b, q, sigma) / lam
    close(got, want, what="mla large scales")
