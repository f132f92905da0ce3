"""Decode and chunk calls captured in a HIP graph (through torch's graph
capture on the caller's stream) and replayed: the library's calls allocate
nothing, clear nothing and keep no state, so every replay must equal the
eager call bit for bit.  Three replays, with eager work between them that
overwrites the output (and, for the static decode, the library's shared
scratch through an eager call over another cache)."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
from parity import build, to_dev_bf16

pytestmark = pytest.mark.gpu


def _mixed(n_blocks, seed):
    rng = np.random.default_rng(seed)
    return [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in n_blocks]


def _replays_match(call, out, want, between=None):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                   # warm once outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        out.fill_(float("nan"))
        if between is not None:
            between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("D,G", [(128, 4), (256, 2), (128, 8)])
def test_graph_decode(D, G):
    H = 2
    n_blocks, window = [9, 3, 0, 14], [40, 129, 17, 0]
    lengths = [64 * n + w for n, w in zip(n_blocks, window)]
    b = build(H, D, lengths, bits=_mixed(n_blocks, D + G), window=window, seed=900 + G)
    c = b.cache
    q = to_dev_bf16(syn.random_normal_bf16((4, G * H, D), 901))
    ws = torch.empty(max(c.decode_workspace_bytes(G * H), 256), dtype=torch.uint8, device="cuda")
    want = c.attend_decode(q, D ** -0.5, workspace=ws).clone()
    out = torch.empty_like(want)
    _replays_match(lambda: c.attend_decode(q, D ** -0.5, out=out, workspace=ws), out, want)


def test_graph_mla_decode():
    D, R, Hq = 512, 64, 16
    n_blocks, window = [12, 5], [30, 0]
    lengths = [64 * n + w for n, w in zip(n_blocks, window)]
    b = build(1, D, lengths, bits=_mixed(n_blocks, 7), latent=True, rope_dim=R, window=window, seed=910)
    c = b.cache
    q = to_dev_bf16(syn.random_normal_bf16((2, Hq, D + R), 911, scale=2.0))
    s = (D + R) ** -0.5
    ws = torch.empty(max(c.decode_workspace_bytes(Hq), 256), dtype=torch.uint8, device="cuda")
    want = c.attend_decode(q, s, workspace=ws).clone()
    out = torch.empty_like(want)
    _replays_match(lambda: c.attend_decode(q, s, out=out, workspace=ws), out, want)


def test_graph_static_decode_with_eager_calls_between():
    H, D, G = 2, 128, 4
    n_blocks, window = [20, 7], [65, 3]
    lengths = [64 * n + w for n, w in zip(n_blocks, window)]
    b = build(H, D, lengths, bits=_mixed(n_blocks, 3), window=window, seed=920)
    c = b.cache
    q = to_dev_bf16(syn.random_normal_bf16((2, G * H, D), 921))
    want = c.attend_decode_static(q, D ** -0.5).clone()
    other = build(H, D, [64 * 30 + 5], seed=922).cache
    q_other = to_dev_bf16(syn.random_normal_bf16((1, G * H, D), 923))
    out = torch.empty_like(want)
    _replays_match(lambda: c.attend_decode_static(q, D ** -0.5, out=out), out, want,
                   between=lambda: other.attend_decode_static(q_other, D ** -0.5))


@pytest.mark.parametrize("D", [128, 256])
def test_graph_chunk(D):
    H, G, n_new = 2, 2, 40
    n_blocks, window = [6, 0], [33, 10]
    lengths = [64 * n + w for n, w in zip(n_blocks, window)]
    b = build(H, D, lengths, bits=_mixed(n_blocks, D), window=window, seed=930)
    c = b.cache
    qn = to_dev_bf16(syn.random_normal_bf16((2, n_new, G * H, D), 931))
    kn = to_dev_bf16(syn.random_normal_bf16((2, n_new, H, D), 932))
    vn = to_dev_bf16(syn.random_normal_bf16((2, n_new, H, D), 933))
    ws = torch.empty(max(c.chunk_workspace_bytes(G * H, n_new), 256), dtype=torch.uint8, device="cuda")
    want = c.attend_chunk(qn, kn, vn, D ** -0.5, workspace=ws).clone()
    out = torch.empty_like(want)
    _replays_match(lambda: c.attend_chunk(qn, kn, vn, D ** -0.5, out=out, workspace=ws), out, want)
