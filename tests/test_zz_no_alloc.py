"""kvq_attend_decode_static (the decode for callers that cannot allocate:
split partials in the library's own device array) against kvq_attend_decode
with a caller workspace, on two calls in a row, the second over a smaller
cache, through the C ABI.  Both run the same kernels, so the outputs must
agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import kvq_synth as syn
from parity import build, close, ref_decode, to_dev_bf16

pytestmark = pytest.mark.gpu


def _both(b, q_bits, scale):
    c = b.cache
    q = to_dev_bf16(q_bits)
    ws = torch.empty(max(c.decode_workspace_bytes(q.shape[1]), 256), dtype=torch.uint8, device="cuda")
    want = c.attend_decode(q, scale, workspace=ws)
    got = torch.full_like(want, float("nan"))
    c.attend_decode_static(q, scale, out=got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), want.cpu().numpy()


def test_static_decode_matches_workspace_decode_twice():
    # first call: Gemma-like head_dim 256, mixed widths and windows, 4 agents
    rng = np.random.default_rng(5)
    H, D, G = 4, 256, 2
    lengths = [64 * 40 + 150, 64 * 25 + 130, 64 * 61 + 129, 64 * 7 + 140]
    window = [150, 130, 129, 140]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=(L - w) // 64) for L, w in zip(lengths, window)]
    b1 = build(H, D, lengths, bits=bits, window=window, seed=501)
    q1 = syn.random_normal_bf16((4, G * H, D), 502)
    got, want = _both(b1, q1, D ** -0.5)
    assert np.array_equal(got, want)
    close(got, ref_decode(b1, q1, D ** -0.5), what="static call 1")
    # second call, smaller: Llama-like head_dim 128, 2 agents, fewer blocks
    H, D, G = 2, 128, 4
    lengths = [64 * 9 + 3, 64 * 4]
    b2 = build(H, D, lengths, keep_recent=3, seed=503)
    q2 = syn.random_normal_bf16((2, G * H, D), 504)
    got, want = _both(b2, q2, D ** -0.5)
    assert np.array_equal(got, want)
    close(got, ref_decode(b2, q2, D ** -0.5), what="static call 2")


def test_static_decode_rejects_oversized_call():
    import quantized_kv_cache_group_amd as kvq
    # a layout whose workspace exceeds the 16 MiB scratch: ENOSPC, nothing launched
    c = kvq.LayerCache(2, 64, [16] * 512, [0] * 512, [np.full(16, 4, np.uint8)] * 512)
    assert c.decode_workspace_bytes(32) > 16 << 20
    q = torch.zeros((512, 32, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvq.KVQError) as e:
        c.attend_decode_static(q, 0.1)
    assert e.value.status == kvq.KVQ_ENOSPC
