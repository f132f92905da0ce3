"""GPU block sensitivity against the oracle (fp32 against fp64, 1e-5
relative), on raw K/V rows with outlier channels, then the budgeted widths
of the mixed-width workload's shape chosen from it."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
import quantized_kv_cache_group_amd as kvq
from parity import to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,D,G,q_offset", [(8, 128, 4, 0), (8, 256, 2, 0), (2, 64, 8, 0), (1, 512, 16, 0),
                                            (8, 512, 1, 0), (2, 128, 2, 1)])
def test_sensitivity_matches_oracle(H, D, G, q_offset):
    """(8, 512): per-block tables past 48 KB of LDS, and q_offset 1: a query
    not 16-byte aligned; both take the thread-per-row kernel."""
    A, nb = 3, 5
    T = 64 * nb + 17                                     # rows past the last block are ignored
    rng = np.random.default_rng(H * D)
    k = syn.bf16_to_f32(syn.random_normal_bf16((A, T, H, D), 1)).copy()
    k[:, :, :, rng.choice(D, 3, replace=False)] *= 8.0
    kb = syn.bf16_bits(k)
    vb = syn.random_normal_bf16((A, T, H, D), 2)
    q = syn.random_normal_bf16((A, G * H, D), 3)
    scale = D ** -0.5
    qd = to_dev_bf16(np.concatenate([np.zeros(q_offset, np.uint16), q.ravel()]))[q_offset:].view(q.shape)
    got = kvq.block_sensitivity(to_dev_bf16(kb), to_dev_bf16(vb), qd, scale, n_blocks=nb)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for a in range(A):
        for i in range(nb):
            want = oracle.block_sensitivity(kb[a, 64 * i:64 * i + 64], vb[a, 64 * i:64 * i + 64], H, D, q[a], scale)
            assert abs(got[a, i] - want) <= 1e-5 * want, (a, i, got[a, i], want)


def test_widths_for_mixed_workload_shape():
    """Sensitivities of one Gemma-shaped layer's blocks, widths for a mean
    of 3 bits: the host allocator gives the oracle's choice."""
    H, D, A, nb = 8, 256, 4, 12
    kb = syn.random_normal_bf16((A, 64 * nb, H, D), 4)
    vb = syn.random_normal_bf16((A, 64 * nb, H, D), 5)
    q = syn.random_normal_bf16((A, 2 * H, D), 6)
    S = kvq.block_sensitivity(to_dev_bf16(kb), to_dev_bf16(vb), to_dev_bf16(q), 1 / 16).cpu().numpy().ravel()
    budget = S.size * kvq.block_bytes(3, H, D)
    w = kvq.allocate_widths(S, H, D, budget)
    assert np.array_equal(w, oracle.allocate_widths(S.astype(np.float64), lambda b: kvq.block_bytes(b, H, D), budget))
