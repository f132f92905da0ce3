"""kvq_append_counts (host copy of the counts kvq_append leaves) against the
oracle's window roll: for window + new token streams that fit, the counts
equal those kvq_ref_append_seq produces; argument checks on the host."""
import ctypes
import os

import numpy as np
import pytest

import kvq_synth as syn
import oracle
import quantized_kv_cache_group_amd as kvq

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")


def _counts(nb, nw, n_new, keep, max_blocks, window_cap):
    A = len(nb)
    nbh = np.ascontiguousarray(nb, np.int32)
    nwh = np.ascontiguousarray(nw, np.int32)
    nbo = np.zeros(A, np.int32)
    nwo = np.zeros(A, np.int32)
    vp = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    st = kvq.lib().kvq_append_counts(A, max_blocks, window_cap, vp(nbh), vp(nwh), n_new, keep, vp(nbo), vp(nwo))
    return st, nbo, nwo


def _oracle_counts(nb, nw, n_new, keep, max_blocks, window_cap, seed):
    H, D = 1, 64
    bits = np.full(max_blocks, 4, np.uint8)
    off, tot = oracle.packed_offsets(bits, H, D)
    kp, vp_ = np.zeros(max(tot, 256), np.uint8), np.zeros(max(tot, 256), np.uint8)
    kw = np.zeros((max(window_cap, 1), H, D), np.uint16)
    vw = np.zeros_like(kw)
    kw[:nw] = syn.random_normal_bf16((nw, H, D), seed)
    vw[:nw] = syn.random_normal_bf16((nw, H, D), seed + 1)
    kn = syn.random_normal_bf16((n_new, H, D), seed + 2)
    vn = syn.random_normal_bf16((n_new, H, D), seed + 3)
    return oracle.append_seq(kp, vp_, bits, off, off, nb, kw[:window_cap] if window_cap else None,
                             vw[:window_cap] if window_cap else None, nw, H, D, kn, vn, keep)


def test_counts_match_oracle_window_roll():
    rng = np.random.default_rng(17)
    checked = 0
    for case in range(300):
        keep = int(rng.choice([0, 1, 64, 128, 200]))
        window_cap = keep + 63 + int(rng.integers(0, 40))
        max_blocks = int(rng.integers(1, 30))
        n_new = int(rng.integers(0, 400))
        nb = int(rng.integers(0, max_blocks + 1))
        nw = int(rng.integers(0, window_cap + 1))
        T = nw + n_new
        k = (T - keep) // 64 if T > keep else 0
        if nb + k > max_blocks:                 # does not fit: the oracle refuses it
            continue
        want = _oracle_counts(nb, nw, n_new, keep, max_blocks, window_cap, 1000 + case)
        st, nbo, nwo = _counts([nb], [nw], n_new, keep, max_blocks, window_cap)
        assert st == 0 and (int(nbo[0]), int(nwo[0])) == want, (nb, nw, n_new, keep, want, nbo, nwo)
        checked += 1
    assert checked > 150


def test_counts_without_window():
    st, nbo, _ = _counts([3, 0], [0, 0], 128, 0, 10, 0)
    assert st == 0 and list(nbo) == [5, 2]
    assert oracle.append_seq(np.zeros(4096 * 10, np.uint8), None, np.full(10, 4, np.uint8),
                             oracle.packed_offsets(np.full(10, 4, np.uint8), 1, 64)[0], None, 3, None, None, 0,
                             1, 64, syn.random_normal_bf16((128, 1, 64), 5), None, 0) == (5, 0)


def test_counts_clamp_like_the_kernels():
    # a result past max_blocks keeps the blocks that fit (the kernels write no more)
    st, nbo, nwo = _counts([9], [150], 300, 128, 10, 191)
    assert st == 0 and int(nbo[0]) == 10 and int(nwo[0]) == 191


@pytest.mark.parametrize("args", [
    dict(n_new=-1), dict(keep=-1), dict(keep=129), dict(window_cap=0, keep=0, n_new=5),
])
def test_counts_reject(args):
    d = dict(nb=[0], nw=[0], n_new=10, keep=128, max_blocks=4, window_cap=191)
    d.update(args)
    st, _, _ = _counts(d["nb"], d["nw"], d["n_new"], d["keep"], d["max_blocks"], d["window_cap"])
    assert st == kvq.KVQ_EINVAL
