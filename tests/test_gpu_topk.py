"""GPU top-K sparse decode against the oracle.

The kept set is an integer decision taken from fp32 scores on the GPU and
fp64 scores in the oracle, so it is checked for validity: every kept block
scores (in the oracle) at least the K-th best minus the fp32 rounding
allowance, every dropped block at most the K-th best plus it, and the kept
indices are ascending and distinct.  The output must then equal the
oracle's decode over exactly the GPU's kept set (2e-3 max-abs, 1e-3 rel-L2),
and keeping every block must reproduce the full decode."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
from parity import build, close, ref_decode, to_dev_bf16

pytestmark = pytest.mark.gpu


def _check_selection(b, q, scale, K, sel):
    c = b.cache
    for a in range(c.A):
        s = b.seq(a)
        nb = c.n_blocks_host[a]
        rope = None if b.rope is None else b.rope[a][:64 * nb]
        sc = oracle.block_scores_seq(b.ref_pool, s["bits"], s["koff"], rope, c.H, c.D, q[a], scale)
        Kk = min(K, nb)
        got = sel[a, :Kk]
        assert np.all(sel[a, Kk:] == -1)
        assert np.all(np.diff(got) > 0) and (Kk == 0 or (got[0] >= 0 and got[-1] < nb))
        if Kk == 0 or Kk == nb:
            assert Kk == 0 or np.array_equal(got, np.arange(nb))
            continue
        # fp32 rounding allowance: |sum q k| error <= ~Dk * 2^-23 * sum |q||k|, times the scale
        kr = oracle.restore_seq(b.ref_pool, s["bits"], s["koff"], None, c.H, c.D).astype(np.float64)
        qf = np.abs(syn.bf16_to_f32(q[a]).astype(np.float64))
        bound = np.abs(kr).max() * qf.sum(axis=1).max() * abs(scale)
        if rope is not None:
            bound += np.abs(syn.bf16_to_f32(rope)).max() * qf.sum(axis=1).max() * abs(scale)
        tol = 64 * 2.0 ** -23 * bound + 1e-7
        G = q.shape[1] // c.H
        if rope is None and G <= 4 and c.D in (64, 128, 256):
            # scored by the decode's own products: sum_d q (1024 + code) accumulates in fp32
            # over 64 dims and 1024 Q_g is subtracted, an error of at most ~0.0088 sum|q| per
            # group, times the group's scale (<= 2 max|k|/3 at 2 bits) and the softmax scale
            qg = np.abs(syn.bf16_to_f32(q[a]).astype(np.float64)).reshape(q.shape[1], c.D // 64, 64).sum(axis=2)
            tol = max(tol, abs(scale) * (c.D // 64) * (2 * np.abs(kr).max() / 3) * 0.0088 * qg.max())
        kth = np.sort(sc)[::-1][Kk - 1]
        kept = np.zeros(nb, bool)
        kept[got] = True
        assert np.all(sc[kept] >= kth - tol), (a, sc[kept].min(), kth)
        assert np.all(sc[~kept] <= kth + tol), (a, sc[~kept].max(), kth)


def _ref_sparse(b, q, scale, sel):
    c = b.cache
    out = np.zeros((c.A, q.shape[1], c.D), np.float32)
    for a in range(c.A):
        s = b.seq(a)
        nb = c.n_blocks_host[a]
        idx = sel[a][sel[a] >= 0]
        rope = None
        if b.rope is not None:
            r = b.rope[a]
            rope = np.concatenate([r[64 * j:64 * j + 64] for j in idx] + [r[64 * nb:64 * nb + c.n_window_host[a]]])
        out[a] = oracle.attend_decode_seq(b.ref_pool, s["bits"][idx], s["koff"][idx],
                                          None if s["voff"] is None else s["voff"][idx], s["kw"], s["vw"], rope,
                                          c.H, c.D, q[a], scale)
    return out


def _run(b, q, scale, K):
    c = b.cache
    sel = torch.full((c.A, K), -7, dtype=torch.int32, device="cuda")
    out = c.attend_decode_topk(to_dev_bf16(q), scale, K, selected=sel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy()


@pytest.mark.parametrize("D,G,K", [(128, 4, 3), (128, 4, 1), (64, 8, 5), (256, 2, 4), (128, 16, 2)])
def test_topk_gqa(D, G, K):
    H = 2
    lengths = [64 * 12 + 40, 64 * 3 + 100, 64 * 20, 130]
    rng = np.random.default_rng(D + G)
    window = [40, 100, 0, 130]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    b = build(H, D, lengths, bits=bits, window=window, seed=D + G)
    q = syn.random_normal_bf16((4, G * H, D), 61 + K, scale=2.0)
    scale = D ** -0.5
    got, sel = _run(b, q, scale, K)
    _check_selection(b, q, scale, K, sel)
    close(got, _ref_sparse(b, q, scale, sel), what=f"topk D={D} G={G} K={K}")


def test_topk_all_blocks_is_full_decode():
    H, D = 8, 128
    b = build(H, D, [64 * 10 + 5, 64 * 7], window=[5, 0], seed=12)
    q = syn.random_normal_bf16((2, 32, D), 62)
    got, sel = _run(b, q, D ** -0.5, 10)
    assert np.array_equal(sel[0], np.arange(10)) and np.array_equal(sel[1], list(range(7)) + [-1] * 3)
    close(got, ref_decode(b, q, D ** -0.5), what="topk = all")


def test_topk_latent_rope():
    H, D, R, Hq = 1, 512, 64, 16
    lengths = [64 * 30 + 20, 64 * 9]
    b = build(H, D, lengths, latent=True, rope_dim=R, window=[20, 0], seed=13)
    q = syn.random_normal_bf16((2, Hq, D + R), 63, scale=2.0)
    scale = 576 ** -0.5
    got, sel = _run(b, q, scale, 6)
    _check_selection(b, q, scale, 6, sel)
    close(got, _ref_sparse(b, q, scale, sel), what="topk latent+rope")


@pytest.mark.parametrize("G", [4, 16])
def test_topk_latent_rope_kept_rows_in_place(G):
    """The latent route reads the kept blocks' rope rows where they lie (at
    the selected block's position, and the window's after the sequence's full
    block count): sequences with fewer blocks than K (all kept, window after
    them), none (window only), K of many with a window, and K of many without
    one; 2-, 3-, 4- and 8-bit latents mixed."""
    H, D, R = 1, 512, 64
    lengths = [64 * 3 + 10, 40, 64 * 25 + 33, 64 * 18]
    window = [10, 40, 33, 0]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [np.array([(2, 3, 4, 8)[(a + j) % 4] for j in range(n)], np.uint8) for a, n in enumerate(nb)]
    b = build(H, D, lengths, bits=bits, window=window, latent=True, rope_dim=R, seed=97 + G)
    q = syn.random_normal_bf16((len(lengths), G, D + R), 98 + G, scale=2.0)
    scale = (D + R) ** -0.5
    got, sel = _run(b, q, scale, 5)
    _check_selection(b, q, scale, 5, sel)
    close(got, _ref_sparse(b, q, scale, sel), what=f"topk latent rope in place G={G}")


def test_topk_many_blocks_per_thread():
    """More blocks than the selection's 256 threads (several blocks per
    thread in the scans), mixed widths, one short sequence."""
    H, D, G, K = 2, 64, 4, 37
    lengths = [64 * 600, 64 * 300 + 17, 64 * 20]
    window = [0, 17, 0]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    rng = np.random.default_rng(71)
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) for n in nb]
    b = build(H, D, lengths, bits=bits, window=window, seed=71)
    q = syn.random_normal_bf16((3, G * H, D), 72, scale=2.0)
    scale = D ** -0.5
    got, sel = _run(b, q, scale, K)
    _check_selection(b, q, scale, K, sel)
    close(got, _ref_sparse(b, q, scale, sel), what="topk 600 blocks")


@pytest.mark.parametrize("n_blocks,K,G,D", [(8, 3, 4, 128), (256, 100, 4, 64), (300, 100, 4, 64), (300, 100, 8, 64), (520, 257, 2, 256)])
def test_topk_ties_keep_lowest_indices(n_blocks, K, G, D):
    """Every block holds the same keys, so every score ties exactly (the same
    arithmetic on the same bytes): the kept set must be blocks 0..K-1."""
    H = 2
    blk = syn.random_normal_bf16((64, H, D), 73)
    k = np.tile(blk, (n_blocks, 1, 1))
    v = syn.random_normal_bf16((64 * n_blocks, H, D), 74)
    b = build(H, D, [64 * n_blocks], window=[0], k_src=[k], v_src=[v], seed=73)
    q = syn.random_normal_bf16((1, G * H, D), 75)
    scale = D ** -0.5
    got, sel = _run(b, q, scale, K)
    assert np.array_equal(sel[0], np.arange(K)), sel[0][:10]
    close(got, _ref_sparse(b, q, scale, sel), what=f"topk ties {n_blocks}/{K}")


@pytest.mark.parametrize("nb,K,D,H,G", [(1300, 400, 64, 1, 4), (2100, 1100, 64, 2, 2)])
def test_topk_long_runs_per_thread(nb, K, D, H, G):
    """Over 1 024 blocks per sequence: each selection thread owns runs of more
    than four blocks, past the table entries it loads ahead."""
    rng = np.random.default_rng(nb)
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=nb)]
    b = build(H, D, [64 * nb], bits=bits, window=[0], seed=nb)
    q = syn.random_normal_bf16((1, G * H, D), 76, scale=2.0)
    scale = D ** -0.5
    got, sel = _run(b, q, scale, K)
    _check_selection(b, q, scale, K, sel)
    close(got, _ref_sparse(b, q, scale, sel), what=f"topk {nb} blocks")


def test_topk_window_only_null_tables():
    """A window-only layout through the C ABI with null widths, offsets and
    pools: no block is kept, `selected` is all -1, and the output is the
    decode over the windows."""
    import ctypes
    import quantized_kv_cache_group_amd as kvq
    A, H, D, G, K, cap = 2, 2, 128, 4, 3, 100
    nw = [100, 37]
    kw = [syn.random_normal_bf16((n, H, D), 80 + a) for a, n in enumerate(nw)]
    vw = [syn.random_normal_bf16((n, H, D), 90 + a) for a, n in enumerate(nw)]
    kwin = torch.zeros((A, cap, H, D), dtype=torch.bfloat16, device="cuda")
    vwin = torch.zeros_like(kwin)
    for a in range(A):
        kwin[a, :nw[a]] = to_dev_bf16(kw[a])
        vwin[a, :nw[a]] = to_dev_bf16(vw[a])
    n_blocks = torch.zeros(A, dtype=torch.int32, device="cuda")
    n_window = torch.tensor(nw, dtype=torch.int32, device="cuda")
    L = kvq.Layout(n_seqs=A, n_heads=H, head_dim=D, max_blocks=0, window_cap=cap,
                   n_blocks=n_blocks.data_ptr(), n_window=n_window.data_ptr(), bits=None)
    Ks = kvq.Store(offset=None, pool=None, window=kwin.data_ptr())
    Vs = kvq.Store(offset=None, pool=None, window=vwin.data_ptr())
    q = syn.random_normal_bf16((A, G * H, D), 81)
    qd = to_dev_bf16(q)
    out = torch.full((A, G * H, D), 7.0, dtype=torch.float32, device="cuda")
    sel = torch.full((A, K), 5, dtype=torch.int32, device="cuda")
    n = ctypes.c_size_t(0)
    lib = kvq.lib()
    assert lib.kvq_topk_workspace(ctypes.byref(L), G * H, 0, K, ctypes.byref(n)) == 0
    ws = torch.zeros(n.value, dtype=torch.uint8, device="cuda")
    scale = D ** -0.5
    st = lib.kvq_attend_decode_topk(ctypes.byref(L), ctypes.byref(Ks), ctypes.byref(Vs), None, 0,
                                    qd.data_ptr(), G * H, scale, K, out.data_ptr(), sel.data_ptr(),
                                    ws.data_ptr(), n.value, None)
    assert st == 0, kvq.lib().kvq_strerror(st)
    torch.cuda.synchronize()
    assert np.all(sel.cpu().numpy() == -1)
    got = out.cpu().numpy()
    for a in range(A):
        want = oracle.attend_decode_seq(np.zeros(256, np.uint8), np.zeros(0, np.uint8), np.zeros(0, np.uint64),
                                        np.zeros(0, np.uint64), kw[a], vw[a], None, H, D, q[a], scale)
        close(got[a], want, what=f"window-only topk a={a}")
