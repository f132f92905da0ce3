"""GPU parity where the kernels' arithmetic is most stressed, against the
oracle at 2e-3 max-abs and 1e-3 relative L2 (the oracle's fp64 attention over
its own restored rows; QKVShare, Metodologia: restore, then ordinary
attention).

* Peaked attention.  Keys planted along the query direction make the largest
  score of each 64-key tile rise by more than 8 log2 units over every earlier
  tile of its period, so the kernels that keep their running maximum lazily
  (it moves only when a tile's maximum exceeds it by more than 8 log2 units)
  take the branch that rescales their accumulators, and the split merge
  combines partials whose maxima differ by tens of log2 units.  Each test
  asserts, from the oracle's restored keys, that such rises occur.
* Raw-code decode.  The decode for up to four query heads per KV head runs
  its products on the codes themselves; its weakest regime is 2- and 3-bit
  blocks, outlier key channels (wide groups) and large queries, and long
  splits (1024 tokens per split at the size below).
* Full-size chunk rows at the row-tile and causal boundaries.
"""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
from parity import build, close, ref_decode, to_dev_bf16

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
PERIOD, STEP, BASE = 8, 9.5, 20.0       # staircase of tile maxima, log2 units


def _unit_dirs(H, D, seed):
    u = np.random.Generator(np.random.Philox(key=[seed, 91])).standard_normal((H, D))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def _peaked_q(shape_lead, H, G, dirs, seed, gain=3.0, noise=0.3):
    """bf16 queries [..., H*G, D]: gain*sqrt(D)*u_g plus N(0, noise^2), so the
    G heads of KV head g share direction u_g."""
    D = dirs.shape[1]
    x = np.random.Generator(np.random.Philox(key=[seed, 92])).standard_normal(
        tuple(shape_lead) + (H * G, D)) * noise
    x += gain * np.sqrt(D) * np.repeat(dirs, G, axis=0)
    return syn.bf16_bits(x.astype(np.float32))


def _plant(k_bits, dirs, sigma, gain, n_tiles, seed):
    """Plant one key per 64-token tile j < n_tiles along u_g, with a score of
    about BASE + STEP*(j mod PERIOD) log2 units for every query head.
    k_bits bf16 [L][H][D'] (D' >= D: only the first D dims are set)."""
    L, H = k_bits.shape[0], k_bits.shape[1]
    D = dirs.shape[1]
    r = np.random.Generator(np.random.Philox(key=[seed, 93]))
    out = k_bits.copy()
    for j in range(min(n_tiles, L // 64)):
        t = 64 * j + int(r.integers(0, 64))
        target = BASE + STEP * (j % PERIOD)                  # log2 units
        lam = target / (sigma * gain * np.sqrt(D) * LOG2E)   # <q, lam u> ~ gain sqrt(D) lam
        out[t, :, :D] = syn.bf16_bits((lam * dirs).astype(np.float32))
    return out


def _tile_rises(scores_log2, valid):
    """Number of 64-key tiles whose max exceeds the max of every earlier tile
    of the same period by more than 8 (scores [heads][T])."""
    T = scores_log2.shape[1]
    n = 0
    for h in range(scores_log2.shape[0]):
        run = -np.inf
        for j in range((min(T, valid) + 63) // 64):
            if j % PERIOD == 0:
                run = -np.inf
            m = scores_log2[h, 64 * j:min(64 * j + 64, valid)].max()
            if run > -np.inf and m > run + 8.0:
                n += 1
            run = max(run, m)
    return n


def _oracle_scores(b, a, q_bits, scale, rope=None):
    """log2-domain scores [Hq][T] from the oracle's restored keys of sequence a."""
    s = b.seq(a)
    c = b.cache
    K = oracle.restore_seq(b.ref_pool, s["bits"], s["koff"], s["kw"], c.H, c.D)   # [T][H][D]
    q = syn.bf16_to_f32(q_bits).astype(np.float64)                               # [Hq][D(+R)]
    G = q.shape[0] // c.H
    R = None if rope is None else syn.bf16_to_f32(rope[:K.shape[0]]).astype(np.float64)   # [T][H][R]
    sc = np.zeros((q.shape[0], K.shape[0]))
    for h in range(q.shape[0]):
        g = h // G
        sc[h] = K[:, g, :].astype(np.float64) @ q[h, :c.D]
        if R is not None:
            sc[h] += R[:, g, :] @ q[h, c.D:]
    return sc * scale * LOG2E


def _decode(b, q_bits, scale):
    out = b.cache.attend_decode(to_dev_bf16(q_bits), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ---- peaked attention: running-max rescale -----------------------------------
@pytest.mark.parametrize("D,G", [(128, 4), (256, 2), (64, 1), (128, 8), (128, 16)])
def test_decode_peaked_staircase(D, G):
    H, A = 2, 2
    lengths = [64 * 40 + 70, 64 * 33]
    window = [70, 0]
    sigma, gain = D ** -0.5, 3.0
    dirs = _unit_dirs(H, D, D + G)
    k_src = [_plant(syn.random_normal_bf16((L, H, D), 300 + a), dirs, sigma, gain, L // 64, 40 + a)
             for a, L in enumerate(lengths)]
    rng = np.random.default_rng(D * G)
    # 4- and 8-bit blocks: narrower codes move a planted score by several log2
    # units, and the staircase needs steps above 8 in the restored keys
    bits = [rng.choice(np.array([4, 8], np.uint8), size=(L - w) // 64) for L, w in zip(lengths, window)]
    b = build(H, D, lengths, bits=bits, window=window, k_src=k_src, seed=D + G)
    q = _peaked_q((A,), H, G, dirs, 7 + G)
    for a in range(A):
        assert _tile_rises(_oracle_scores(b, a, q[a], sigma), lengths[a]) >= H * G * 20
    close(_decode(b, q, sigma), ref_decode(b, q, sigma), what=f"peaked decode D={D} G={G}")


def test_mla_peaked_staircase():
    """Latent cache (512 Q4 dims + 64 bf16 rope dims, 16 heads on one latent
    head); 300 and 260 blocks give splits of several tiles each."""
    H, D, R, Hq = 1, 512, 64, 16
    lengths = [64 * 300, 64 * 260 + 9]
    window = [0, 9]
    sigma, gain = 576 ** -0.5, 3.0
    dirs = _unit_dirs(H, D, 5120)
    k_src = [_plant(syn.random_normal_bf16((L, H, D), 400 + a), dirs, sigma, gain, L // 64, 50 + a)
             for a, L in enumerate(lengths)]
    b = build(H, D, lengths, latent=True, rope_dim=R, window=window, k_src=k_src, seed=55)
    qz = _peaked_q((2,), H, Hq, dirs, 61)                      # [2][16][512]
    rq = syn.random_normal_bf16((2, Hq, R), 62)
    q = np.concatenate([qz, rq], axis=2)
    for a in range(2):
        sc = _oracle_scores(b, a, q[a], sigma, rope=b.rope[a])
        assert _tile_rises(sc, lengths[a]) >= Hq * 200
    close(_decode(b, q, sigma), ref_decode(b, q, sigma), what="peaked mla")


def _chunk(b, qn, kn, vn, scale):
    out = b.cache.attend_chunk(to_dev_bf16(qn), to_dev_bf16(kn), to_dev_bf16(vn), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ref_chunk(b, a, qn, kn, vn, scale, rows=None):
    s = b.seq(a)
    c = b.cache
    r0, r1 = (0, qn.shape[0]) if rows is None else rows
    return oracle.attend_chunk_seq(b.ref_pool, s["bits"], s["koff"], s["voff"], s["kw"], s["vw"],
                                   c.H, c.D, qn, kn, vn, scale, r0, r1)


@pytest.mark.parametrize("D,G", [(64, 4), (128, 4), (256, 2)])
def test_chunk_peaked_staircase(D, G):
    H, A, n_new = 2, 1, 96
    lengths = [64 * 120 + 30]
    window = [30]
    sigma, gain = D ** -0.5, 3.0
    dirs = _unit_dirs(H, D, 700 + D)
    k_src = [_plant(syn.random_normal_bf16((lengths[0], H, D), 710 + D), dirs, sigma, gain, 120, 720 + D)]
    b = build(H, D, lengths, window=window, k_src=k_src, seed=D)
    qn = _peaked_q((A, n_new), H, G, dirs, 730 + D)
    kn = syn.random_normal_bf16((A, n_new, H, D), 731)
    vn = syn.random_normal_bf16((A, n_new, H, D), 732)
    for i in (0, n_new - 1):
        assert _tile_rises(_oracle_scores(b, 0, qn[0, i], sigma), lengths[0]) >= H * G * 90
    got = _chunk(b, qn, kn, vn, sigma)
    close(got[0], _ref_chunk(b, 0, qn[0], kn[0], vn[0], sigma), what=f"peaked chunk D={D} G={G}")


# ---- raw-code decode: narrow widths, outlier channels, large queries ----------
def _outlier_keys(L, H, D, seed, n_out=4, gain=10.0):
    r = np.random.Generator(np.random.Philox(key=[seed, 94]))
    x = r.standard_normal((L, H, D), dtype=np.float32)
    for h in range(H):
        x[:, h, r.choice(D, size=n_out, replace=False)] *= np.float32(gain)
    return syn.bf16_bits(x)


@pytest.mark.parametrize("D,G", [(128, 2), (128, 4), (256, 2), (256, 4)])
@pytest.mark.parametrize("widths", [(2,), (3,), (2, 3)])
def test_decode_narrow_widths_outliers(D, G, widths):
    H, A = 2, 3
    lengths = [64 * 30 + 5, 64 * 17 + 140, 64 * 41]
    window = [5, 140, 0]
    rng = np.random.default_rng(D + 10 * G + len(widths))
    bits = [rng.choice(np.array(widths, np.uint8), size=(L - w) // 64) for L, w in zip(lengths, window)]
    k_src = [_outlier_keys(L, H, D, 800 + a) for a, L in enumerate(lengths)]
    b = build(H, D, lengths, bits=bits, window=window, k_src=k_src, seed=D + G)
    q = syn.random_normal_bf16((A, H * G, D), 810 + G, scale=4.0)
    close(_decode(b, q, D ** -0.5), ref_decode(b, q, D ** -0.5), what=f"narrow {widths} D={D} G={G}")


def test_decode_long_splits_narrow_outliers():
    """4 sequences x 8 KV heads x 1024 blocks: the plan runs 16 blocks (1024
    tokens) per split, with 2- and 3-bit blocks, x10 outlier key channels and
    queries x4."""
    H, D, G, A, nb = 8, 128, 4, 4, 1024
    lengths = [64 * nb] * A
    rng = np.random.default_rng(1024)
    bits = [rng.choice(np.array([2, 3], np.uint8), size=nb) for _ in range(A)]
    k_src = [_outlier_keys(64 * nb, H, D, 900 + a) for a in range(A)]
    b = build(H, D, lengths, bits=bits, window=[0] * A, k_src=k_src, seed=91)
    q = syn.random_normal_bf16((A, H * G, D), 95, scale=4.0)
    close(_decode(b, q, D ** -0.5), ref_decode(b, q, D ** -0.5), what="long splits")


# ---- full-size chunk: rows at tile and causal boundaries ---------------------
def test_chunk_llama_32k_restore_512_boundary_rows():
    """Full 32768-token restore + 512-token causal chunk (the benchmark's
    launch); every 16th query row and the rows either side of the 64-row
    boundaries 64, 256 and 448, against the oracle."""
    w = syn.workload(3)
    b = build(w.n_kv_heads, w.head_dim, w.lengths, k_src=[w.kv(0, 0, syn.TAG_K)],
              v_src=[w.kv(0, 0, syn.TAG_V)])
    qn, kn, vn = w.chunk_new()
    got = _chunk(b, qn[None], kn[None], vn[None], w.scale)[0]
    rows = sorted(set(range(0, 512, 16)) | {1, 63, 64, 255, 256, 447, 448, 510, 511})
    for r in rows:
        want = _ref_chunk(b, 0, qn, kn, vn, w.scale, rows=(r, r + 1))
        close(got[r:r + 1], want[r:r + 1], what=f"chunk row {r}")
