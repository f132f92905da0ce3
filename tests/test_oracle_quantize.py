"""Pins of the oracle's quantizer, packer and block layout.

The pages name the format (quantized KV groups, 4-bit "Q4", mixed widths)
but print no formula or worked code, so these tests pin the oracle to what
mathematics and the pages' printed figures fix:
  * reconstruction error at most half a step (plus stated rounding slack);
  * exact round trip of values already on a quantization grid;
  * constant groups, monotone codes, endpoint codes;
  * fp16 metadata equal to numpy's IEEE float32 arithmetic then float16 cast;
  * bijective packing and hand-derived bit positions (tests/golden);
  * block layout at the documented byte addresses;
  * packed size against the ratios the pages print (tests/golden).
"""
import json
import os

import numpy as np
import pytest

import kvq_synth as syn

GOLD = os.path.join(os.path.dirname(__file__), "golden")
WIDTHS = (2, 3, 4, 8)


def _groups(seed):
    """A mix of value distributions, as bf16 bit patterns [n][64]."""
    r = np.random.default_rng(seed)
    out = [
        r.standard_normal((300, 64)).astype(np.float32),
        (r.standard_normal((100, 64)) * 10.0).astype(np.float32),
        r.uniform(-1000, 1000, (100, 64)).astype(np.float32),
        r.uniform(0.5, 0.75, (100, 64)).astype(np.float32),        # narrow range, offset
        r.uniform(-60000, 60000, (30, 64)).astype(np.float32),     # near the fp16 limit
        (r.standard_normal((100, 64)) * 1e-3).astype(np.float32),
    ]
    x = np.concatenate(out)
    # outlier channels as in a key cache
    x[:50, 3] *= 10.0
    return syn.bf16_bits(x)


def _f32(h):
    return syn.bf16_to_f32(h)


def _h2f(h):
    return np.array([h], np.uint16).view(np.float16).astype(np.float32)[0]


@pytest.mark.parametrize("bits", WIDTHS)
def test_reconstruction_within_half_step(ref, bits):
    """Every element: |x_hat - x| <= s_h/2 + s_h*2^-14 + 2^-23*max(|x|,|x_hat|),
    for groups whose min is an fp16 value and whose step is an fp16 normal."""
    G = _groups(bits)
    n_checked = 0
    for g in G:
        w, sh, bh = ref.quantize_group(g, bits)
        x = _f32(g).astype(np.float64)
        xh = ref.dequantize_group(w, bits, sh, bh).astype(np.float64)
        s = float(_h2f(sh))
        if not (s >= 2.0 ** -14 and float(_h2f(bh)) == x.min()):
            continue
        bound = s / 2 + s * 2.0 ** -14 + 2.0 ** -23 * np.maximum(np.abs(x), np.abs(xh))
        assert np.all(np.abs(xh - x) <= bound), (bits, np.max(np.abs(xh - x) - bound))
        n_checked += 1
    assert n_checked > 600


@pytest.mark.parametrize("bits", WIDTHS)
def test_tiny_groups_bounded(ref, bits):
    """Groups in the fp16 subnormal range: the stored step/bias carry at most
    half an fp16 subnormal unit each; the error stays within that slack."""
    r = np.random.default_rng(10 + bits)
    n = (1 << bits) - 1
    for _ in range(200):
        x = syn.bf16_bits((r.standard_normal(64) * 10.0 ** r.uniform(-9, -5)).astype(np.float32))
        w, sh, bh = ref.quantize_group(x, bits)
        xf = _f32(x).astype(np.float64)
        xh = ref.dequantize_group(w, bits, sh, bh).astype(np.float64)
        s = float(_h2f(sh))
        s_true = (xf.max() - xf.min()) / n
        slack = s / 2 + n * abs(s_true - s) + 2.0 ** -25 + 2.0 ** -23 * np.abs(xf).max() + 1e-12
        assert np.all(np.abs(xh - xf) <= slack)


@pytest.mark.parametrize("bits", WIDTHS)
def test_metadata_is_ieee_fp32_then_fp16(ref, bits):
    n = np.float32((1 << bits) - 1)
    for g in _groups(100 + bits)[::3]:
        x = _f32(g)
        _, sh, bh = ref.quantize_group(g, bits)
        with np.errstate(over="ignore"):
            s = (x.max() - x.min()) / n                          # numpy float32: IEEE RNE
            want_s = np.float16(s).view(np.uint16)
            want_b = np.float16(x.min() + np.float32(0)).view(np.uint16)
        assert sh == int(want_s)
        assert bh == int(want_b)


@pytest.mark.parametrize("bits", WIDTHS)
def test_grid_round_trip(ref, bits):
    """x_i = beta + q_i * 2^-k with both end codes present: codes == q_i and
    the dequantized values equal x bit for bit."""
    n = (1 << bits) - 1
    r = np.random.default_rng(7 * bits)
    for trial in range(200):
        k = int(r.integers(1, 6))
        lo = -255 if bits == 8 else -120
        hi = 0 if bits == 8 else 120
        m = int(r.integers(lo, hi + 1))
        if m == 0 and trial % 2:
            m = -1
        q = r.integers(0, n + 1, 64)
        q[r.integers(0, 64)] = 0
        q[r.integers(0, 64)] = n
        if q.min() != 0:
            q[q.argmin()] = 0
        x = ((m + q) * 2.0 ** -k).astype(np.float32)
        xb = syn.bf16_bits(x)
        assert np.array_equal(_f32(xb), x)                           # bf16-exact by construction
        w, sh, bh = ref.quantize_group(xb, bits)
        assert np.array_equal(ref.unpack_group(w, bits), q.astype(np.uint8))
        xh = ref.dequantize_group(w, bits, sh, bh)
        assert np.array_equal(xh.view(np.uint32), (x + np.float32(0)).view(np.uint32))


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("c", [0.0, -0.0, 1.5, -3.25, 1000.0, 2.0 ** -20])
def test_constant_group(ref, bits, c):
    xb = syn.bf16_bits(np.full(64, c, np.float32))
    w, sh, bh = ref.quantize_group(xb, bits)
    assert sh == 0
    assert np.all(ref.unpack_group(w, bits) == 0)
    assert bh == int(np.float16(np.float32(c) + np.float32(0)).view(np.uint16))
    xh = ref.dequantize_group(w, bits, sh, bh)
    assert np.all(xh == np.float32(np.float16(c)))


def test_mixed_signed_zero_bias_is_positive(ref):
    x = np.zeros(64, np.float32)
    x[5] = -0.0
    x[9] = 1.0
    _, _, bh = ref.quantize_group(syn.bf16_bits(x), 4)
    assert bh == 0


@pytest.mark.parametrize("bits", WIDTHS)
def test_codes_monotone_and_endpoints(ref, bits):
    n = (1 << bits) - 1
    for g in _groups(200 + bits)[::2]:
        x = _f32(g)
        w, sh, _ = ref.quantize_group(g, bits)
        c = ref.unpack_group(w, bits).astype(int)
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(c[order]) >= 0)
        if sh != 0 and _h2f(sh) >= 2.0 ** -14:
            assert c[np.argmin(x)] == 0
            assert c[np.argmax(x)] == n


@pytest.mark.parametrize("bits", WIDTHS)
def test_pack_bijection(ref, bits):
    r = np.random.default_rng(bits)
    for _ in range(50):
        c = r.integers(0, 1 << bits, 64).astype(np.uint8)
        w = ref.pack_group(c, bits)
        assert w.size == 2 * bits
        assert np.array_equal(ref.unpack_group(w, bits), c)
    # closed forms of the little-endian stream for the byte-aligned widths
    c = r.integers(0, 256, 64).astype(np.uint8)
    assert np.array_equal(ref.pack_group(c, 8).view(np.uint8), c)
    c4 = r.integers(0, 16, 64).astype(np.uint8)
    want = (c4[0::2] | (c4[1::2] << 4)).astype(np.uint8)
    assert np.array_equal(ref.pack_group(c4, 4).view(np.uint8), want)
    c2 = r.integers(0, 4, 64).astype(np.uint8)
    want = (c2[0::4] | (c2[1::4] << 2) | (c2[2::4] << 4) | (c2[3::4] << 6)).astype(np.uint8)
    assert np.array_equal(ref.pack_group(c2, 2).view(np.uint8), want)


def test_pack_b3_straddle_positions(ref):
    gold = json.load(open(os.path.join(GOLD, "pack_b3_straddle.json")))
    for idx, places in gold["codes"].items():
        i = int(idx)
        for code in range(8):
            c = np.zeros(64, np.uint8)
            c[i] = code
            w = ref.pack_group(c, 3)
            want = np.zeros(6, np.uint32)
            for p in places:
                if code >> p["code_bit"] & 1:
                    want[p["word"]] |= np.uint32(1) << np.uint32(p["bit"])
            assert np.array_equal(w, want), (i, code)


def test_block_layout_addresses(ref):
    """Meta of (h, token r, group g) sits at
    H*64*D*b/8 + ((h*64 + r)*(D/64) + g)*4 (scale then bias); codes of that
    group start at (h*64 + r)*(D*b/8) + g*8b."""
    H, D = 2, 128
    ng = D // 64
    bits = np.array([3, 8], np.uint8)
    off, total = ref.packed_offsets(bits, H, D)
    assert off[1] % 256 == 0 and off[1] == ref.block_bytes(3, H, D)
    x = np.zeros((128, H, D), np.float32)
    for j in range(2):
        for h in range(H):
            for r in range(64):
                for g in range(ng):
                    uid = (h * 64 + r) * ng + g                # 0..255, bf16/fp16 exact
                    grp = np.full(64, float(uid), np.float32)
                    grp[uid % 64] = uid + 1.0 if uid < 255 else 254.0
                    x[j * 64 + r, h, g * 64:(g + 1) * 64] = grp
    xb = syn.bf16_bits(x)
    pool = np.zeros(total, np.uint8)
    ref.quantize_seq(xb, H, D, bits, off, pool)
    for j, b in enumerate(bits):
        n = (1 << int(b)) - 1
        blk = pool[int(off[j]):]
        codes_total = H * 64 * D * int(b) // 8
        for h in range(H):
            for r in range(64):
                for g in range(ng):
                    uid = (h * 64 + r) * ng + g
                    m = codes_total + ((h * 64 + r) * ng + g) * 4
                    sh, bh = blk[m:m + 4].view(np.uint16)
                    lo = min(uid, 254) if uid == 255 else uid
                    assert _h2f(bh) == lo
                    c0 = (h * 64 + r) * (D * int(b) // 8) + g * 8 * int(b)
                    w = blk[c0:c0 + 8 * int(b)].view(np.uint32)
                    codes = ref.unpack_group(w, int(b))
                    hot = uid % 64
                    assert codes[hot] == (n if uid < 255 else 0)
                    assert np.all(np.delete(codes, hot) == (0 if uid < 255 else n))


def test_restore_concatenates_window(ref):
    H, D = 1, 64
    bits = np.array([4], np.uint8)
    off, total = ref.packed_offsets(bits, H, D)
    x = syn.random_normal_bf16((64, H, D), 3)
    win = syn.random_normal_bf16((5, H, D), 4)
    pool = np.zeros(total, np.uint8)
    ref.quantize_seq(x, H, D, bits, off, pool)
    out = ref.restore_seq(pool, bits, off, win, H, D)
    assert out.shape == (69, H, D)
    assert np.array_equal(out[64:], syn.bf16_to_f32(win))


# ---- size arithmetic against the pages' printed figures ---------------------
def test_size_ratio_matches_printed_q4(ref):
    gold = json.load(open(os.path.join(GOLD, "size_claims.json")))
    for H, D in [(8, 128), (8, 256), (1, 512), (2, 64)]:
        bf16 = 64 * H * D * 2
        r4 = ref.block_bytes(4, H, D) / bf16
        assert r4 == 4.5 / 16
        assert round(100 * r4, 1) == gold["q4_0_size_pct_of_bf16"]["value"]
        for b in WIDTHS:
            assert ref.block_bytes(b, H, D) / bf16 == (b + 0.5) / 16
    # the printed 5.5-bit figure follows the same (bits + metadata)/16 rule
    assert round(100 * gold["q5_0_size_pct_of_bf16"]["bits_per_element"] / 16, 1) == \
        gold["q5_0_size_pct_of_bf16"]["value"]
    # codes alone: 16 / 4 = 4x more contexts than 16-bit
    assert 16 // 4 == gold["q4_capacity_vs_fp16"]["value"]


def test_capacity_arithmetic_gemma(ref):
    gold = json.load(open(os.path.join(GOLD, "size_claims.json")))["fp16_agents_in_budget"]
    layers, H, D, T = 48, 8, 256, gold["context_tokens"]
    fp16_per_agent = layers * 2 * H * D * 2 * T
    assert fp16_per_agent == 3_221_225_472
    budget = gold["budget_gb"] * 1e9
    assert int(budget // fp16_per_agent) == gold["value"]
    q4_per_agent = layers * 2 * (T // 64) * ref.block_bytes(4, H, D)
    assert q4_per_agent == 905_969_664
    assert 10 * q4_per_agent <= budget                 # the 10-agent workflow fits in Q4


def test_unsupported_widths(ref):
    assert ref.block_bytes(5, 8, 128) == 0
    assert ref.block_bytes(4, 8, 100) == 0
    with pytest.raises(ValueError):
        ref.quantize_group(np.zeros(64, np.uint16), 5)
