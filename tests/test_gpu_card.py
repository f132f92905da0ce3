"""GPU CacheCards: the gathered image equals the oracle's image byte for
byte; a card saved to a file and restored into a fresh batched cache gives
back the same restored rows (bit-exact) and the same attention (against the
oracle); loading into an existing cache's matching slots round-trips."""
import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
import quantized_kv_cache_group_amd as kvq
from quantized_kv_cache_group_amd import card
from parity import build, close, ref_decode, to_dev_bf16

pytestmark = pytest.mark.gpu


def _oracle_image(b, a):
    s = b.seq(a)
    c = b.cache
    nb, nw = c.n_blocks_host[a], c.n_window_host[a]
    kw = s["kw"] if nw else np.zeros((0, c.H, c.D), np.uint16)
    vw = None if c.latent else (s["vw"] if nw else np.zeros((0, c.H, c.D), np.uint16))
    rope = None if b.rope is None else b.rope[a][:64 * nb + nw]
    return oracle.card_image(b.ref_pool, s["bits"], s["koff"], s["voff"], kw, vw, rope, c.H, c.D)


def _dequant(c):
    out = torch.zeros((c.A, 64 * c.max_blocks + c.window_cap, c.H, c.D), dtype=torch.float32, device="cuda")
    c.dequantize("k", out)
    k = out.cpu().numpy()
    v = None
    if not c.latent:
        out.zero_()
        c.dequantize("v", out)
        v = out.cpu().numpy()
    return k, v


CASES = [dict(H=2, D=128, lengths=[64 * 5 + 150, 64 * 2 + 10, 130], mixed=True),
         dict(H=1, D=512, lengths=[64 * 6 + 9, 64 * 3 + 100], latent=True, R=64),
         dict(H=8, D=64, lengths=[64 * 4, 200], mixed=False)]


@pytest.mark.parametrize("case", CASES)
def test_gather_matches_oracle_image(case):
    rng = np.random.default_rng(case["D"])
    lengths = case["lengths"]
    window = [L - 64 * (max(L - 128, 0) // 64) for L in lengths]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) if case.get("mixed") else np.full(n, 4, np.uint8)
            for n in nb]
    b = build(case["H"], case["D"], lengths, bits=bits, window=window, latent=case.get("latent", False),
              rope_dim=case.get("R", 0), seed=case["D"])
    for a in range(len(lengths)):
        img = b.cache.card_gather(a).cpu().numpy()
        want = _oracle_image(b, a)
        assert img.size == want.size and np.array_equal(img, want), f"sequence {a}"


@pytest.mark.parametrize("case", CASES)
def test_save_restore_batched(case, tmp_path):
    rng = np.random.default_rng(case["D"] + 1)
    lengths = case["lengths"]
    window = [L - 64 * (max(L - 128, 0) // 64) for L in lengths]
    nb = [(L - w) // 64 for L, w in zip(lengths, window)]
    bits = [rng.choice(np.array([2, 3, 4, 8], np.uint8), size=n) if case.get("mixed") else np.full(n, 4, np.uint8)
            for n in nb]
    b = build(case["H"], case["D"], lengths, bits=bits, window=window, latent=case.get("latent", False),
              rope_dim=case.get("R", 0), seed=case["D"] + 7)
    paths = []
    for a in range(len(lengths)):
        p = tmp_path / f"agent{a}.kvqcard"
        card.save_card(b.cache, a, p, model_id="synthetic", position_offset=3 * a)
        paths.append(p)
    # restore in reverse order into a fresh cache (other pool offsets)
    c2, metas = card.cache_from_cards(list(reversed(paths)))
    assert [m["position_offset"] for m in metas] == [str(3 * a) for a in reversed(range(len(lengths)))]
    torch.cuda.synchronize()
    k1, v1 = _dequant(b.cache)
    k2, v2 = _dequant(c2)
    A = len(lengths)
    for a in range(A):
        L = lengths[a]
        assert np.array_equal(k1[a, :64 * nb[a]], k2[A - 1 - a, :64 * nb[a]]), f"K blocks {a}"
        if not b.cache.latent:
            assert np.array_equal(v1[a, :64 * nb[a]], v2[A - 1 - a, :64 * nb[a]]), f"V blocks {a}"
        # windows follow the blocks in the restored rows
        r1 = b.cache.max_blocks * 64
        r2 = c2.max_blocks * 64
        assert np.array_equal(k1[a, r1:r1 + window[a]], k2[A - 1 - a, r2:r2 + window[a]]), f"K window {a}"
    Dk = case["D"] + case.get("R", 0)
    Hq = 16 if case.get("latent") else 4 * case["H"]
    q = syn.random_normal_bf16((A, Hq, Dk), 31)
    scale = Dk ** -0.5
    got = c2.attend_decode(to_dev_bf16(q[::-1].copy()), scale).cpu().numpy()[::-1]
    close(got, ref_decode(b, q, scale), what="decode over restored cards")


def test_load_into_matching_slots():
    H, D = 2, 128
    lengths = [64 * 3 + 140, 64 * 2 + 150]
    window = [140, 150]
    bits = [np.array([4, 3, 8], np.uint8), np.array([2, 4], np.uint8)]
    b = build(H, D, lengths, bits=bits, window=window, seed=3)
    img0 = b.cache.card_gather(0).clone()
    img1 = b.cache.card_gather(1).clone()
    # a second cache with the same slot widths, empty, then swap the agents' contents in
    c = kvq.LayerCache(H, D, [3, 2], [0, 0], bits, window_cap=b.cache.window_cap)
    c.card_scatter(0, img0, 3, 140, bits[0])
    c.card_scatter(1, img1, 2, 150, bits[1])
    torch.cuda.synchronize()
    assert torch.equal(c.card_gather(0), img0) and torch.equal(c.card_gather(1), img1)
    with pytest.raises(ValueError):
        c.card_scatter(1, img0, 3, 140, bits[0])          # widths differ from the slots
