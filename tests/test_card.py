"""CacheCard files on the host: the oracle's image (plain concatenation of a
sequence's blocks, windows, rope rows and widths) has the size the library
states, and a file framed from it is a valid safetensors file whose tensors,
read back by the independent safetensors parser, are those pieces."""
import os

import numpy as np
import pytest
import torch

import kvq_synth as syn
import oracle
import quantized_kv_cache_group_amd as kvq
from quantized_kv_cache_group_amd import card

lib_built = os.path.exists(kvq.LIB_PATH)


def _oracle_seq(H, D, bits, nw, latent=False, R=0, seed=0):
    nb = len(bits)
    T = 64 * nb + nw
    k = syn.random_normal_bf16((T, H, D), seed)
    v = None if latent else syn.random_normal_bf16((T, H, D), seed + 1)
    rope = syn.random_normal_bf16((T, H, R), seed + 2) if R else None
    koff, tot = oracle.packed_offsets(bits, H, D)
    pool = np.zeros(2 * max(tot, 256), np.uint8)
    voff = None if latent else koff + np.uint64(max(tot, 256))
    oracle.quantize_seq(k, H, D, bits, koff, pool)
    if not latent:
        oracle.quantize_seq(v, H, D, bits, voff, pool)
    img = oracle.card_image(pool, bits, koff, voff, k[64 * nb:] if nw else np.zeros((0, H, D), np.uint16),
                            None if latent else (v[64 * nb:] if nw else np.zeros((0, H, D), np.uint16)),
                            rope, H, D)
    total = sum(oracle.block_bytes(int(b), H, D) for b in bits)
    layout = dict(n_heads=H, head_dim=D, rope_dim=R, latent=int(latent), n_blocks=nb, n_window=nw,
                  block_bytes_total=total)
    return img, layout, pool, koff, voff, k, v, rope


CASES = [dict(H=2, D=128, bits=[4, 3, 2, 8, 4], nw=150),
         dict(H=1, D=512, bits=[4, 4, 4], nw=9, latent=True, R=64),
         dict(H=4, D=64, bits=[], nw=100),
         dict(H=2, D=256, bits=[2, 8], nw=0)]


@pytest.mark.skipif(not lib_built, reason="libkvq.so not built")
@pytest.mark.parametrize("case", CASES)
def test_image_size_matches_library(case):
    img, layout, *_ = _oracle_seq(case["H"], case["D"], np.asarray(case["bits"], np.uint8), case["nw"],
                                  case.get("latent", False), case.get("R", 0))
    bits = np.ascontiguousarray(np.asarray(case["bits"], np.uint8))
    n = kvq.lib().kvq_card_bytes(case["H"], case["D"], case.get("R", 0), 0 if case.get("latent") else 1,
                                 bits.size, bits.ctypes.data_as(kvq.ctypes.c_void_p) if bits.size else None,
                                 case["nw"])
    assert n == img.size == card.segments(**layout)[-1][4]
    # every segment but the widths is a multiple of 128 bytes
    assert all((e - b) % 128 == 0 for _, _, _, b, e in card.segments(**layout)[:-1])


@pytest.mark.parametrize("case", CASES)
def test_card_file_is_safetensors(case, tmp_path):
    from safetensors.torch import load_file
    bits = np.asarray(case["bits"], np.uint8)
    img, layout, pool, koff, voff, k, v, rope = _oracle_seq(case["H"], case["D"], bits, case["nw"],
                                                             case.get("latent", False), case.get("R", 0), seed=3)
    path = tmp_path / "a.kvqcard"
    card.write_file(path, img, dict(model_id="synthetic-llama", seq_len=64 * bits.size + case["nw"],
                                    position_offset=17), layout)
    t = load_file(str(path))
    H, D, nb, nw = case["H"], case["D"], bits.size, case["nw"]
    blocks = [pool[int(o):int(o) + oracle.block_bytes(int(b), H, D)] for o, b in zip(koff, bits)]
    want_k = np.concatenate(blocks) if blocks else np.zeros(0, np.uint8)
    assert np.array_equal(t["k_blocks"].numpy(), want_k)
    assert np.array_equal(t["k_window"].view(torch.int16).numpy().view(np.uint16), k[64 * nb:64 * nb + nw])
    if not case.get("latent"):
        vb = [pool[int(o):int(o) + oracle.block_bytes(int(b), H, D)] for o, b in zip(voff, bits)]
        assert np.array_equal(t["v_blocks"].numpy(), np.concatenate(vb) if vb else np.zeros(0, np.uint8))
        assert np.array_equal(t["v_window"].view(torch.int16).numpy().view(np.uint16), v[64 * nb:64 * nb + nw])
    else:
        assert "v_blocks" not in t and "v_window" not in t
    if case.get("R"):
        assert np.array_equal(t["rope"].view(torch.int16).numpy().view(np.uint16), rope)
    assert np.array_equal(t["bits"].numpy(), bits)
    meta, lay, img2 = card.read_file(path)
    assert lay == layout and np.array_equal(img2, img)
    assert meta["model_id"] == "synthetic-llama" and meta["position_offset"] == "17"
    assert meta["seq_len"] == str(64 * nb + nw)


def test_card_file_rejects_damage(tmp_path):
    bits = np.asarray([4, 2], np.uint8)
    img, layout, *_ = _oracle_seq(2, 64, bits, 70)
    path = tmp_path / "b.kvqcard"
    card.write_file(path, img, {}, layout)
    data = open(path, "rb").read()
    open(tmp_path / "short", "wb").write(data[:-5])
    with pytest.raises(ValueError):
        card.read_file(tmp_path / "short")
