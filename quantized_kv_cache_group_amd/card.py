"""CacheCard files: one sequence of a LayerCache persisted and restored.

A CacheCard carries an agent's quantized KV groups, their widths and the
recent native-precision rows, with the metadata needed to inject it again
(sequence length, model id, position offset): QKVShare, section Metodologia
(the CacheCard handoff between agents) and Agent Memory Below the Prompt,
arXiv 2603.04428, Abstract (per-agent 4-bit caches persisted and reloaded,
then batched in one attention call).

The file is a safetensors file: an 8-byte little-endian header length, a JSON
header (tensor dtypes, shapes and byte ranges, plus string metadata), then
the device image that ``kvq_card_gather`` writes, unchanged:
    k_blocks U8 [bytes]  v_blocks U8 [bytes]  k_window BF16 [W][H][D]
    v_window BF16 [W][H][D]  rope BF16 [T][H][R]  bits U8 [n_blocks]
(v_* absent for a latent cache, rope absent when R is 0).  The GPU moves the
bytes; this module only frames them.
"""
from __future__ import annotations

import json
import struct

import numpy as np
import torch

FORMAT = "kvq-cachecard"
VERSION = "1"


def segments(n_heads, head_dim, rope_dim, latent, n_blocks, n_window, block_bytes_total):
    """[(name, dtype, shape, begin, end)] of an image, in image order."""
    H, D, R = n_heads, head_dim, rope_dim
    row = H * D * 2
    out, pos = [], 0

    def add(name, dtype, shape, n):
        nonlocal pos
        out.append((name, dtype, list(shape), pos, pos + n))
        pos += n
    add("k_blocks", "U8", [block_bytes_total], block_bytes_total)
    if not latent:
        add("v_blocks", "U8", [block_bytes_total], block_bytes_total)
    add("k_window", "BF16", [n_window, H, D], n_window * row)
    if not latent:
        add("v_window", "BF16", [n_window, H, D], n_window * row)
    if R:
        T = 64 * n_blocks + n_window
        add("rope", "BF16", [T, H, R], T * H * R * 2)
    add("bits", "U8", [n_blocks], n_blocks)
    return out


def write_file(path, image: np.ndarray, meta: dict, layout: dict):
    """Frame a host image as a safetensors file.  layout: n_heads, head_dim,
    rope_dim, latent, n_blocks, n_window, block_bytes_total."""
    segs = segments(**layout)
    assert image.dtype == np.uint8 and image.size == segs[-1][4], (image.size, segs[-1][4])
    md = {"format": FORMAT, "version": VERSION, "group": "64"}
    md.update({k: str(v) for k, v in meta.items()})
    md.update({k: str(int(v)) for k, v in layout.items()})
    header = {"__metadata__": md}
    for name, dtype, shape, b, e in segs:
        header[name] = {"dtype": dtype, "shape": shape, "data_offsets": [b, e]}
    hb = json.dumps(header, separators=(",", ":")).encode()
    hb += b" " * (-len(hb) % 8)
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(hb)))
        f.write(hb)
        f.write(image.tobytes())


def read_file(path):
    """(metadata dict, layout dict, image uint8 array) of a card file."""
    with open(path, "rb") as f:
        n = struct.unpack("<Q", f.read(8))[0]
        header = json.loads(f.read(n))
        image = np.frombuffer(f.read(), np.uint8)
    md = header.pop("__metadata__")
    if md.get("format") != FORMAT:
        raise ValueError("not a kvq CacheCard")
    keys = ("n_heads", "head_dim", "rope_dim", "latent", "n_blocks", "n_window", "block_bytes_total")
    layout = {k: int(md[k]) for k in keys}
    segs = segments(**layout)
    if image.size != segs[-1][4]:
        raise ValueError("truncated CacheCard")
    for name, dtype, shape, b, e in segs:
        h = header[name]
        if h["dtype"] != dtype or h["shape"] != shape or h["data_offsets"] != [b, e]:
            raise ValueError(f"CacheCard tensor {name} does not match its layout")
    meta = {k: v for k, v in md.items() if k not in keys}
    return meta, layout, image


def card_bits(layout: dict, image: np.ndarray) -> np.ndarray:
    b, e = segments(**layout)[-1][3:5]
    return image[b:e].copy()


def save_card(cache, seq: int, path, model_id: str = "", position_offset: int = 0, stream=None):
    """Gather sequence seq of cache on the GPU and write it as a card file."""
    from . import block_bytes
    nb, nw = cache.n_blocks_host[seq], cache.n_window_host[seq]
    img = cache.card_gather(seq, stream=stream)
    host = img.cpu().numpy()
    total = sum(block_bytes(int(b), cache.H, cache.D) for b in cache.bits_host[seq, :nb])
    layout = dict(n_heads=cache.H, head_dim=cache.D, rope_dim=cache.rope_dim, latent=int(cache.latent),
                  n_blocks=nb, n_window=nw, block_bytes_total=total)
    meta = dict(model_id=model_id, seq_len=64 * nb + nw, position_offset=position_offset)
    write_file(path, host, meta, layout)


def load_card(cache, seq: int, path, stream=None) -> dict:
    """Restore a card file into sequence seq of cache (its slots must have the
    card's widths).  Returns the card's metadata."""
    meta, layout, image = read_file(path)
    if (layout["n_heads"], layout["head_dim"], layout["rope_dim"], layout["latent"]) != \
            (cache.H, cache.D, cache.rope_dim, int(cache.latent)):
        raise ValueError("CacheCard shape differs from the cache")
    dev = torch.from_numpy(image.copy()).to(cache.k_pool.device)
    cache.card_scatter(seq, dev, layout["n_blocks"], layout["n_window"], card_bits(layout, image),
                       stream=stream)
    return meta


def cache_from_cards(paths, window_cap=None, device="cuda"):
    """A LayerCache holding one sequence per card (batched over the restored
    agents), and the cards' metadata."""
    from . import LayerCache
    cards = [read_file(p) for p in paths]
    shapes = {(l["n_heads"], l["head_dim"], l["rope_dim"], l["latent"]) for _, l, _ in cards}
    if len(shapes) != 1:
        raise ValueError("cards of different shapes")
    H, D, R, latent = shapes.pop()
    nbs = [l["n_blocks"] for _, l, _ in cards]
    nws = [l["n_window"] for _, l, _ in cards]
    bits = [card_bits(l, im) for _, l, im in cards]
    cap = max(nws + [0]) if window_cap is None else window_cap
    cache = LayerCache(H, D, nbs, nws, bits, window_cap=cap, latent=bool(latent), rope_dim=R, device=device)
    for a, (_, l, im) in enumerate(cards):
        dev = torch.from_numpy(im.copy()).to(cache.k_pool.device)
        cache.card_scatter(a, dev, l["n_blocks"], l["n_window"], bits[a])
    return cache, [m for m, _, _ in cards]
