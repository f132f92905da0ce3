"""Loader and numpy wrappers for the C oracle ``libkvq_ref.so``.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``.  The product package never imports it.

The C source (``kvq_ref.c``) is the oracle; this module only compiles it
with gcc and marshals numpy arrays into its host-pointer calls.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_ref.c")
LIB = os.path.join(HERE, "libkvq_ref.so")
SAN_LIB = os.path.join(HERE, "libkvq_ref_san.so")
# KVQ_ORACLE_LIB selects another build of the same source (the sanitized one
# below, for the pin tests run under AddressSanitizer/UBSan).
_LIB_OVERRIDE = os.environ.get("KVQ_ORACLE_LIB")

# ISO C99 (so gcc does not contract a*b+c into an FMA), no fast-math,
# OpenMP for the independent loops.
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


SAN_FLAGS = ["-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build_sanitized() -> str:
    """The same source with AddressSanitizer and UBSan (gcc), into
    ``oracle/libkvq_ref_san.so``; loaded with KVQ_ORACLE_LIB and the ASan
    runtime preloaded."""
    tmp = SAN_LIB + ".tmp"
    subprocess.check_call(["gcc", *SAN_FLAGS, SRC, "-o", tmp, "-lm"])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libkvq_ref.so``."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build(force=True)
            L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, f32, u64, i64 = ctypes.c_int, ctypes.c_float, ctypes.c_uint64, ctypes.c_long
        L.kvq_ref_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvq_ref_bf16_to_f32.restype = f32
        L.kvq_ref_f32_to_bf16.argtypes = [f32]
        L.kvq_ref_f32_to_bf16.restype = ctypes.c_uint16
        L.kvq_ref_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvq_ref_f16_to_f32.restype = f32
        L.kvq_ref_f32_to_f16.argtypes = [f32]
        L.kvq_ref_f32_to_f16.restype = ctypes.c_uint16
        for n in ("kvq_ref_f32_to_f16_n", "kvq_ref_f32_to_bf16_n", "kvq_ref_f16_to_f32_n"):
            getattr(L, n).argtypes = [P, P, ctypes.c_size_t]
            getattr(L, n).restype = None
        L.kvq_ref_quantize_group.argtypes = [P, i32, P, P, P]
        L.kvq_ref_quantize_group.restype = i32
        L.kvq_ref_unpack_group.argtypes = [P, i32, P]
        L.kvq_ref_unpack_group.restype = i32
        L.kvq_ref_pack_group.argtypes = [P, i32, P]
        L.kvq_ref_pack_group.restype = i32
        L.kvq_ref_dequantize_group.argtypes = [P, i32, ctypes.c_uint16, ctypes.c_uint16, P]
        L.kvq_ref_dequantize_group.restype = i32
        L.kvq_ref_block_bytes.argtypes = [i32, i32, i32]
        L.kvq_ref_block_bytes.restype = u64
        L.kvq_ref_quantize_seq.argtypes = [P, i32, i32, i32, P, P, P]
        L.kvq_ref_quantize_seq.restype = i32
        L.kvq_ref_restore_seq.argtypes = [P, P, P, i32, P, i32, i32, i32, P]
        L.kvq_ref_restore_seq.restype = i32
        L.kvq_ref_attention.argtypes = [P, i64, i64, i32, P, i64, i64, i32, i32, i32, P, i32,
                                        ctypes.c_double, P]
        L.kvq_ref_attention.restype = None
        L.kvq_ref_attend_decode_seq.argtypes = [P, P, P, P, i32, P, P, i32, P, i32, i32, i32,
                                                P, i32, f32, P]
        L.kvq_ref_attend_decode_seq.restype = i32
        L.kvq_ref_attend_chunk_seq.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, P, P, P,
                                               i32, i32, f32, i32, i32, P]
        L.kvq_ref_attend_chunk_seq.restype = i32
        L.kvq_ref_append_seq.argtypes = [P, P, P, P, P, i32, i32, P, P, i32, i32, i32, i32, P, P, i32,
                                         i32, P, P, i32, P, P]
        L.kvq_ref_append_seq.restype = i32
        L.kvq_ref_block_scores_seq.argtypes = [P, P, P, i32, P, i32, i32, i32, P, i32, ctypes.c_double, P]
        L.kvq_ref_block_scores_seq.restype = i32
        L.kvq_ref_block_sensitivity.argtypes = [P, P, i32, i32, P, i32, ctypes.c_double, P]
        L.kvq_ref_block_sensitivity.restype = i32
        L.kvq_ref_block_error_bound.argtypes = [P, P, i32, i32, P, i32, i32, ctypes.c_double, i32]
        L.kvq_ref_block_error_bound.restype = ctypes.c_double
        L.kvq_ref_max_threads.argtypes = []
        L.kvq_ref_max_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---- conversions ----------------------------------------------------------
def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32).ravel(), np.float32)
    y = np.empty(x.size, np.uint16)
    lib().kvq_ref_f32_to_f16_n(_p(x), _p(y), x.size)
    return y


def f32_to_bf16_bits(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32).ravel(), np.float32)
    y = np.empty(x.size, np.uint16)
    lib().kvq_ref_f32_to_bf16_n(_p(x), _p(y), x.size)
    return y


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(np.asarray(h, dtype=np.uint16).ravel(), np.uint16)
    y = np.empty(h.size, np.float32)
    lib().kvq_ref_f16_to_f32_n(_p(h), _p(y), h.size)
    return y


# ---- groups ---------------------------------------------------------------
def quantize_group(x_bf16, bits: int):
    """Returns (words uint32[2*bits], scale fp16 bits, bias fp16 bits)."""
    x = _c(x_bf16, np.uint16)
    assert x.size == 64
    w = np.zeros(16, np.uint32)
    s = np.zeros(1, np.uint16)
    b = np.zeros(1, np.uint16)
    rc = lib().kvq_ref_quantize_group(_p(x), bits, _p(w), _p(s), _p(b))
    if rc:
        raise ValueError("unsupported width")
    return w[: 2 * bits].copy(), int(s[0]), int(b[0])


def unpack_group(words, bits: int) -> np.ndarray:
    w = np.zeros(16, np.uint32)
    w[: 2 * bits] = np.asarray(words, np.uint32)
    c = np.zeros(64, np.uint8)
    if lib().kvq_ref_unpack_group(_p(w), bits, _p(c)):
        raise ValueError("unsupported width")
    return c


def pack_group(codes, bits: int) -> np.ndarray:
    c = _c(codes, np.uint8)
    w = np.zeros(16, np.uint32)
    if lib().kvq_ref_pack_group(_p(c), bits, _p(w)):
        raise ValueError("unsupported width")
    return w[: 2 * bits].copy()


def dequantize_group(words, bits: int, scale_h: int, bias_h: int) -> np.ndarray:
    w = np.zeros(16, np.uint32)
    w[: 2 * bits] = np.asarray(words, np.uint32)
    out = np.zeros(64, np.float32)
    if lib().kvq_ref_dequantize_group(_p(w), bits, scale_h, bias_h, _p(out)):
        raise ValueError("unsupported width")
    return out


def block_bytes(bits: int, n_heads: int, head_dim: int) -> int:
    return int(lib().kvq_ref_block_bytes(bits, n_heads, head_dim))


def packed_offsets(bits, n_heads: int, head_dim: int, align: int = 256) -> tuple[np.ndarray, int]:
    """Byte offsets of consecutive blocks packed back to back (each padded to
    ``align``), and the total size."""
    bits = np.asarray(bits, np.uint8).ravel()
    off = np.zeros(bits.size, np.uint64)
    pos = 0
    for j, b in enumerate(bits):
        off[j] = pos
        nb = block_bytes(int(b), n_heads, head_dim)
        pos += (nb + align - 1) // align * align
    return off, pos


# ---- sequences ------------------------------------------------------------
def quantize_seq(x_bf16, n_heads, head_dim, bits, offset, pool):
    """Quantize x [64*nb][H][D] (uint16 bf16 bits) into ``pool`` (uint8, in place)."""
    x = _c(x_bf16, np.uint16)
    bits = _c(bits, np.uint8)
    offset = _c(offset, np.uint64)
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    nb = bits.size
    assert x.size >= nb * 64 * n_heads * head_dim
    rc = lib().kvq_ref_quantize_seq(_p(x), n_heads, head_dim, nb, _p(bits), _p(offset), _p(pool))
    if rc:
        raise ValueError("kvq_ref_quantize_seq failed")


def restore_seq(pool, bits, offset, window, n_heads, head_dim) -> np.ndarray:
    """fp32 rows [64*nb + W][H][D]: dequantized blocks, then the window."""
    bits = _c(bits, np.uint8)
    offset = _c(offset, np.uint64)
    nw = 0 if window is None else window.size // (n_heads * head_dim)
    win = None if window is None else _c(window, np.uint16)
    T = bits.size * 64 + nw
    out = np.zeros((T, n_heads, head_dim), np.float32)
    rc = lib().kvq_ref_restore_seq(_p(pool), _p(bits), _p(offset), bits.size, _p(win), nw,
                                   n_heads, head_dim, _p(out))
    if rc:
        raise ValueError("kvq_ref_restore_seq failed")
    return out


def attention(K, V, q_bf16, scale: float) -> np.ndarray:
    """K fp32 [T][Hkv][dk], V fp32 [T][Hkv][dv], q bf16 bits [Hq][dk] -> fp32 [Hq][dv]."""
    K = _c(K, np.float32)
    V = _c(V, np.float32)
    q = _c(q_bf16, np.uint16)
    T, H, dk = K.shape
    dv = V.shape[2]
    Hq = q.shape[0]
    out = np.zeros((Hq, dv), np.float32)
    lib().kvq_ref_attention(_p(K), H * dk, dk, dk, _p(V), H * dv, dv, dv, T, H, _p(q), Hq,
                            float(scale), _p(out))
    return out


def attend_decode_seq(pool, bits, k_offset, v_offset, k_window, v_window, rope, n_kv_heads,
                      head_dim, q_bf16, scale) -> np.ndarray:
    bits = _c(bits, np.uint8)
    k_offset = _c(k_offset, np.uint64)
    v_offset = _c(v_offset, np.uint64)
    nw = 0 if k_window is None else k_window.size // (n_kv_heads * head_dim)
    k_window = _c(k_window, np.uint16)
    v_window = _c(v_window, np.uint16)
    rope = _c(rope, np.uint16)
    T = bits.size * 64 + nw
    rope_dim = 0 if rope is None else rope.size // max(1, T * n_kv_heads)
    q = _c(q_bf16, np.uint16)
    Hq = q.size // (head_dim + rope_dim)
    out = np.zeros((Hq, head_dim), np.float32)
    rc = lib().kvq_ref_attend_decode_seq(_p(pool), _p(bits), _p(k_offset), _p(v_offset), bits.size,
                                         _p(k_window), _p(v_window), nw, _p(rope), rope_dim,
                                         n_kv_heads, head_dim, _p(q), Hq, float(scale), _p(out))
    if rc:
        raise ValueError("kvq_ref_attend_decode_seq failed")
    return out


def attend_chunk_seq(pool, bits, k_offset, v_offset, k_window, v_window, n_kv_heads, head_dim,
                     q_new, k_new, v_new, scale, row_begin=0, row_end=None) -> np.ndarray:
    bits = _c(bits, np.uint8)
    k_offset = _c(k_offset, np.uint64)
    v_offset = _c(v_offset, np.uint64)
    nw = 0 if k_window is None else k_window.size // (n_kv_heads * head_dim)
    k_window = _c(k_window, np.uint16)
    v_window = _c(v_window, np.uint16)
    q_new = _c(q_new, np.uint16)
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    n_new = k_new.size // (n_kv_heads * head_dim)
    Hq = q_new.size // max(1, n_new * head_dim) if n_new else 0
    if row_end is None:
        row_end = n_new
    out = np.zeros((n_new, Hq, head_dim), np.float32)
    rc = lib().kvq_ref_attend_chunk_seq(_p(pool), _p(bits), _p(k_offset), _p(v_offset), bits.size,
                                        _p(k_window), _p(v_window), nw, n_kv_heads, head_dim,
                                        _p(q_new), _p(k_new), _p(v_new), n_new, Hq, float(scale),
                                        row_begin, row_end, _p(out))
    if rc:
        raise ValueError("kvq_ref_attend_chunk_seq failed")
    return out


def append_seq(k_pool, v_pool, bits, k_offset, v_offset, n_blocks, k_window, v_window, n_window,
               n_heads, head_dim, k_new, v_new, keep, rope=None, rope_new=None):
    """Window roll of one sequence, in place.  ``bits``/``*_offset`` are the
    sequence's full table rows [max_blocks]; ``k_window``/``v_window`` uint16
    [window_cap][H][D]; ``rope`` uint16 [64*max_blocks + window_cap][H][R].
    Returns the new (n_blocks, n_window)."""
    bits = _c(bits, np.uint8)
    k_offset = _c(k_offset, np.uint64)
    v_offset = _c(v_offset, np.uint64)
    for a in (k_pool, v_pool, k_window, v_window, rope):
        assert a is None or a.flags.c_contiguous
    max_blocks = bits.size
    window_cap = 0 if k_window is None else k_window.size // (n_heads * head_dim)
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    rope_new = _c(rope_new, np.uint16)
    n_new = 0 if k_new is None else k_new.size // (n_heads * head_dim)
    rope_dim = 0
    if rope is not None:
        rope_dim = rope.size // ((64 * max_blocks + window_cap) * n_heads)
    nb_out = ctypes.c_int(0)
    nw_out = ctypes.c_int(0)
    rc = lib().kvq_ref_append_seq(_p(k_pool), _p(v_pool), _p(bits), _p(k_offset), _p(v_offset),
                                  max_blocks, int(n_blocks), _p(k_window), _p(v_window), window_cap,
                                  int(n_window), n_heads, head_dim, _p(k_new), _p(v_new), n_new,
                                  int(keep), _p(rope), _p(rope_new), rope_dim, ctypes.byref(nb_out),
                                  ctypes.byref(nw_out))
    if rc:
        raise ValueError("kvq_ref_append_seq: result does not fit or bad arguments")
    return nb_out.value, nw_out.value


def card_image(pool, bits, k_offset, v_offset, k_window, v_window, rope, n_heads, head_dim) -> np.ndarray:
    """A sequence's CacheCard image, by concatenation: K block payloads, V
    block payloads (v_offset None: latent), K window rows, V window rows,
    rope rows by token position, widths (uint8)."""
    bits = np.asarray(bits, np.uint8)
    parts = []
    for off in (k_offset, v_offset):
        if off is None:
            continue
        for j, b in enumerate(bits):
            o = int(off[j])
            parts.append(pool[o:o + block_bytes(int(b), n_heads, head_dim)])
    for w in (k_window, v_window):
        if w is not None:
            parts.append(np.ascontiguousarray(w, np.uint16).view(np.uint8).ravel())
    if rope is not None:
        parts.append(np.ascontiguousarray(rope, np.uint16).view(np.uint8).ravel())
    parts.append(bits)
    return np.concatenate([np.asarray(p, np.uint8).ravel() for p in parts])


def block_scores_seq(pool, bits, k_offset, rope, n_kv_heads, head_dim, q_bf16, scale) -> np.ndarray:
    """fp64 score of each block: max over its tokens and the query heads of
    scale * <q, k> (restored keys, plus rope dims)."""
    bits = _c(bits, np.uint8)
    k_offset = _c(k_offset, np.uint64)
    nb = bits.size
    rope = _c(rope, np.uint16)
    rope_dim = 0 if rope is None else rope.size // max(1, 64 * nb * n_kv_heads)
    q = _c(q_bf16, np.uint16)
    Hq = q.size // (head_dim + rope_dim)
    out = np.zeros(nb, np.float64)
    rc = lib().kvq_ref_block_scores_seq(_p(pool), _p(bits), _p(k_offset), nb, _p(rope), rope_dim,
                                        n_kv_heads, head_dim, _p(q), Hq, float(scale), _p(out))
    if rc:
        raise ValueError("kvq_ref_block_scores_seq failed")
    return out


def topk_blocks(scores, k: int) -> np.ndarray:
    """Indices (ascending) of the min(k, n) highest scores; equal scores
    rank the lower index first."""
    s = np.asarray(scores, np.float64)
    order = sorted(range(s.size), key=lambda i: (-s[i], i))
    return np.array(sorted(order[:min(k, s.size)]), np.int64)


def block_sensitivity(k_bf16, v_bf16, n_kv_heads, head_dim, q_bf16, scale) -> float:
    """S of one block (k, v bf16 [64][H][D], q bf16 [Hq][D]): the width-free
    factor of the block's first-order attention-error bound."""
    k = _c(k_bf16, np.uint16)
    v = _c(v_bf16, np.uint16)
    q = _c(q_bf16, np.uint16)
    out = np.zeros(1, np.float64)
    if lib().kvq_ref_block_sensitivity(_p(k), _p(v), n_kv_heads, head_dim, _p(q), q.size // head_dim,
                                       float(scale), _p(out)):
        raise ValueError("kvq_ref_block_sensitivity failed")
    return float(out[0])


def block_error_bound(k_bf16, v_bf16, n_kv_heads, head_dim, q_bf16, h, scale, bits) -> float:
    k = _c(k_bf16, np.uint16)
    v = _c(v_bf16, np.uint16)
    q = _c(q_bf16, np.uint16)
    return float(lib().kvq_ref_block_error_bound(_p(k), _p(v), n_kv_heads, head_dim, _p(q), q.size // head_dim,
                                                 h, float(scale), bits))


WIDTHS = (2, 3, 4, 8)


def width_cost(b) -> float:
    """c(b) = 1/(2(2^b - 1)): the error factor of width b."""
    return 1.0 / (2.0 * ((1 << int(b)) - 1))


def allocate_widths(S, bytes_per_block_at, budget) -> np.ndarray:
    """Greedy budgeted allocation: every block starts at 2 bits; repeatedly
    take the (block, next width) step with the largest error reduction
    S_i (c(b) - c(b')) per extra byte that still fits the budget (equal
    ratios: lower block index first), until no step fits.
    bytes_per_block_at(b) -> bytes of one block at width b."""
    S = np.asarray(S, np.float64)
    w = np.full(S.size, 0, np.int64)                 # index into WIDTHS
    used = S.size * bytes_per_block_at(WIDTHS[0])
    if used > budget:
        raise ValueError("budget below the all-2-bit size")
    while True:
        best, bi = None, -1
        for i in range(S.size):
            if w[i] + 1 >= len(WIDTHS):
                continue
            b0, b1 = WIDTHS[w[i]], WIDTHS[w[i] + 1]
            extra = bytes_per_block_at(b1) - bytes_per_block_at(b0)
            if used + extra > budget:
                continue
            r = S[i] * (width_cost(b0) - width_cost(b1)) / extra
            if best is None or r > best:
                best, bi = r, i
        if bi < 0:
            break
        used += bytes_per_block_at(WIDTHS[w[bi] + 1]) - bytes_per_block_at(WIDTHS[w[bi]])
        w[bi] += 1
    return np.array([WIDTHS[i] for i in w], np.uint8)


def max_threads() -> int:
    return int(lib().kvq_ref_max_threads())
