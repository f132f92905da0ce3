/*
 * kvq_ref.c — CPU oracle for group-wise quantized KV caches.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).
 * Plain, slow and written to be checked by eye.  Compile as ISO C99 with
 * -ffp-contract=off and without -ffast-math: every float operation below is
 * one IEEE binary32 operation rounded to nearest even, and the only fused
 * multiply-add is the explicit fmaf() of the dequantizer.
 *
 * Sources (the pages state the problem, not the formula):
 *   [QKVShare]  QKVShare: Quantized KV-Cache Handoff for Multi-Agent
 *               On-Device LLMs, section Metodologia (CacheCard of quantized
 *               KV groups; injection path that rebuilds FP16 past_key_values).
 *   [AgentMem]  Agent Memory Below the Prompt: Persistent Q4 KV Cache for
 *               Multi-Agent LLM Inference on Edge Devices (arXiv 2603.04428),
 *               Abstract (4-bit caches in a block pool, restored into the
 *               attention layer, batched over agents, cross-phase injection;
 *               GQA and MLA model families).
 *   [CoMixKV]   Coordinated Mixed-Precision KV Cache Quantization for
 *               Efficient LLM-based Multi-agent Systems (arXiv 2611.10096),
 *               Abstract (per-agent/layer widths, applied only to newly
 *               quantized blocks; recent states stay in native precision).
 */
#include "kvq_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int kvq_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 conversions.                                                      */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 is the upper half of a binary32. */
float kvq_ref_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even on the 16 dropped bits. */
uint16_t kvq_ref_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)          /* NaN: keep sign, make quiet */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;                            /* carries into the exponent as needed */
    return (uint16_t)(u >> 16);
}

/* binary16 -> binary32 (exact). */
float kvq_ref_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t m = h & 0x3ffu;
    if (e == 0x1f)                                  /* inf / NaN */
        return bits_f32(sign | 0x7f800000u | (m << 13));
    if (e == 0) {                                   /* zero / subnormal: m * 2^-24 */
        float v = (float)m * 0x1p-24f;              /* exact: m < 2^10 */
        return sign ? -v : v;
    }
    return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

/* Shift a significand right by sh bits, rounding to nearest even. */
static uint32_t shr_rne(uint32_t sig, unsigned sh)
{
    if (sh == 0) return sig;
    if (sh >= 32) return 0;
    uint32_t q = sig >> sh;
    uint32_t rem = sig & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    return q;
}

/* binary32 -> binary16, round to nearest even. */
uint16_t kvq_ref_f32_to_f16(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);  /* NaN */
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520 rounds to inf */
    uint32_t E = a >> 23;                                    /* biased binary32 exponent */
    uint32_t mant = a & 0x7fffffu;
    if (E >= 113) {                                          /* binary16 normal range */
        uint32_t h = ((E - 112u) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
        return (uint16_t)(sign | h);
    }
    /* binary16 subnormal (or zero): value = sig * 2^(E-150), units of 2^-24. */
    uint32_t sig = E ? (mant | 0x800000u) : mant;
    unsigned sh = E ? (126u - E) : 125u;                     /* E=0 means 2^-149 units */
    return (uint16_t)(sign | shr_rne(sig, sh));
}

void kvq_ref_f32_to_f16_n(const float *x, uint16_t *y, size_t n)
{ for (size_t i = 0; i < n; i++) y[i] = kvq_ref_f32_to_f16(x[i]); }
void kvq_ref_f32_to_bf16_n(const float *x, uint16_t *y, size_t n)
{ for (size_t i = 0; i < n; i++) y[i] = kvq_ref_f32_to_bf16(x[i]); }
void kvq_ref_f16_to_f32_n(const uint16_t *x, float *y, size_t n)
{ for (size_t i = 0; i < n; i++) y[i] = kvq_ref_f16_to_f32(x[i]); }

/* ------------------------------------------------------------------------ */
/* Codes: a little-endian bitstream of 64 b-bit codes in 2b uint32 words.     */
/* Code i occupies stream bits [b*i, b*i+b); word w holds bits [32w, 32w+32). */
/* ------------------------------------------------------------------------ */

static int width_ok(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8; }

int kvq_ref_pack_group(const uint8_t *codes, int bits, uint32_t *words)
{
    if (!width_ok(bits)) return -1;
    for (int w = 0; w < 2 * bits; w++) words[w] = 0;
    for (int i = 0; i < 64; i++) {
        uint32_t q = codes[i] & ((1u << bits) - 1u);
        int pos = bits * i, w = pos >> 5, o = pos & 31;
        words[w] |= q << o;
        if (o + bits > 32) words[w + 1] |= q >> (32 - o);   /* code straddles two words */
    }
    return 0;
}

int kvq_ref_unpack_group(const uint32_t *words, int bits, uint8_t *codes)
{
    if (!width_ok(bits)) return -1;
    for (int i = 0; i < 64; i++) {
        int pos = bits * i, w = pos >> 5, o = pos & 31;
        uint32_t v = words[w] >> o;
        if (o + bits > 32) v |= words[w + 1] << (32 - o);
        codes[i] = (uint8_t)(v & ((1u << bits) - 1u));
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Quantize one group of 64 values (affine, min/max, one width).              */
/* ------------------------------------------------------------------------ */
int kvq_ref_quantize_group(const uint16_t *x, int bits, uint32_t *words,
                           uint16_t *scale_h, uint16_t *bias_h)
{
    if (!width_ok(bits)) return -1;
    const int n = (1 << bits) - 1;                 /* codes 0..n, both ends reachable */
    float xf[64];
    uint8_t codes[64];

    /* Step 1: widen the bf16 inputs (exact). */
    for (int i = 0; i < 64; i++) xf[i] = kvq_ref_bf16_to_f32(x[i]);

    /* Step 2: group minimum and maximum; a zero result is taken as +0 so
     * the stored bias does not depend on the order of +0 and -0. */
    float mn = xf[0], mx = xf[0];
    for (int i = 1; i < 64; i++) {
        if (xf[i] < mn) mn = xf[i];
        if (xf[i] > mx) mx = xf[i];
    }
    mn = mn + 0.0f;
    mx = mx + 0.0f;

    /* Step 3: step size over 2^b - 1 intervals: one rounded subtract, one
     * correctly rounded divide. */
    float s = (mx - mn) / (float)n;

    /* Step 4: the stored metadata are fp16 (round to nearest even). */
    uint16_t sh = kvq_ref_f32_to_f16(s);
    uint16_t bh = kvq_ref_f32_to_f16(mn);

    /* Step 5: codes are computed against the stored values; one reciprocal
     * per group; a zero step (constant group) gives all-zero codes. */
    float sf = kvq_ref_f16_to_f32(sh);
    float bf = kvq_ref_f16_to_f32(bh);
    float inv = (sf == 0.0f) ? 0.0f : 1.0f / sf;

    /* Step 6: offset, scale, round half to even, clamp to [0, n]. */
    for (int i = 0; i < 64; i++) {
        float t = (xf[i] - bf) * inv;
        float r = rintf(t);
        if (!(r >= 0.0f)) r = 0.0f;                /* also maps NaN to 0 */
        if (r > (float)n) r = (float)n;
        codes[i] = (uint8_t)(int)r;
    }

    /* Step 7: pack. */
    kvq_ref_pack_group(codes, bits, words);
    *scale_h = sh;
    *bias_h = bh;
    return 0;
}

/* Dequantize: code * scale + bias with a single rounding (fmaf). */
int kvq_ref_dequantize_group(const uint32_t *words, int bits, uint16_t scale_h,
                             uint16_t bias_h, float *out)
{
    uint8_t codes[64];
    if (kvq_ref_unpack_group(words, bits, codes)) return -1;
    float sf = kvq_ref_f16_to_f32(scale_h);
    float bf = kvq_ref_f16_to_f32(bias_h);
    for (int i = 0; i < 64; i++) out[i] = fmaf((float)codes[i], sf, bf);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Block payload: codes [H][64][D*b/32] words, then meta [H][64][D/64]        */
/* {scale, bias}.  One width per block (a block is created once, CoMixKV).    */
/* ------------------------------------------------------------------------ */

static int dims_ok(int n_heads, int head_dim)
{
    return n_heads >= 1 && head_dim >= 64 && head_dim <= 512 && head_dim % 64 == 0;
}

uint64_t kvq_ref_block_bytes(int bits, int n_heads, int head_dim)
{
    if (!width_ok(bits) || !dims_ok(n_heads, head_dim)) return 0;
    uint64_t code_row = (uint64_t)head_dim * (uint64_t)bits / 8u;      /* bytes per (head, token) */
    uint64_t meta_row = (uint64_t)(head_dim / 64) * 4u;                /* {fp16, fp16} per group */
    return (uint64_t)n_heads * 64u * (code_row + meta_row);
}

/* Byte address of the codes of (head h, token r, group g) inside a block. */
static uint64_t code_at(int bits, int head_dim, int h, int r, int g)
{
    uint64_t code_row = (uint64_t)head_dim * bits / 8u;
    return ((uint64_t)h * 64u + (uint64_t)r) * code_row + (uint64_t)g * 8u * (uint64_t)bits;
}

static uint64_t meta_at(int bits, int n_heads, int head_dim, int h, int r, int g)
{
    uint64_t codes_total = (uint64_t)n_heads * 64u * ((uint64_t)head_dim * bits / 8u);
    return codes_total + (((uint64_t)h * 64u + (uint64_t)r) * (uint64_t)(head_dim / 64) + (uint64_t)g) * 4u;
}

int kvq_ref_quantize_seq(const uint16_t *x, int n_heads, int head_dim, int n_blocks,
                         const uint8_t *bits, const uint64_t *offset, uint8_t *pool)
{
    if (!dims_ok(n_heads, head_dim) || n_blocks < 0) return -1;
    for (int j = 0; j < n_blocks; j++)
        if (!width_ok(bits[j])) return -1;
    const int ng = head_dim / 64;
    long units = (long)n_blocks * n_heads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (long u = 0; u < units; u++) {
        int j = (int)(u / n_heads), h = (int)(u % n_heads);
        int b = bits[j];
        uint8_t *blk = pool + offset[j];
        for (int r = 0; r < 64; r++) {
            long t = (long)j * 64 + r;
            for (int g = 0; g < ng; g++) {
                const uint16_t *src = x + (t * n_heads + h) * head_dim + g * 64;
                uint32_t words[16];
                uint16_t sh, bh;
                kvq_ref_quantize_group(src, b, words, &sh, &bh);
                memcpy(blk + code_at(b, head_dim, h, r, g), words, (size_t)8 * b);
                uint8_t *m = blk + meta_at(b, n_heads, head_dim, h, r, g);
                memcpy(m, &sh, 2);
                memcpy(m + 2, &bh, 2);
            }
        }
    }
    return 0;
}

/* Rows [0, n) of the stream window[0 .. n_window) ++ x_new[0 .. n_new) of
 * row width w (elements) into dst [n][w]. */
static void stream_rows(uint16_t *dst, const uint16_t *window, int n_window, const uint16_t *x_new,
                        int n, size_t w)
{
    for (int t = 0; t < n; t++) {
        const uint16_t *src = t < n_window ? window + (size_t)t * w : x_new + (size_t)(t - n_window) * w;
        memcpy(dst + (size_t)t * w, src, w * sizeof(uint16_t));
    }
}

int kvq_ref_append_seq(uint8_t *k_pool, uint8_t *v_pool, const uint8_t *bits,
                       const uint64_t *k_offset, const uint64_t *v_offset,
                       int max_blocks, int n_blocks, uint16_t *k_window, uint16_t *v_window,
                       int window_cap, int n_window, int n_heads, int head_dim,
                       const uint16_t *k_new, const uint16_t *v_new, int n_new, int keep,
                       uint16_t *rope, const uint16_t *rope_new, int rope_dim,
                       int *n_blocks_out, int *n_window_out)
{
    if (!dims_ok(n_heads, head_dim) || n_new < 0 || keep < 0 || n_window < 0 || n_blocks < 0) return -1;
    const int total = n_window + n_new;                    /* stream length */
    const int k = total > keep ? (total - keep) / 64 : 0;   /* new blocks */
    const int rest = total - 64 * k;                        /* new window */
    if (n_blocks + k > max_blocks || rest > window_cap) return -1;
    for (int i = 0; i < k; i++)
        if (!width_ok(bits[n_blocks + i])) return -1;
    const size_t w = (size_t)n_heads * head_dim, wr = (size_t)n_heads * rope_dim;
    const int n_kv = v_pool ? 2 : 1;
    for (int kv = 0; kv < n_kv; kv++) {
        uint8_t *pool = kv ? v_pool : k_pool;
        uint16_t *window = kv ? v_window : k_window;
        const uint64_t *offset = kv ? v_offset : k_offset;
        uint16_t *T = malloc(((size_t)total + 1) * w * sizeof(uint16_t));
        if (!T) return -1;
        stream_rows(T, window, n_window, kv ? v_new : k_new, total, w);
        /* the first 64k rows become blocks n_blocks .. n_blocks+k-1 */
        kvq_ref_quantize_seq(T, n_heads, head_dim, k, bits + n_blocks, offset + n_blocks, pool);
        /* the rest becomes the window */
        if (rest > 0) memcpy(window, T + (size_t)64 * k * w, (size_t)rest * w * sizeof(uint16_t));
        free(T);
    }
    if (rope_dim > 0) {
        /* rows are token positions: new token i is position 64*n_blocks + n_window + i */
        memcpy(rope + ((size_t)64 * n_blocks + n_window) * wr, rope_new, (size_t)n_new * wr * sizeof(uint16_t));
    }
    *n_blocks_out = n_blocks + k;
    *n_window_out = rest;
    return 0;
}

int kvq_ref_restore_seq(const uint8_t *pool, const uint8_t *bits, const uint64_t *offset,
                        int n_blocks, const uint16_t *window, int n_window,
                        int n_heads, int head_dim, float *out)
{
    if (!dims_ok(n_heads, head_dim) || n_blocks < 0 || n_window < 0) return -1;
    for (int j = 0; j < n_blocks; j++)
        if (!width_ok(bits[j])) return -1;
    const int ng = head_dim / 64;
    long units = (long)n_blocks * n_heads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (long u = 0; u < units; u++) {
        int j = (int)(u / n_heads), h = (int)(u % n_heads);
        int b = bits[j];
        const uint8_t *blk = pool + offset[j];
        for (int r = 0; r < 64; r++) {
            long t = (long)j * 64 + r;
            for (int g = 0; g < ng; g++) {
                uint32_t words[16];
                uint16_t sh, bh;
                memcpy(words, blk + code_at(b, head_dim, h, r, g), (size_t)8 * b);
                const uint8_t *m = blk + meta_at(b, n_heads, head_dim, h, r, g);
                memcpy(&sh, m, 2);
                memcpy(&bh, m + 2, 2);
                kvq_ref_dequantize_group(words, b, sh, bh,
                                         out + (t * n_heads + h) * head_dim + g * 64);
            }
        }
    }
    /* The window tokens follow the quantized ones, widened exactly. */
    long base = (long)n_blocks * 64;
    for (long w = 0; w < n_window; w++)
        for (long e = 0; e < (long)n_heads * head_dim; e++)
            out[(base + w) * n_heads * head_dim + e] =
                kvq_ref_bf16_to_f32(window[w * n_heads * head_dim + e]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention in fp64.                                                         */
/* ------------------------------------------------------------------------ */
void kvq_ref_attention(const float *K, long k_tok_stride, long k_head_stride, int dk,
                       const float *V, long v_tok_stride, long v_head_stride, int dv,
                       int T, int n_kv_heads, const uint16_t *q, int n_q_heads,
                       double scale, float *out)
{
    const int G = n_q_heads / n_kv_heads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) if (T > 4096 || n_q_heads > 8)
#endif
    for (int h = 0; h < n_q_heads; h++) {
        const int g = h / G;                        /* consecutive grouping of query heads */
        double *s = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double *o = (double *)calloc((size_t)dv, sizeof(double));
        double qd[1024];
        for (int d = 0; d < dk; d++) qd[d] = (double)kvq_ref_bf16_to_f32(q[(long)h * dk + d]);
        double m = -INFINITY;
        for (int t = 0; t < T; t++) {
            const float *k = K + (long)t * k_tok_stride + (long)g * k_head_stride;
            double acc = 0.0;
            for (int d = 0; d < dk; d++) acc += qd[d] * (double)k[d];
            s[t] = scale * acc;
            if (s[t] > m) m = s[t];
        }
        double l = 0.0;
        for (int t = 0; t < T; t++) {
            double p = exp(s[t] - m);
            l += p;
            const float *v = V + (long)t * v_tok_stride + (long)g * v_head_stride;
            for (int d = 0; d < dv; d++) o[d] += p * (double)v[d];
        }
        for (int d = 0; d < dv; d++)
            out[(long)h * dv + d] = (T > 0) ? (float)(o[d] / l) : 0.0f;
        free(s);
        free(o);
    }
}

/* Build fp32 keys [T][H][D+R] (restored latent, then rope) and values. */
static int build_kv(const uint8_t *pool, const uint8_t *bits, const uint64_t *k_offset,
                    const uint64_t *v_offset, int n_blocks, const uint16_t *k_window,
                    const uint16_t *v_window, int n_window, const uint16_t *rope, int rope_dim,
                    int H, int D, float **Kout, float **Vout)
{
    long T = (long)n_blocks * 64 + n_window;
    long dk = D + rope_dim;
    float *Kl = (float *)malloc(sizeof(float) * (size_t)(T * H * D + 1));
    float *K = (float *)malloc(sizeof(float) * (size_t)(T * H * dk + 1));
    float *V = NULL;
    if (!Kl || !K) { free(Kl); free(K); return -1; }
    if (kvq_ref_restore_seq(pool, bits, k_offset, n_blocks, k_window, n_window, H, D, Kl)) {
        free(Kl); free(K); return -1;
    }
    for (long t = 0; t < T; t++)
        for (long g = 0; g < H; g++) {
            memcpy(K + (t * H + g) * dk, Kl + (t * H + g) * D, sizeof(float) * (size_t)D);
            for (long r = 0; r < rope_dim; r++)
                K[(t * H + g) * dk + D + r] = kvq_ref_bf16_to_f32(rope[(t * H + g) * rope_dim + r]);
        }
    if (v_offset) {
        V = (float *)malloc(sizeof(float) * (size_t)(T * H * D + 1));
        if (!V || kvq_ref_restore_seq(pool, bits, v_offset, n_blocks, v_window, n_window, H, D, V)) {
            free(V); free(Kl); free(K); return -1;
        }
        free(Kl);
    } else {
        V = Kl;   /* values are the restored key latent */
    }
    *Kout = K;
    *Vout = V;
    return 0;
}

int kvq_ref_attend_decode_seq(const uint8_t *pool, const uint8_t *bits,
                              const uint64_t *k_offset, const uint64_t *v_offset,
                              int n_blocks, const uint16_t *k_window, const uint16_t *v_window,
                              int n_window, const uint16_t *rope, int rope_dim,
                              int n_kv_heads, int head_dim, const uint16_t *q, int n_q_heads,
                              float scale, float *out)
{
    if (!dims_ok(n_kv_heads, head_dim) || n_q_heads < 1 || n_q_heads % n_kv_heads) return -1;
    if (rope_dim < 0 || (rope_dim > 0 && !rope) || head_dim + rope_dim > 1024) return -1;
    float *K, *V;
    if (build_kv(pool, bits, k_offset, v_offset, n_blocks, k_window, v_window, n_window,
                 rope, rope_dim, n_kv_heads, head_dim, &K, &V))
        return -1;
    int T = n_blocks * 64 + n_window;
    long dk = head_dim + rope_dim;
    kvq_ref_attention(K, (long)n_kv_heads * dk, dk, (int)dk,
                      V, (long)n_kv_heads * head_dim, head_dim, head_dim,
                      T, n_kv_heads, q, n_q_heads, (double)scale, out);
    free(K);
    free(V);
    return 0;
}

int kvq_ref_attend_chunk_seq(const uint8_t *pool, const uint8_t *bits,
                             const uint64_t *k_offset, const uint64_t *v_offset,
                             int n_blocks, const uint16_t *k_window, const uint16_t *v_window,
                             int n_window, int n_kv_heads, int head_dim,
                             const uint16_t *q_new, const uint16_t *k_new, const uint16_t *v_new,
                             int n_new, int n_q_heads, float scale,
                             int row_begin, int row_end, float *out)
{
    if (!dims_ok(n_kv_heads, head_dim) || n_q_heads < 1 || n_q_heads % n_kv_heads) return -1;
    if (n_new < 0 || row_begin < 0 || row_end > n_new || row_begin > row_end) return -1;
    float *Kr, *Vr;
    if (build_kv(pool, bits, k_offset, v_offset, n_blocks, k_window, v_window, n_window,
                 NULL, 0, n_kv_heads, head_dim, &Kr, &Vr))
        return -1;
    long P = (long)n_blocks * 64 + n_window;      /* restored tokens */
    long row = (long)n_kv_heads * head_dim;
    long T = P + n_new;
    float *K = (float *)malloc(sizeof(float) * (size_t)(T * row + 1));
    float *V = (float *)malloc(sizeof(float) * (size_t)(T * row + 1));
    if (!K || !V) { free(K); free(V); free(Kr); free(Vr); return -1; }
    memcpy(K, Kr, sizeof(float) * (size_t)(P * row));
    memcpy(V, Vr, sizeof(float) * (size_t)(P * row));
    for (long e = 0; e < (long)n_new * row; e++) {
        K[P * row + e] = kvq_ref_bf16_to_f32(k_new[e]);
        V[P * row + e] = kvq_ref_bf16_to_f32(v_new[e]);
    }
    free(Kr);
    free(Vr);
    /* Causal over the new tokens: query i sees the first P + i + 1 keys. */
    for (int i = row_begin; i < row_end; i++)
        kvq_ref_attention(K, row, head_dim, head_dim, V, row, head_dim, head_dim,
                          (int)(P + i + 1), n_kv_heads,
                          q_new + (long)i * n_q_heads * head_dim, n_q_heads, (double)scale,
                          out + (long)i * n_q_heads * head_dim);
    free(K);
    free(V);
    return 0;
}

int kvq_ref_block_scores_seq(const uint8_t *pool, const uint8_t *bits, const uint64_t *k_offset,
                             int n_blocks, const uint16_t *rope, int rope_dim, int n_kv_heads,
                             int head_dim, const uint16_t *q, int n_q_heads, double scale,
                             double *scores)
{
    if (!dims_ok(n_kv_heads, head_dim) || n_blocks < 0 || n_q_heads < 1 || n_q_heads % n_kv_heads) return -1;
    const int G = n_q_heads / n_kv_heads, dk = head_dim + rope_dim;
    const size_t T = (size_t)64 * n_blocks;
    float *K = malloc((T + 1) * n_kv_heads * head_dim * sizeof(float));
    if (!K) return -1;
    int rc = kvq_ref_restore_seq(pool, bits, k_offset, n_blocks, NULL, 0, n_kv_heads, head_dim, K);
    if (rc) { free(K); return rc; }
    for (int j = 0; j < n_blocks; j++) {
        double best = -INFINITY;
        for (int t = 64 * j; t < 64 * j + 64; t++) {
            for (int h = 0; h < n_q_heads; h++) {
                const int g = h / G;
                const float *k = K + ((size_t)t * n_kv_heads + g) * head_dim;
                const uint16_t *qh = q + (size_t)h * dk;
                double dot = 0.0;
                for (int d = 0; d < head_dim; d++) dot += (double)kvq_ref_bf16_to_f32(qh[d]) * (double)k[d];
                for (int d = 0; d < rope_dim; d++)
                    dot += (double)kvq_ref_bf16_to_f32(qh[head_dim + d]) *
                           (double)kvq_ref_bf16_to_f32(rope[((size_t)t * n_kv_heads + g) * rope_dim + d]);
                const double sc = scale * dot;
                if (sc > best) best = sc;
            }
        }
        scores[j] = best;
    }
    free(K);
    return 0;
}

/* Per-token pieces of the block bound for query head h: the score term
 * sum_grp rK * sum|q| (without the width factor), the value term
 * sqrt(sum_grp rV^2), and the value norm. */
static void sens_terms(const uint16_t *k, const uint16_t *v, int H, int D, const uint16_t *qh, int g, int t,
                       double *kt, double *vt, double *vn)
{
    double ks = 0.0, vs = 0.0, nn = 0.0;
    for (int grp = 0; grp < D / 64; grp++) {
        double kmn = INFINITY, kmx = -INFINITY, vmn = INFINITY, vmx = -INFINITY, qa = 0.0;
        for (int d = 64 * grp; d < 64 * grp + 64; d++) {
            const double kk = kvq_ref_bf16_to_f32(k[((size_t)t * H + g) * D + d]);
            const double vv = kvq_ref_bf16_to_f32(v[((size_t)t * H + g) * D + d]);
            kmn = fmin(kmn, kk); kmx = fmax(kmx, kk);
            vmn = fmin(vmn, vv); vmx = fmax(vmx, vv);
            qa += fabs((double)kvq_ref_bf16_to_f32(qh[d]));
            nn += vv * vv;
        }
        ks += (kmx - kmn) * qa;
        vs += (vmx - vmn) * (vmx - vmn);
    }
    *kt = ks;
    *vt = sqrt(vs);
    *vn = sqrt(nn);
}

int kvq_ref_block_sensitivity(const uint16_t *k, const uint16_t *v, int n_kv_heads, int head_dim,
                              const uint16_t *q, int n_q_heads, double scale, double *S)
{
    if (!dims_ok(n_kv_heads, head_dim) || n_q_heads < 1 || n_q_heads % n_kv_heads) return -1;
    const int G = n_q_heads / n_kv_heads;
    double total = 0.0;
    for (int h = 0; h < n_q_heads; h++) {
        double kmax = 0.0, vmax_t = 0.0, vnorm = 0.0;
        for (int t = 0; t < 64; t++) {
            double kt, vt, vn;
            sens_terms(k, v, n_kv_heads, head_dim, q + (size_t)h * head_dim, h / G, t, &kt, &vt, &vn);
            kmax = fmax(kmax, kt);
            vmax_t = fmax(vmax_t, vt);
            vnorm = fmax(vnorm, vn);
        }
        total += 2.0 * vnorm * fabs(scale) * kmax + 8.0 * vmax_t;
    }
    *S = total;
    return 0;
}

double kvq_ref_block_error_bound(const uint16_t *k, const uint16_t *v, int n_kv_heads, int head_dim,
                                 const uint16_t *q, int n_q_heads, int h, double scale, int bits)
{
    const int G = n_q_heads / n_kv_heads;
    const double c = 1.0 / (2.0 * (double)((1 << bits) - 1));
    double kmax = 0.0, vmax_t = 0.0, vnorm = 0.0;
    for (int t = 0; t < 64; t++) {
        double kt, vt, vn;
        sens_terms(k, v, n_kv_heads, head_dim, q + (size_t)h * head_dim, h / G, t, &kt, &vt, &vn);
        kmax = fmax(kmax, kt);
        vmax_t = fmax(vmax_t, vt);
        vnorm = fmax(vnorm, vn);
    }
    return (exp(2.0 * fabs(scale) * c * kmax) - 1.0) * vnorm + 8.0 * c * vmax_t;
}
