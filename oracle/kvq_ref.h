/*
 * kvq_ref — CPU oracle for group-wise quantized KV caches.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it, and the two share no
 * code, header, table or constant.
 *
 * What it computes, and where the pages state it:
 *
 *  - Quantization of a K/V cache into a low-bit format with per-group
 *    metadata ("quantized KV groups" in the CacheCard, QKVShare:
 *    Quantized KV-Cache Handoff for Multi-Agent On-Device LLMs, section
 *    Metodologia; "4-bit quantized format" / Q4, Agent Memory Below the
 *    Prompt, arXiv 2603.04428, Abstract).  The pages give no formula.  The
 *    affine min/max reading (scale and offset, as for the "asymmetric" KIVI
 *    entry in that page's related-paper list) is fixed here step by step:
 *    kvq_ref_quantize_group documents each step.
 *  - Mixed widths per block, written only when a block is created, with the
 *    most recent tokens kept in native precision (Coordinated Mixed-Precision
 *    KV Cache Quantization, arXiv 2611.10096, Abstract).
 *  - Restoring: dequantize back to 16-bit key/value rows before an ordinary
 *    attention pass (QKVShare, Metodologia: the injection path rebuilds the
 *    FP16 past_key_values from the CacheCard).
 *  - Attention over the restored cache, batched over agents and used for
 *    new-phase queries (Agent Memory Below the Prompt, Abstract: a batched
 *    quantized cache and cross-phase context injection).  Because the pages'
 *    prototype dequantizes and then runs ordinary attention, the oracle is
 *    exactly that composition, in fp64.
 *
 * Every function works on host memory and one sequence at a time.
 * Layouts (little-endian host):
 *
 *   source rows      bf16 [T][H][D]             token-major, as a model emits K or V
 *   block payload    codes [H][64][D*b/32] u32, then meta [H][64][D/64] of
 *                    {fp16 scale, fp16 bias} (scale at the lower address);
 *                    bytes = H*D*(8b+4), a multiple of 256 when D % 64 == 0
 *   window           bf16 [W][H][D]             the newest tokens, unquantized
 *   rope             bf16 [T][H][R]             raw key dims appended after D
 *
 * Parity status: every function here is pinned by tests/test_oracle_*.py
 * (closed forms, invariants, library conversions, brute force).  None is
 * "parity unpinned".
 */
#ifndef KVQ_REF_H
#define KVQ_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- IEEE 754 conversions (written from the format definitions) -------- */
float    kvq_ref_bf16_to_f32(uint16_t h);
uint16_t kvq_ref_f32_to_bf16(float f);  /* round to nearest even; NaN stays NaN */
float    kvq_ref_f16_to_f32(uint16_t h);
uint16_t kvq_ref_f32_to_f16(float f);   /* round to nearest even, subnormals, overflow to inf */

/* Vector forms used by the tests (n elements). */
void kvq_ref_f32_to_f16_n(const float *x, uint16_t *y, size_t n);
void kvq_ref_f32_to_bf16_n(const float *x, uint16_t *y, size_t n);
void kvq_ref_f16_to_f32_n(const uint16_t *x, float *y, size_t n);

/* ---- one 64-element group ------------------------------------------------ */
/* Quantize 64 bf16 values at width bits (2, 3, 4 or 8).  Writes 2*bits
 * uint32 words of codes, the fp16 scale and the fp16 bias.  Returns 0, or -1
 * for an unsupported width. */
int  kvq_ref_quantize_group(const uint16_t *x, int bits, uint32_t *words,
                            uint16_t *scale_h, uint16_t *bias_h);
/* Codes of a group as integers (64 of them). */
int  kvq_ref_unpack_group(const uint32_t *words, int bits, uint8_t *codes);
/* Pack 64 integer codes (each < 2^bits) into 2*bits words. */
int  kvq_ref_pack_group(const uint8_t *codes, int bits, uint32_t *words);
/* Dequantize a group to fp32 (one fused multiply-add per element). */
int  kvq_ref_dequantize_group(const uint32_t *words, int bits, uint16_t scale_h,
                              uint16_t bias_h, float *out);

/* ---- block pool ---------------------------------------------------------- */
/* Bytes of one 64-token block payload; 0 for unsupported arguments. */
uint64_t kvq_ref_block_bytes(int bits, int n_heads, int head_dim);

/* Quantize the first 64*n_blocks tokens of x [T][H][D] into the blocks of
 * one sequence: block j has width bits[j] and starts at pool + offset[j]. */
int kvq_ref_quantize_seq(const uint16_t *x, int n_heads, int head_dim, int n_blocks,
                         const uint8_t *bits, const uint64_t *offset, uint8_t *pool);

/* Append n_new tokens to one sequence, the window roll (Coordinated
 * Mixed-Precision KV Cache Quantization, arXiv 2611.10096, Abstract: widths
 * are chosen only for newly quantized blocks and recent states stay in native
 * precision).  The stream T = window[0 .. n_window) ++ x_new[0 .. n_new) is
 * cut into k = (n_window + n_new - keep) / 64 new blocks (none when
 * n_window + n_new <= keep): block n_blocks + i receives T[64i .. 64i+63] at
 * width bits[n_blocks + i], at pool + offset[n_blocks + i]; the window then
 * holds T[64k ..].  v_pool NULL: a latent cache (K only).  With rope_dim > 0,
 * rope [64*max_blocks + window_cap][H][rope_dim] holds one row per token
 * position (as the decode reads it), so only the new tokens' rows are written:
 * new token i at row 64*n_blocks + n_window + i, from rope_new
 * [n_new][H][rope_dim].  Writes the new counts.
 * Returns 0, or -1 when the result would not fit max_blocks or window_cap
 * (nothing is written then). */
int kvq_ref_append_seq(uint8_t *k_pool, uint8_t *v_pool, const uint8_t *bits,
                       const uint64_t *k_offset, const uint64_t *v_offset,
                       int max_blocks, int n_blocks, uint16_t *k_window, uint16_t *v_window,
                       int window_cap, int n_window, int n_heads, int head_dim,
                       const uint16_t *k_new, const uint16_t *v_new, int n_new, int keep,
                       uint16_t *rope, const uint16_t *rope_new, int rope_dim,
                       int *n_blocks_out, int *n_window_out);

/* Restore one sequence to fp32 rows out [64*n_blocks + n_window][H][D]:
 * dequantized blocks first, then the bf16 window. */
int kvq_ref_restore_seq(const uint8_t *pool, const uint8_t *bits, const uint64_t *offset,
                        int n_blocks, const uint16_t *window, int n_window,
                        int n_heads, int head_dim, float *out);

/* ---- attention (fp64) ---------------------------------------------------- */
/* Softmax attention of n_q_heads query rows over T keys.
 *   K   fp32, key t of KV head g at K[t*k_tok_stride + g*k_head_stride + d], d < dk
 *   V   fp32, same with v_* strides, d < dv
 *   q   bf16 [n_q_heads][dk]
 *   out fp32 [n_q_heads][dv]
 * Query head h reads KV head h / (n_q_heads / n_kv_heads).  With T == 0 the
 * output is zero.  Scores are scale * <q, k>, the softmax subtracts the row
 * maximum and uses libm exp. */
void kvq_ref_attention(const float *K, long k_tok_stride, long k_head_stride, int dk,
                       const float *V, long v_tok_stride, long v_head_stride, int dv,
                       int T, int n_kv_heads, const uint16_t *q, int n_q_heads,
                       double scale, float *out);

/* Decode step for one sequence: attend the query rows to every cached token
 * (blocks, then window).  V blocks are given by v_offset; if v_offset is NULL
 * the values are the dequantized key latent (first head_dim dims of each key,
 * multi-head latent attention).  If rope_dim > 0, each key is extended by
 * rope[t][g][0..rope_dim) (bf16) and q has head_dim + rope_dim dims.
 * out fp32 [n_q_heads][head_dim]. */
int kvq_ref_attend_decode_seq(const uint8_t *pool, const uint8_t *bits,
                              const uint64_t *k_offset, const uint64_t *v_offset,
                              int n_blocks, const uint16_t *k_window, const uint16_t *v_window,
                              int n_window, const uint16_t *rope, int rope_dim,
                              int n_kv_heads, int head_dim, const uint16_t *q, int n_q_heads,
                              float scale, float *out);

/* Chunk step for one sequence: new query token i (row_begin <= i < row_end)
 * attends to every restored token and to new tokens 0..i.
 *   q_new bf16 [n_new][n_q_heads][head_dim]
 *   k_new, v_new bf16 [n_new][n_kv_heads][head_dim]
 *   out fp32 [n_new][n_q_heads][head_dim]; only rows in [row_begin,row_end) are written. */
int kvq_ref_attend_chunk_seq(const uint8_t *pool, const uint8_t *bits,
                             const uint64_t *k_offset, const uint64_t *v_offset,
                             int n_blocks, const uint16_t *k_window, const uint16_t *v_window,
                             int n_window, int n_kv_heads, int head_dim,
                             const uint16_t *q_new, const uint16_t *k_new, const uint16_t *v_new,
                             int n_new, int n_q_heads, float scale,
                             int row_begin, int row_end, float *out);

/* Block scores for top-K sparse decode (Reasoning-Aware Error-Bounded
 * KV-Cache Compression and Sparse Attention for Long-Context LLMs, section
 * 2C: the active set is the top-K entries by a score built on the
 * instantaneous query-key compatibility).  The entry is a 64-token block; its
 * score is the largest scale * <q_h, k_t> over the block's tokens t and all
 * query heads h (query head h reads KV head h / (n_q_heads / n_kv_heads)),
 * with the restored keys of kvq_ref_restore_seq and, if rope_dim > 0, the
 * rope dims (rope [64*n_blocks][H][rope_dim], q rows of head_dim + rope_dim).
 * fp64.  scores[n_blocks]. */
int kvq_ref_block_scores_seq(const uint8_t *pool, const uint8_t *bits, const uint64_t *k_offset,
                             int n_blocks, const uint16_t *rope, int rope_dim, int n_kv_heads,
                             int head_dim, const uint16_t *q, int n_q_heads, double scale,
                             double *scores);

/* Width-allocation sensitivity of 64-token blocks (Coordinated
 * Mixed-Precision KV Cache Quantization, arXiv 2611.10096, Abstract: a
 * sensitivity from a local attention-error bound using recent queries, keys
 * and values; the formula is this library's, derived from the reconstruction
 * bound |x_hat - x| <= s/2, s = range / (2^b - 1), of each 64-element group).
 * For query head h (KV head g) and block tokens t, a key error within that
 * bound moves the score by at most
 *     eps_t(b) = scale * sum_groups (rK_t,grp / (2(2^b-1))) * sum_{d in grp} |q_h,d|
 * and a value row by at most |dv_t|(b) = sqrt(64 * sum_grp (rV_t,grp/(2(2^b-1)))^2);
 * attention restricted to the block then moves by at most
 *     (exp(2 max_t eps_t) - 1) * Vmax + max_t |dv_t|        (Vmax = max_t |v_t|)
 * which to first order is c(b) * S_h, c(b) = 1/(2(2^b-1)),
 *     S_h = 2 Vmax scale max_t sum_grp rK_t,grp sum_{d in grp}|q_h,d| + 8 max_t sqrt(sum_grp rV_t,grp^2).
 * The block's sensitivity is S = sum_h S_h.  rK, rV: max - min of the group
 * (fp32 from bf16).  k, v bf16 [64][H][D] (one block), q bf16 [n_q_heads][D].
 * Writes S; returns 0. */
int kvq_ref_block_sensitivity(const uint16_t *k, const uint16_t *v, int n_kv_heads, int head_dim,
                              const uint16_t *q, int n_q_heads, double scale, double *S);

/* The bound itself at width bits for query head h (the exponential form
 * above, not its first-order part). */
double kvq_ref_block_error_bound(const uint16_t *k, const uint16_t *v, int n_kv_heads, int head_dim,
                                 const uint16_t *q, int n_q_heads, int h, double scale, int bits);

/* Threads the OpenMP runtime uses for the parallel loops (1 without OpenMP). */
int kvq_ref_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
