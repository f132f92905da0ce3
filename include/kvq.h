/*
 * kvq.h — C ABI of the MI355X (gfx950) quantized KV-cache library.
 *
 * The library quantizes a bf16 key/value cache into packed low-bit blocks and
 * runs attention directly over those blocks, dequantizing on the fly.  The
 * problem statement comes from these pages:
 *
 *   [QKVShare] QKVShare: Quantized KV-Cache Handoff for Multi-Agent On-Device
 *              LLMs, section Metodologia — a CacheCard packs quantized KV
 *              groups with per-token widths and metadata; the receiver rebuilds
 *              16-bit past_key_values and a fused quantized attention kernel is
 *              left as future work.
 *   [AgentMem] Agent Memory Below the Prompt: Persistent Q4 KV Cache for
 *              Multi-Agent LLM Inference on Edge Devices (arXiv 2603.04428),
 *              Abstract — per-agent 4-bit caches in a block pool, restored
 *              directly into the attention layer, batched inference over several
 *              agents' quantized caches, and cross-phase context injection.
 *   [CoMixKV]  Coordinated Mixed-Precision KV Cache Quantization for Efficient
 *              LLM-based Multi-agent Systems (arXiv 2611.10096), Abstract —
 *              widths chosen per agent and layer apply only to newly quantized
 *              blocks; recent states stay in native precision.
 *
 * Format (the pages give none; this library's reading):
 *   group    64 consecutive elements along head_dim of one (token, head)
 *   codes    q = clamp(rint((x - bias) * (1/scale)), 0, 2^b - 1), scale =
 *            (max - min)/(2^b - 1) and bias = min rounded to fp16; codes are
 *            computed against the stored fp16 values; a zero min/max is +0
 *   packing  little-endian bitstream: code i at bits [b*i, b*i+b) of 2b uint32
 *            words per group
 *   block    64 tokens x all KV heads of one sequence, one width b in
 *            {2,3,4,8}: codes [H][64][D*b/32] uint32, then meta [H][64][D/64]
 *            of {fp16 scale, fp16 bias}; H*D*(8b+4) bytes, 256-byte aligned
 *   window   the newest tokens of a sequence, kept as bf16 [W][H][D]
 *   restore  x_hat = fma(code, scale, bias) in fp32
 *
 * Conventions of every entry point:
 *   - returns KVQ_OK (0) or a negative KVQ_E* code; kvq_strerror names it;
 *   - every argument check runs on the host before any HIP call, so an error
 *     return launches nothing and leaves device memory untouched;
 *   - work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream); nothing is allocated, no state is kept,
 *     and calls are thread-safe;
 *   - all data pointers are device pointers owned by the caller, except the
 *     descriptor structs themselves, which live in host memory and are read
 *     only during the call;
 *   - device tables (lengths, widths, offsets) are trusted: lengths are clamped
 *     to the declared capacities, but a width outside {2,3,4,8} or an offset
 *     outside the pool is a precondition violation (the output is then
 *     unspecified);
 *   - NaN, Inf or |x| > 65504 in a cache input is a precondition violation.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_OK            0
#define KVQ_EINVAL       (-1)   /* a null pointer, bad size or misalignment */
#define KVQ_ENOSPC       (-2)   /* workspace smaller than the matching *_workspace size */
#define KVQ_EUNSUPPORTED (-3)   /* valid request outside what the kernels implement */
#define KVQ_EHIP         (-4)   /* the HIP runtime reported an error at launch */

#define KVQ_OUT_BF16 0
#define KVQ_OUT_F32  1

/* Token bookkeeping of one layer for a batch of A sequences (agents).  The K
 * and V caches of the layer share it: one width per (sequence, block), used
 * for both, and the same block/window counts. */
typedef struct kvq_layout {
    int32_t n_seqs;            /* A >= 1 */
    int32_t n_heads;           /* KV heads H >= 1 */
    int32_t head_dim;          /* D: quantized dims per head, multiple of 64, 64..512 */
    int32_t max_blocks;        /* >= 0: row stride of bits[] and offset[]; n_blocks[a] <= max_blocks */
    int32_t window_cap;        /* >= 0: row stride (tokens) of the windows; n_window[a] <= window_cap */
    const int32_t *n_blocks;   /* device int32 [A]: quantized 64-token blocks of each sequence */
    const int32_t *n_window;   /* device int32 [A]: bf16 window tokens; NULL allowed if window_cap == 0 */
    const uint8_t *bits;       /* device uint8 [A][max_blocks]: width of each block (2, 3, 4 or 8) */
} kvq_layout;

/* Storage of one of K or V of a layer. */
typedef struct kvq_store {
    const uint64_t *offset;    /* device uint64 [A][max_blocks]: byte offset of each block in pool, multiple of 256 */
    uint8_t *pool;             /* device byte pool, 256-byte aligned */
    uint16_t *window;          /* device bf16 [A][window_cap][H][D]; NULL allowed if window_cap == 0 */
} kvq_store;

/* Bytes of one block payload of `bits` width for n_heads x head_dim, i.e.
 * n_heads*head_dim*(8*bits+4); 0 if an argument is unsupported.  With a group
 * of 64 and 32 bits of metadata this is (bits + 0.5)/16 of the bf16 size: 4-bit
 * gives 28.125 %, the 4.5-bit figure printed as 28.1 % on KVarN su llama.cpp
 * (section Dettagli Tecnici e Risultati dei Benchmark KLD), and 4x the capacity
 * of 16-bit before metadata (AgentMem, Abstract). */
uint64_t kvq_block_bytes(int32_t bits, int32_t n_heads, int32_t head_dim);

/* Quantize (AgentMem: persist each agent's cache in 4-bit form; CoMixKV: one
 * width per new block).  For every sequence a and block j < n_blocks[a], read
 * the 64 bf16 tokens src[a][64j .. 64j+63][H][D] (token-major, as a model emits
 * K or V; sequence a starts at src + a*src_seq_tokens*H*D) and write the block
 * payload of width bits[a][j] at dst->pool + dst->offset[a][j].  Windows are
 * not touched.  Codes, scales and biases are bit-exact to the format above.
 *   src_seq_tokens >= 64*max_blocks; src 16-byte aligned.
 * Errors: KVQ_EINVAL (null L/dst/src/tables, bad dims, misalignment),
 *         KVQ_EHIP. */
int kvq_quantize(const kvq_layout *L, const kvq_store *dst, const uint16_t *src,
                 int64_t src_seq_tokens, void *stream);

/* kvq_quantize of a layer's K and V caches in one launch (QKVShare,
 * Metodologia: an agent's K and V groups are quantized together when its
 * cache is packed for handoff).  The result is bit-exact to kvq_quantize(L, K,
 * k_src, ...) followed by kvq_quantize(L, V, v_src, ...); both sources share
 * src_seq_tokens and the layout's widths.  V == NULL quantizes K alone
 * (v_src ignored), for a latent cache.
 * Errors: as kvq_quantize; KVQ_EUNSUPPORTED when 2*n_seqs exceeds 65535. */
int kvq_quantize_kv(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *k_src,
                    const uint16_t *v_src, int64_t src_seq_tokens, void *stream);

/* Quantize on append, the window roll (CoMixKV, Abstract: a width is chosen
 * only for newly quantized blocks and the most recent states stay in native
 * precision; AgentMem, Abstract: each agent's cache keeps growing as the agent
 * works).  For every sequence a, with nb = n_blocks[a] and W = n_window[a],
 * the token stream
 *     T = window[a][0 .. W) ++ new[a][0 .. n_new)
 * is cut into k = (W + n_new - keep_recent) / 64 new blocks (integer
 * division; none when W + n_new <= keep_recent), T[64i .. 64i+63] becoming
 * block nb + i at width bits[a][nb+i] and pool offset offset[a][nb+i] (table
 * entries the caller fills beforehand), and a window holding the remaining
 * W + n_new - 64k tokens T[64k ..] (keep_recent .. keep_recent+63 of them
 * once a block has been cut).  Then n_blocks_out[a] = nb + k and
 * n_window_out[a] = W + n_new - 64k.  Block payloads are bit-exact to
 * kvq_quantize of the same rows; window rows are copied unchanged.
 *   k_new, v_new  bf16 [A][n_new][H][D], 16-byte aligned; V NULL for a latent
 *                 cache (K only; v_new ignored).
 *   rope          NULL, or bf16 [A][64*max_blocks + window_cap][H][rope_dim]
 *                 (rope_dim 64): raw key dims, one row per token position as
 *                 kvq_attend_decode reads them (token t of sequence a at row
 *                 t), so the roll moves none of them: new token i is written
 *                 at row 64*nb + W + i from rope_new bf16 [A][n_new][H][rope_dim].
 *   n_blocks_out, n_window_out  device int32 [A]; they may be L->n_blocks and
 *                 L->n_window (written after every read, in a launch of their
 *                 own); n_window_out may be NULL when window_cap == 0.  Outputs
 *                 that overlap neither input count array are written by the
 *                 window launch, one launch fewer per call (a caller can keep
 *                 two count arrays and alternate them between calls).
 *   keep_recent   >= 0 with keep_recent + 63 <= window_cap, so the window
 *                 always fits; with window_cap == 0, keep_recent must be 0
 *                 and n_new a multiple of 64.
 * Device preconditions: nb + k <= max_blocks and W <= window_cap.  Blocks past
 * max_blocks and window rows past window_cap are never written.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (rope_dim other than 0 or 64),
 *         KVQ_EHIP. */
int kvq_append(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
               const uint16_t *k_new, const uint16_t *v_new,
               uint16_t *rope, const uint16_t *rope_new, int32_t rope_dim,
               int32_t n_new, int32_t keep_recent,
               int32_t *n_blocks_out, int32_t *n_window_out, void *stream);

/* The counts kvq_append leaves, computed on the host from host copies of
 * the counts it starts from (the same window-roll rule and clamping, one
 * definition shared with the append kernels), so a caller can keep host
 * mirrors of the device counts without a device-to-host copy.
 *   n_blocks, n_window  host int32 [n_seqs]: counts before the append
 *                       (n_window may be NULL when window_cap == 0)
 *   n_blocks_out, n_window_out  host int32 [n_seqs]; may alias the inputs
 * Other arguments as for kvq_append with a layout of these capacities.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED. */
int kvq_append_counts(int32_t n_seqs, int32_t max_blocks, int32_t window_cap, const int32_t *n_blocks,
                      const int32_t *n_window, int32_t n_new, int32_t keep_recent, int32_t *n_blocks_out,
                      int32_t *n_window_out);

/* Restore (QKVShare injection path: rebuild 16-bit key/value rows).  For
 * every sequence a write dst[a][t][H][D] for t < 64*n_blocks[a] + n_window[a]:
 * dequantized blocks first (fma(code, scale, bias) in fp32, then rounded to
 * bf16 nearest-even when out_dtype is KVQ_OUT_BF16, or stored as fp32 for
 * KVQ_OUT_F32), then the window tokens copied unchanged (or widened).  Rows
 * beyond a sequence's length are not written.
 *   dst_seq_tokens >= 64*max_blocks + window_cap; dst 16-byte aligned.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (out_dtype), KVQ_EHIP. */
int kvq_dequantize(const kvq_layout *L, const kvq_store *src, int32_t out_dtype, void *dst,
                   int64_t dst_seq_tokens, void *stream);

/* CacheCard image of one sequence (QKVShare, Metodologia: a CacheCard packs
 * an agent's quantized KV groups with their widths and metadata for handoff;
 * AgentMem, Abstract: per-agent 4-bit caches persisted and reloaded).  The
 * image concatenates, in this order: the K block payloads (block j is
 * kvq_block_bytes(bits[j], H, D) bytes, j < n_blocks, no padding), the V
 * block payloads (absent for a latent cache), the K window rows bf16
 * [n_window][H][D], the V window rows (absent for a latent cache), the rope
 * rows bf16 [64*n_blocks + n_window][H][rope_dim] (absent when rope_dim is 0),
 * and the widths uint8 [n_blocks].  Every segment but the last is a multiple
 * of 128 bytes.
 *
 * kvq_card_bytes: the image size for these counts, from host copies of the
 * sequence's widths (bits_host [n_blocks]); 0 for unsupported arguments. */
uint64_t kvq_card_bytes(int32_t n_heads, int32_t head_dim, int32_t rope_dim, int32_t has_v,
                        int32_t n_blocks, const uint8_t *bits_host, int32_t n_window);

/* Gather sequence seq of the cache into image (device memory, 16-byte
 * aligned), with the counts and widths the device tables hold.  Bytes past
 * image_bytes are not written.  V NULL: latent cache.  rope as in
 * kvq_attend_decode (rows by token position).
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (rope_dim), KVQ_EHIP. */
int kvq_card_gather(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *rope,
                    int32_t rope_dim, int32_t seq, void *image, uint64_t image_bytes, void *stream);

/* Scatter an image back into sequence seq: the caller first sets the
 * sequence's counts and widths (and pool offsets sized for those widths) in
 * the device tables to the card's; the image's own width segment is not read.
 * Bytes past image_bytes are not read.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (rope_dim), KVQ_EHIP. */
int kvq_card_scatter(const kvq_layout *L, const kvq_store *K, const kvq_store *V, uint16_t *rope,
                     int32_t rope_dim, int32_t seq, const void *image, uint64_t image_bytes, void *stream);

/* Width-allocation sensitivity (CoMixKV, Abstract: sensitivity from a local
 * attention-error bound using recent queries, keys and values; this
 * library's bound, from the per-group reconstruction bound s/2 with s =
 * range / (2^b - 1)).  For sequence a and block i < n_blocks (rows 64i ..
 * 64i+63 of k and v, bf16 [A][seq_tokens][H][D], 16-byte aligned), with
 * scale = softmax_scale (finite, > 0):
 *     S[a][i] = sum_h ( 2 Vmax_g scale max_t sum_grp rK[t][g][grp] sum_{d in grp} |q[a][h][d]|
 *                       + 8 max_t sqrt(sum_grp rV[t][g][grp]^2) ),   g = h / (n_q_heads/H)
 * rK, rV: max - min of a 64-element group; Vmax_g: the largest V row norm of
 * KV head g in the block.  Quantizing the block at width b moves attention
 * restricted to the block by about c(b) S_h per head, c(b) = 1/(2(2^b-1))
 * (to first order in c).  q bf16 [A][n_q_heads][D]; S fp32 device [A][n_blocks].
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (more than 1024 query heads), KVQ_EHIP. */
int kvq_block_sensitivity(const uint16_t *k, const uint16_t *v, int32_t n_seqs, int64_t seq_tokens,
                          int32_t n_blocks, int32_t n_heads, int32_t head_dim, const uint16_t *q,
                          int32_t n_q_heads, float softmax_scale, float *S, void *stream);

/* Budgeted widths (host; CoMixKV: joint allocation under a shared memory
 * budget, applied to newly quantized blocks).  Every block starts at 2 bits;
 * repeatedly the (block, next width in 2 -> 3 -> 4 -> 8) step with the
 * largest S[i] (c(b) - c(b')) per extra byte is taken among the steps that
 * still fit budget_bytes (equal ratios: lower index first), until none fits.
 * Block bytes are kvq_block_bytes(b, n_heads, head_dim).  S and widths are
 * host arrays of n entries.
 * Errors: KVQ_EINVAL (bad sizes, or a budget below the all-2-bit size). */
int kvq_allocate_widths(const float *S, int64_t n, int32_t n_heads, int32_t head_dim,
                        uint64_t budget_bytes, uint8_t *widths);

/* Workspace bytes kvq_attend_decode needs for this layout and head count
 * (written to *bytes).  Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED. */
int kvq_decode_workspace(const kvq_layout *L, int32_t n_q_heads, int32_t rope_dim, size_t *bytes);

/* Batched decode attention over quantized caches (AgentMem: batched
 * inference over several agents' quantized caches, restored directly into the
 * attention layer; QKVShare: the fused quantized attention kernel).  One query
 * token per sequence.  Query head h of sequence a attends, with scores
 * softmax_scale * <q, k>, to every cached token of KV head h / (n_q_heads/H):
 * the 64*n_blocks[a] quantized tokens, then the n_window[a] window tokens.
 * The result equals softmax attention over the restored rows, within fp32
 * rounding; an empty sequence gives zeros.
 *   softmax_scale: finite and > 0 (attention scales are positive; the
 *        kernels take the running maximum of the scaled scores from the
 *        maximum of the raw ones).
 *   q    bf16 [A][n_q_heads][D + rope_dim]
 *   out  fp32 [A][n_q_heads][D]
 *   V    NULL for latent attention: the values are the restored K rows (the
 *        first D dims of each key), as in a multi-head latent cache.
 *   rope NULL or bf16 [A][64*max_blocks + window_cap][H][rope_dim]: raw key
 *        dims appended after the D quantized ones (rope_dim 0 or 64), one row
 *        per token position (token t of sequence a, blocks then window, at
 *        row t).
 *   n_q_heads: a multiple of H with n_q_heads/H <= 16.
 *   workspace: >= kvq_decode_workspace bytes, 256-byte aligned; calls that
 *        share a workspace must not overlap in time.
 * Errors: KVQ_EINVAL (also softmax_scale <= 0), KVQ_ENOSPC, KVQ_EUNSUPPORTED,
 *         KVQ_EHIP. */
int kvq_attend_decode(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                      const uint16_t *rope, int32_t rope_dim, const uint16_t *q,
                      int32_t n_q_heads, float softmax_scale, float *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* kvq_attend_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and kernels, with the split partials in
 * a library-owned device array of 16 MiB per GPU (taken once per device on
 * the first call there, held until the process ends) instead of a caller
 * workspace.  Arguments as for kvq_attend_decode without the workspace.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give undefined results.
 * The array needs no clearing: each call writes every partial it reads.
 * Allocates nothing (no hipMalloc, no allocating library call).
 * Errors: as kvq_attend_decode; KVQ_ENOSPC when the call's workspace
 *         (kvq_decode_workspace) exceeds 16 MiB; KVQ_EHIP when the array's
 *         address cannot be taken on the current device. */
int kvq_attend_decode_static(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                             const uint16_t *rope, int32_t rope_dim, const uint16_t *q,
                             int32_t n_q_heads, float softmax_scale, float *out, void *stream);

/* Workspace bytes kvq_attend_decode_topk needs (written to *bytes).
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED. */
int kvq_topk_workspace(const kvq_layout *L, int32_t n_q_heads, int32_t rope_dim, int32_t top_k,
                       size_t *bytes);

/* Sparse decode over the top-K blocks (Reasoning-Aware Error-Bounded
 * KV-Cache Compression and Sparse Attention for Long-Context LLMs, section 2C:
 * the active set is the top-K entries by a query-aware score built on the
 * query-key compatibility; section 2B: the output then differs from full
 * attention by at most 2 * max_t |v_t| * (attention mass left out)).
 * For each sequence a, block j < n_blocks[a] scores
 *     max over its 64 tokens t and the sequence's query heads h of
 *     softmax_scale * <q[a][h], k_t of KV head h / G>
 * (restored keys, plus the rope dims when rope_dim is 64, in fp32).  The
 * min(top_k, n_blocks[a]) highest-scoring blocks (equal scores: lower index
 * first) and the whole bf16 window form the active set; the result is
 * kvq_attend_decode restricted to it (the same kernels run over a compacted
 * copy of the tables in the workspace).
 *   selected  NULL or device int32 [A][top_k]: the kept block indices in
 *             ascending order, -1 past min(top_k, n_blocks[a]).
 *   top_k >= 1; max_blocks <= 16384 (0 allowed: a window-only layout keeps
 *   no block and `selected` is all -1); (n_q_heads/H) * (head_dim + rope_dim)
 *   <= 9216.  Other arguments (softmax_scale > 0) as for
 *   kvq_attend_decode.
 * Errors: KVQ_EINVAL, KVQ_ENOSPC, KVQ_EUNSUPPORTED, KVQ_EHIP. */
int kvq_attend_decode_topk(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                           const uint16_t *rope, int32_t rope_dim, const uint16_t *q,
                           int32_t n_q_heads, float softmax_scale, int32_t top_k, float *out,
                           int32_t *selected, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes kvq_attend_chunk needs (written to *bytes). */
int kvq_chunk_workspace(const kvq_layout *L, int32_t n_q_heads, int32_t n_new, size_t *bytes);

/* Chunk attention for new-phase tokens over a restored cache (AgentMem:
 * cross-phase context injection that accumulates attention state without
 * recomputing the earlier phase).  For every sequence a, new token i (0 <= i <
 * n_new) and query head h, attend to every cached token of KV head
 * h / (n_q_heads/H) (blocks, then window) and to new tokens 0..i.
 *   q_new bf16 [A][n_new][n_q_heads][D]
 *   k_new, v_new bf16 [A][n_new][H][D]   (unquantized)
 *   out  fp32 [A][n_new][n_q_heads][D]
 *   n_q_heads: a multiple of H with n_q_heads/H <= 16.
 *   softmax_scale: finite and > 0.
 *   workspace: >= kvq_chunk_workspace bytes, 256-byte aligned (no zeroing
 *        needed).
 * Errors: KVQ_EINVAL (also softmax_scale <= 0), KVQ_ENOSPC, KVQ_EUNSUPPORTED,
 *         KVQ_EHIP. */
int kvq_attend_chunk(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                     const uint16_t *q_new, const uint16_t *k_new, const uint16_t *v_new,
                     int32_t n_new, int32_t n_q_heads, float softmax_scale, float *out,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Static text for a status code. */
const char *kvq_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif
