// Internal declarations shared by the host API and the HIP kernels of kvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

// Per-layer token bookkeeping, passed by value to kernels.
struct Tables {
    int A, H, D, max_blocks, window_cap;
    const int32_t *n_blocks;
    const int32_t *n_window;   // may be null (no window)
    const uint8_t *bits;
};

// Storage of one of K or V.
struct Store {
    const uint64_t *offset;
    const uint8_t *pool;
    const uint16_t *window;
};

// One launch quantizes n_tensors (1 or 2: K then V) caches of one layout.
struct QuantArgs {
    Tables t;
    const uint64_t *offset[2];
    uint8_t *pool[2];
    const uint16_t *src[2];
    int64_t src_seq_tokens;
    int n_tensors;
    int j0;             // first block of this launch (set by the launcher)
};

struct DequantArgs {
    Tables t;
    Store s;
    void *dst;
    int64_t dst_seq_tokens;
    int out_f32;
    int j0;             // first block or window tile of this launch (set by the launcher)
};

// Attention over quantized + window (+ new) keys.  Decode is the case
// n_new == 0 with one query token per sequence.
struct AttnArgs {
    Tables t;
    Store k, v;
    int v_is_k;                 // latent attention: values are the K rows
    const uint16_t *rope;       // [A][rope_tokens][H][rope_dim] or null
    int rope_dim;
    int64_t rope_tokens;
    const uint16_t *q;          // [A][n_qtok][Hq][Dk]
    const uint16_t *k_new;      // [A][n_new][H][D] (chunk)
    const uint16_t *v_new;
    int n_new;                  // 0 for decode
    int n_qtok;                 // query tokens per sequence (1 for decode, n_new for chunk)
    int Hq, G, Dk, Dv;
    float scale;
    int tok_per_tile;           // query tokens per row tile
    int n_row_tiles;            // row tiles per (sequence, KV head)
    int split_keys;             // keys per split
    int n_splits;               // splits per row
    float *part;                // [rows][n_splits][Dv + 2]
    float *out;                 // [A][n_qtok][Hq][Dv]
};

// Tuned grouped-query decode (matrix cores), head_dim 64/128/256.
struct DecodeArgs {
    Tables t;
    Store k, v;
    const uint16_t *q;          // [A][Hq][D]
    float *out;                 // [A][Hq][D]
    float *part;                // [A*Hq][n_splits][D + 2]
    int Hq, G;
    int SB;                     // 64-token blocks per split
    int n_splits;               // grid.x: block splits + 1 window split
    float c;                    // softmax_scale * log2(e)
    // Latent decode over a compacted table (top-K): block slot j of sequence
    // a takes its rope rows from block rope_map[a][j] of the full layout, and
    // the window's rope rows follow block min(rope_nb[a], rope_max_blocks) of
    // it.  Null rope_map: rope rows follow the table itself.
    const int32_t *rope_map;
    const int32_t *rope_nb;
    int rope_max_blocks;
};

// Chunk attention (matrix cores), head_dim 64/128/256.
struct ChunkArgs {
    Tables t;
    Store k, v;
    const uint16_t *q_new;      // [A][n_new][Hq][D]
    const uint16_t *k_new;      // [A][n_new][H][D]
    const uint16_t *v_new;
    int n_new, Hq, G;
    float c;                    // softmax_scale * log2(e)
    int n_row_tiles;            // query-row tiles per (sequence, KV head)
    int n_splits;               // key splits (grid.x)
    int split_tiles;            // 64-key tiles per split
    float *part;                // [A*n_new*Hq][n_splits][D + 2]
    float *out;                 // [A][n_new][Hq][D]
};

// Window roll of one sequence with nb blocks and W window tokens (already
// clamped to the capacities) when n_new tokens arrive and keep recent ones
// stay bf16: k new blocks are cut and W2 tokens remain in the window.  The
// append kernels and kvq_append_counts share this one definition.
__host__ __device__ inline void append_counts(int nb, int W, int n_new, int keep, int max_blocks, int window_cap,
                                              int *k, int *W2)
{
    const int T = W + n_new;
    int kk = T > keep ? (T - keep) / 64 : 0;
    if (kk > max_blocks - nb) kk = max_blocks - nb;
    int w2 = T - 64 * kk;
    if (w2 > window_cap) w2 = window_cap;
    *k = kk;
    *W2 = w2;
}

// Append new tokens to the windows, quantizing every full 64-token block
// that leaves the kept recent window.
struct AppendArgs {
    Tables t;
    const uint64_t *k_offset, *v_offset;  // v_offset null: latent cache (K only)
    uint8_t *k_pool, *v_pool;
    uint16_t *k_window, *v_window;
    const uint16_t *k_new, *v_new;      // [A][n_new][H][D]
    uint16_t *rope;                     // [A][64*max_blocks + window_cap][H][rope_dim] or null
    const uint16_t *rope_new;           // [A][n_new][H][rope_dim]
    int rope_dim;
    int n_new, keep;
    int32_t *n_blocks_out, *n_window_out;
    int counts_in_window;   // outputs alias no count the kernels read: the window launch writes them
};

// Top-K block selection for sparse decode: scores, then compacted tables.
struct TopkArgs {
    Tables t;
    Store k, v;                 // v.offset null for a latent cache
    const uint16_t *q;          // [A][Hq][D + rope_dim]
    const uint16_t *rope;       // [A][64*max_blocks + window_cap][H][rope_dim] or null
    int rope_dim;
    int Hq, G;
    float scale;
    int top_k;
    float *scores;              // [A][max_blocks][score_stride], the block score is the max over the last axis
    int score_stride;           // 1 (generic scores) or H (per KV head, from the decode's products)
    int32_t *n_sel;             // [A]
    int32_t *sel_idx;           // [A][top_k], ascending, -1 padded
    uint8_t *sel_bits;          // [A][top_k]
    uint64_t *sel_koff, *sel_voff;   // [A][top_k]
    uint16_t *rope_sel;         // [A][64*top_k + window_cap][H][rope_dim]
    int32_t *selected;          // caller's [A][sel_stride] copy of sel_idx, or null
    int sel_stride;             // >= top_k; columns past top_k get -1
};
bool topk_supported(int max_blocks, int G, int head_dim, int rope_dim);
// g4: score with the decode kernel; copy_rope: write rope_sel for a decode
// that reads the compacted layout's rope rows (the latent kernel reads them
// in place through DecodeArgs::rope_map instead)
hipError_t launch_topk_select(const TopkArgs &p, const DecodeArgs *g4, bool copy_rope, hipStream_t s);

// Width allocation: block sensitivity (GPU) and the budgeted greedy (host).
bool sensitivity_supported(int H, int D, int Hq);
hipError_t launch_sensitivity(const uint16_t *k, const uint16_t *v, int A, int64_t seq_tokens, int n_blocks, int H,
                              int D, const uint16_t *q, int Hq, float scale, float *S, hipStream_t s);
int allocate_widths(const float *S, int64_t n, uint64_t bytes2, uint64_t bytes3, uint64_t bytes4,
                    uint64_t bytes8, uint64_t budget, uint8_t *widths);

// CacheCard image of one sequence: to_image 1 gathers, 0 scatters.
hipError_t launch_card(const Tables &t, const uint64_t *k_offset, const uint64_t *v_offset, uint8_t *k_pool,
                       uint8_t *v_pool, uint16_t *k_window, uint16_t *v_window, uint16_t *rope, int rope_dim,
                       int seq, uint8_t *image, uint64_t image_bytes, int to_image, hipStream_t s);

// Launchers (return hipError_t of the launch).
hipError_t launch_quantize(const QuantArgs &a, hipStream_t s);
hipError_t launch_append(const AppendArgs &a, hipStream_t s);          // blocks, window, counts
hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s);
hipError_t launch_attend_generic(const AttnArgs &a, hipStream_t s);
hipError_t launch_decode_gqa(const DecodeArgs &a, hipStream_t s);     // split + merge
hipError_t launch_decode_g4(const DecodeArgs &a, hipStream_t s);      // split + merge (G <= 4)
hipError_t launch_g4_scores(const DecodeArgs &a, float scale, float *scores_h, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t s);
bool decode_g4_supported(int D, int G);
void decode_g4_plan(int A, int H, int D, int max_blocks, int window_cap, int *SB, int *n_splits);
hipError_t launch_chunk(const ChunkArgs &a, hipStream_t s);          // split + merge
bool chunk_supported(int D);
int chunk_rows_per_wg(int D);
void decode_gqa_plan(int A, int H, int max_blocks, int window_cap, int *SB, int *n_splits);
bool decode_gqa_supported(int D);

// Latent (MLA) decode: one 512-dim latent KV head, optional 64-dim rope.
bool mla_supported(int D, int H, int G, int rope_dim);
void mla_plan(int A, int max_blocks, int window_cap, int *SB, int *n_splits);
hipError_t launch_mla(const DecodeArgs &a, const uint16_t *rope, int rope_dim, int64_t rope_tokens,
                      hipStream_t s);                                  // split + merge

// Generic path's split size and workspace.
void generic_plan(int max_keys, int n_new, int G, int *tok_per_tile, int *split_keys, int *n_splits);

}  // namespace kvq
