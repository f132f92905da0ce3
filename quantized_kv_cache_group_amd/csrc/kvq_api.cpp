// Host side of the kvq C ABI: argument validation (always before any HIP
// call), work planning and kernel dispatch on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

namespace {

constexpr int kMaxGrid = 65535;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_layout(const kvq_layout *L)
{
    if (!L) return KVQ_EINVAL;
    if (L->n_seqs < 1 || L->n_heads < 1 || L->max_blocks < 0 || L->window_cap < 0) return KVQ_EINVAL;
    if (L->head_dim < 64 || L->head_dim % 64) return KVQ_EINVAL;
    if (L->head_dim > 512) return KVQ_EUNSUPPORTED;
    if (L->n_seqs > kMaxGrid || L->n_heads > kMaxGrid) return KVQ_EUNSUPPORTED;
    if (!L->n_blocks || !aligned(L->n_blocks, 4)) return KVQ_EINVAL;
    if (L->max_blocks > 0 && !L->bits) return KVQ_EINVAL;
    if (L->window_cap > 0 && (!L->n_window || !aligned(L->n_window, 4))) return KVQ_EINVAL;
    // Token indices stay within int32 in the kernels.
    if ((int64_t)L->max_blocks * 64 + L->window_cap > (int64_t)1 << 30) return KVQ_EUNSUPPORTED;
    return KVQ_OK;
}

int check_store(const kvq_layout *L, const kvq_store *S)
{
    if (!S) return KVQ_EINVAL;
    if (L->max_blocks > 0) {
        if (!S->offset || !S->pool || !aligned(S->offset, 8) || !aligned(S->pool, 256)) return KVQ_EINVAL;
    }
    if (L->window_cap > 0 && (!S->window || !aligned(S->window, 16))) return KVQ_EINVAL;
    return KVQ_OK;
}

Tables tables(const kvq_layout *L)
{
    Tables t;
    t.A = L->n_seqs;
    t.H = L->n_heads;
    t.D = L->head_dim;
    t.max_blocks = L->max_blocks;
    t.window_cap = L->window_cap;
    t.n_blocks = L->n_blocks;
    t.n_window = L->window_cap > 0 ? L->n_window : nullptr;
    t.bits = L->bits;
    return t;
}

Store store(const kvq_store *S)
{
    Store s;
    s.offset = S->offset;
    s.pool = S->pool;
    s.window = S->window;
    return s;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_EHIP; }

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Plan of one attention call: the generic kernel's decomposition, and for
// decode also the tuned kernel's (the workspace covers whichever runs).
struct Plan {
    int tok_per_tile, split_keys, n_splits, n_row_tiles;
    int sb, dec_splits;         // tuned decode
    int g4_sb, g4_splits;       // tuned decode, <= 4 query heads per KV head
    int mla_sb, mla_splits;     // latent decode
    int ch_row_tiles, ch_splits, ch_split_tiles;   // tuned chunk
    bool ch_ok;
    size_t ws_bytes;
};

int plan_attention(const kvq_layout *L, int n_q_heads, int rope_dim, int n_new, Plan *pl)
{
    int st = check_layout(L);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % L->n_heads) return KVQ_EINVAL;
    if (rope_dim < 0 || n_new < 0) return KVQ_EINVAL;
    if (rope_dim != 0 && rope_dim != 64) return KVQ_EUNSUPPORTED;
    const int G = n_q_heads / L->n_heads;
    if (G > 16) return KVQ_EUNSUPPORTED;
    const int64_t max_keys = (int64_t)L->max_blocks * 64 + L->window_cap + n_new;
    if (max_keys > ((int64_t)1 << 30)) return KVQ_EUNSUPPORTED;
    generic_plan((int)max_keys, n_new, G, &pl->tok_per_tile, &pl->split_keys, &pl->n_splits);
    const int n_qtok = n_new ? n_new : 1;
    pl->n_row_tiles = (n_qtok + pl->tok_per_tile - 1) / pl->tok_per_tile;
    if ((int64_t)pl->n_row_tiles * L->n_heads > kMaxGrid) return KVQ_EUNSUPPORTED;
    const size_t rows = (size_t)L->n_seqs * n_qtok * n_q_heads;
    if (rows > 0x7fffffffu) return KVQ_EUNSUPPORTED;
    pl->ws_bytes = round256(rows * (size_t)pl->n_splits * (size_t)(L->head_dim + 2) * sizeof(float));
    if (n_new == 0) {
        decode_gqa_plan(L->n_seqs, L->n_heads, L->max_blocks, L->window_cap, &pl->sb, &pl->dec_splits);
        size_t t = round256(rows * (size_t)pl->dec_splits * (size_t)(L->head_dim + 2) * sizeof(float));
        if (t > pl->ws_bytes) pl->ws_bytes = t;
        if (decode_g4_supported(L->head_dim, G)) {
            decode_g4_plan(L->n_seqs, L->n_heads, L->head_dim, L->max_blocks, L->window_cap, &pl->g4_sb,
                           &pl->g4_splits);
            t = round256(rows * (size_t)pl->g4_splits * (size_t)(L->head_dim + 2) * sizeof(float));
            if (t > pl->ws_bytes) pl->ws_bytes = t;
        }
        if (mla_supported(L->head_dim, L->n_heads, G, rope_dim)) {
            mla_plan(L->n_seqs, L->max_blocks, L->window_cap, &pl->mla_sb, &pl->mla_splits);
            t = round256(rows * (size_t)pl->mla_splits * (size_t)(L->head_dim + 2) * sizeof(float));
            if (t > pl->ws_bytes) pl->ws_bytes = t;
        }
    }
    pl->ch_ok = false;
    if (n_new > 0 && chunk_supported(L->head_dim)) {
        const int R = chunk_rows_per_wg(L->head_dim);
        const int64_t row_tiles = ((int64_t)n_new * G + R - 1) / R;
        const int64_t tiles = (max_keys + 63) / 64;
        const int64_t units = row_tiles * L->n_heads * L->n_seqs;
        if (row_tiles * L->n_heads <= kMaxGrid) {
            int64_t ns = (256 + units - 1) / units;   // about one workgroup per CU
            if (ns > tiles) ns = tiles;
            if (ns < 1) ns = 1;
            const int64_t st = (tiles + ns - 1) / ns;
            ns = (tiles + st - 1) / st;
            pl->ch_row_tiles = (int)row_tiles;
            pl->ch_split_tiles = (int)st;
            pl->ch_splits = (int)ns;
            pl->ch_ok = true;
            const size_t t = round256(rows * (size_t)ns * (size_t)(L->head_dim + 2) * sizeof(float));
            if (t > pl->ws_bytes) pl->ws_bytes = t;
        }
    }
    return KVQ_OK;
}

// Shared by kvq_quantize (V == NULL) and kvq_quantize_kv: one launch over
// every block of one or two stores.
static int quantize_call(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *k_src,
                         const uint16_t *v_src, int64_t src_seq_tokens, void *stream)
{
    int st = check_layout(L);
    if (st) return st;
    const kvq_store *dst[2] = {K, V};
    const uint16_t *src[2] = {k_src, v_src};
    const int n = V ? 2 : 1;
    for (int x = 0; x < n; x++) {
        if (!dst[x] || !dst[x]->pool || !dst[x]->offset) {
            if (L->max_blocks > 0) return KVQ_EINVAL;
        } else if (!aligned(dst[x]->pool, 256) || !aligned(dst[x]->offset, 8)) {
            return KVQ_EINVAL;
        }
        if (!src[x] || !aligned(src[x], 16)) return KVQ_EINVAL;
    }
    if (src_seq_tokens < (int64_t)L->max_blocks * 64 || (L->n_seqs > 1 && src_seq_tokens < 1))
        return KVQ_EINVAL;
    if ((int64_t)L->n_seqs * n > kMaxGrid) return KVQ_EUNSUPPORTED;
    if (L->max_blocks == 0) return KVQ_OK;
    QuantArgs a;
    a.t = tables(L);
    for (int x = 0; x < 2; x++) {
        const int y = x < n ? x : 0;
        a.offset[x] = dst[y]->offset;
        a.pool[x] = dst[y]->pool;
        a.src[x] = src[y];
    }
    a.src_seq_tokens = src_seq_tokens;
    a.n_tensors = n;
    return hip_status(launch_quantize(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

uint64_t kvq_block_bytes(int32_t bits, int32_t n_heads, int32_t head_dim)
{
    if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return 0;
    if (n_heads < 1 || head_dim < 64 || head_dim > 512 || head_dim % 64) return 0;
    return (uint64_t)n_heads * (uint64_t)head_dim * (uint64_t)(8 * bits + 4);
}

int kvq_quantize(const kvq_layout *L, const kvq_store *dst, const uint16_t *src,
                 int64_t src_seq_tokens, void *stream)
{
    return quantize_call(L, dst, nullptr, src, nullptr, src_seq_tokens, stream);
}

int kvq_quantize_kv(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *k_src,
                    const uint16_t *v_src, int64_t src_seq_tokens, void *stream)
{
    return quantize_call(L, K, V, k_src, v_src, src_seq_tokens, stream);
}

int kvq_append_counts(int32_t n_seqs, int32_t max_blocks, int32_t window_cap, const int32_t *n_blocks,
                      const int32_t *n_window, int32_t n_new, int32_t keep_recent, int32_t *n_blocks_out,
                      int32_t *n_window_out)
{
    if (n_seqs < 1 || max_blocks < 0 || window_cap < 0 || n_new < 0 || keep_recent < 0) return KVQ_EINVAL;
    if (!n_blocks || !n_blocks_out || (window_cap > 0 && (!n_window || !n_window_out))) return KVQ_EINVAL;
    if (window_cap > 0) {
        if ((int64_t)keep_recent + 63 > window_cap) return KVQ_EINVAL;
    } else if (keep_recent != 0 || n_new % 64 != 0) {
        return KVQ_EINVAL;
    }
    if ((int64_t)window_cap + n_new > (int64_t)1 << 30) return KVQ_EUNSUPPORTED;
    for (int32_t a = 0; a < n_seqs; a++) {
        // the kernels' clamping of the device counts to the capacities
        int nb = n_blocks[a] < 0 ? 0 : (n_blocks[a] > max_blocks ? max_blocks : n_blocks[a]);
        int w = 0;
        if (window_cap > 0) w = n_window[a] < 0 ? 0 : (n_window[a] > window_cap ? window_cap : n_window[a]);
        int k = 0, w2 = 0;
        append_counts(nb, w, n_new, keep_recent, max_blocks, window_cap, &k, &w2);
        n_blocks_out[a] = nb + k;
        if (window_cap > 0) n_window_out[a] = w2;
    }
    return KVQ_OK;
}

int kvq_append(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
               const uint16_t *k_new, const uint16_t *v_new,
               uint16_t *rope, const uint16_t *rope_new, int32_t rope_dim,
               int32_t n_new, int32_t keep_recent,
               int32_t *n_blocks_out, int32_t *n_window_out, void *stream)
{
    int st = check_layout(L);
    if (st) return st;
    if ((st = check_store(L, K))) return st;
    if (V && (st = check_store(L, V))) return st;
    if (n_new < 0 || keep_recent < 0) return KVQ_EINVAL;
    if (n_new > 0) {
        if (!k_new || !aligned(k_new, 16)) return KVQ_EINVAL;
        if (V && (!v_new || !aligned(v_new, 16))) return KVQ_EINVAL;
    }
    if (rope_dim != 0 && rope_dim != 64) return KVQ_EUNSUPPORTED;
    if (rope_dim) {
        if (!rope || !aligned(rope, 16)) return KVQ_EINVAL;
        if (n_new > 0 && (!rope_new || !aligned(rope_new, 16))) return KVQ_EINVAL;
    }
    if (L->window_cap > 0) {
        if ((int64_t)keep_recent + 63 > L->window_cap) return KVQ_EINVAL;
        if (!n_window_out || !aligned(n_window_out, 4)) return KVQ_EINVAL;
    } else if (keep_recent != 0 || n_new % 64 != 0) {
        return KVQ_EINVAL;
    }
    if (!n_blocks_out || !aligned(n_blocks_out, 4)) return KVQ_EINVAL;
    // a stream of window + new tokens is indexed in int32
    if ((int64_t)L->window_cap + n_new > (int64_t)1 << 30) return KVQ_EUNSUPPORTED;
    AppendArgs a;
    a.t = tables(L);
    a.k_offset = K->offset;
    a.v_offset = V ? V->offset : nullptr;
    a.k_pool = K->pool;
    a.v_pool = V ? V->pool : nullptr;
    a.k_window = L->window_cap > 0 ? K->window : nullptr;
    a.v_window = (V && L->window_cap > 0) ? V->window : nullptr;
    a.k_new = k_new;
    a.v_new = V ? v_new : nullptr;
    a.rope = rope_dim ? rope : nullptr;
    a.rope_new = rope_dim ? rope_new : nullptr;
    a.rope_dim = rope_dim;
    a.n_new = n_new;
    a.keep = keep_recent;
    a.n_blocks_out = n_blocks_out;
    a.n_window_out = L->window_cap > 0 ? n_window_out : nullptr;
    // With outputs that overlap no count the kernels read, the window launch
    // writes the new counts and the separate counts launch is skipped.
    {
        const size_t nbytes = (size_t)L->n_seqs * sizeof(int32_t);
        auto overlap = [nbytes](const void *x, const void *y) {
            if (!x || !y) return false;
            const char *p = static_cast<const char *>(x), *q = static_cast<const char *>(y);
            return p < q + nbytes && q < p + nbytes;
        };
        const void *ins[2] = {L->n_blocks, L->window_cap > 0 ? L->n_window : nullptr};
        const void *outs[2] = {a.n_blocks_out, a.n_window_out};
        bool alias = overlap(outs[0], outs[1]);
        for (const void *o : outs)
            for (const void *i : ins) alias = alias || overlap(o, i);
        a.counts_in_window = (!alias && (L->window_cap > 0 || rope_dim)) ? 1 : 0;
    }
    return hip_status(launch_append(a, static_cast<hipStream_t>(stream)));
}

uint64_t kvq_card_bytes(int32_t n_heads, int32_t head_dim, int32_t rope_dim, int32_t has_v,
                        int32_t n_blocks, const uint8_t *bits_host, int32_t n_window)
{
    if (n_heads < 1 || head_dim < 64 || head_dim % 64 || head_dim > 512) return 0;
    if (rope_dim != 0 && rope_dim != 64) return 0;
    if (n_blocks < 0 || n_window < 0 || (n_blocks > 0 && !bits_host)) return 0;
    const int n_kv = has_v ? 2 : 1;
    uint64_t blocks = 0;
    for (int j = 0; j < n_blocks; j++) {
        const uint64_t b = kvq_block_bytes(bits_host[j], n_heads, head_dim);
        if (!b) return 0;
        blocks += b;
    }
    const uint64_t row = (uint64_t)n_heads * head_dim * 2;
    return n_kv * blocks + n_kv * (uint64_t)n_window * row +
           (uint64_t)(64 * (uint64_t)n_blocks + n_window) * n_heads * rope_dim * 2 + (uint64_t)n_blocks;
}

namespace {
static int card_call(const kvq_layout *L, const kvq_store *K, const kvq_store *V, uint16_t *rope, int32_t rope_dim,
              int32_t seq, uint8_t *image, uint64_t image_bytes, int to_image, void *stream)
{
    int st = check_layout(L);
    if (st) return st;
    if ((st = check_store(L, K))) return st;
    if (V && (st = check_store(L, V))) return st;
    if (seq < 0 || seq >= L->n_seqs) return KVQ_EINVAL;
    if (rope_dim != 0 && rope_dim != 64) return KVQ_EUNSUPPORTED;
    if (rope_dim && (!rope || !aligned(rope, 16))) return KVQ_EINVAL;
    if (!image || !aligned(image, 16)) return KVQ_EINVAL;
    return hip_status(launch_card(tables(L), K->offset, V ? V->offset : nullptr, K->pool, V ? V->pool : nullptr,
                                  L->window_cap > 0 ? K->window : nullptr,
                                  (V && L->window_cap > 0) ? V->window : nullptr, rope_dim ? rope : nullptr,
                                  rope_dim, seq, image, image_bytes, to_image, static_cast<hipStream_t>(stream)));
}
}  // namespace

int kvq_card_gather(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *rope,
                    int32_t rope_dim, int32_t seq, void *image, uint64_t image_bytes, void *stream)
{
    return card_call(L, K, V, const_cast<uint16_t *>(rope), rope_dim, seq, static_cast<uint8_t *>(image),
                     image_bytes, 1, stream);
}

int kvq_card_scatter(const kvq_layout *L, const kvq_store *K, const kvq_store *V, uint16_t *rope,
                     int32_t rope_dim, int32_t seq, const void *image, uint64_t image_bytes, void *stream)
{
    return card_call(L, K, V, rope, rope_dim, seq, const_cast<uint8_t *>(static_cast<const uint8_t *>(image)),
                     image_bytes, 0, stream);
}

int kvq_dequantize(const kvq_layout *L, const kvq_store *src, int32_t out_dtype, void *dst,
                   int64_t dst_seq_tokens, void *stream)
{
    int st = check_layout(L);
    if (st) return st;
    if ((st = check_store(L, src))) return st;
    if (out_dtype != KVQ_OUT_BF16 && out_dtype != KVQ_OUT_F32) return KVQ_EUNSUPPORTED;
    if (!dst || !aligned(dst, 16)) return KVQ_EINVAL;
    if (dst_seq_tokens < (int64_t)L->max_blocks * 64 + L->window_cap) return KVQ_EINVAL;
    DequantArgs a;
    a.t = tables(L);
    a.s = store(src);
    a.dst = dst;
    a.dst_seq_tokens = dst_seq_tokens;
    a.out_f32 = out_dtype == KVQ_OUT_F32;
    return hip_status(launch_dequantize(a, static_cast<hipStream_t>(stream)));
}

int kvq_block_sensitivity(const uint16_t *k, const uint16_t *v, int32_t n_seqs, int64_t seq_tokens,
                          int32_t n_blocks, int32_t n_heads, int32_t head_dim, const uint16_t *q,
                          int32_t n_q_heads, float softmax_scale, float *S, void *stream)
{
    if (n_seqs < 1 || n_blocks < 0 || n_heads < 1 || head_dim < 64 || head_dim % 64 || head_dim > 512)
        return KVQ_EINVAL;
    if (n_q_heads < 1 || n_q_heads % n_heads || seq_tokens < (int64_t)n_blocks * 64) return KVQ_EINVAL;
    if (n_seqs > kMaxGrid || n_blocks > 0x7fffffff) return KVQ_EUNSUPPORTED;
    if (!sensitivity_supported(n_heads, head_dim, n_q_heads)) return KVQ_EUNSUPPORTED;
    if (!k || !v || !q || !S || !aligned(k, 16) || !aligned(v, 16) || !aligned(q, 2) || !aligned(S, 4))
        return KVQ_EINVAL;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return KVQ_EINVAL;
    return hip_status(launch_sensitivity(k, v, n_seqs, seq_tokens, n_blocks, n_heads, head_dim, q, n_q_heads,
                                         softmax_scale, S, static_cast<hipStream_t>(stream)));
}

int kvq_allocate_widths(const float *S, int64_t n, int32_t n_heads, int32_t head_dim,
                        uint64_t budget_bytes, uint8_t *widths)
{
    if (n < 0 || (n > 0 && (!S || !widths))) return KVQ_EINVAL;
    const uint64_t b2 = kvq_block_bytes(2, n_heads, head_dim), b3 = kvq_block_bytes(3, n_heads, head_dim);
    const uint64_t b4 = kvq_block_bytes(4, n_heads, head_dim), b8 = kvq_block_bytes(8, n_heads, head_dim);
    if (!b2) return KVQ_EINVAL;
    for (int64_t i = 0; i < n; i++)
        if (!(S[i] >= 0.0f) || !isfinite(S[i])) return KVQ_EINVAL;
    return allocate_widths(S, n, b2, b3, b4, b8, budget_bytes, widths) ? KVQ_EINVAL : KVQ_OK;
}

int kvq_decode_workspace(const kvq_layout *L, int32_t n_q_heads, int32_t rope_dim, size_t *bytes)
{
    if (!bytes) return KVQ_EINVAL;
    Plan pl;
    int st = plan_attention(L, n_q_heads, rope_dim, 0, &pl);
    if (st) return st;
    *bytes = pl.ws_bytes;
    return KVQ_OK;
}

}  // extern "C"

namespace {
// Argument checks of a decode call other than the workspace (host only).
int check_decode(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *rope,
                 int32_t rope_dim, const uint16_t *q, int32_t n_q_heads, float softmax_scale, float *out, Plan *pl)
{
    int st = plan_attention(L, n_q_heads, rope_dim, 0, pl);
    if (st) return st;
    if ((st = check_store(L, K))) return st;
    if (V && (st = check_store(L, V))) return st;
    if ((rope_dim > 0) != (rope != nullptr)) return KVQ_EINVAL;
    if (rope && !aligned(rope, 16)) return KVQ_EINVAL;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return KVQ_EINVAL;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return KVQ_EINVAL;
    return KVQ_OK;
}

// Rope rows of a compacted (top-K) latent layout read in place from the full
// layout: slot j of sequence a takes block map[a][j]; the window follows
// block min(nb[a], max_blocks); tokens is the full layout's rows per sequence.
struct RopeMap {
    const int32_t *map;
    const int32_t *nb;
    int max_blocks;
    int64_t tokens;
};

int attend_decode_impl(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *rope,
                       int32_t rope_dim, const uint16_t *q, int32_t n_q_heads, float softmax_scale, float *out,
                       void *workspace, const Plan &pl, void *stream, const RopeMap *rm = nullptr);
}  // namespace

extern "C" {

int kvq_attend_decode(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                      const uint16_t *rope, int32_t rope_dim, const uint16_t *q,
                      int32_t n_q_heads, float softmax_scale, float *out,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    Plan pl;
    int st = check_decode(L, K, V, rope, rope_dim, q, n_q_heads, softmax_scale, out, &pl);
    if (st) return st;
    if (workspace_bytes < pl.ws_bytes) return KVQ_ENOSPC;
    if (!workspace || !aligned(workspace, 256)) return KVQ_EINVAL;
    return attend_decode_impl(L, K, V, rope, rope_dim, q, n_q_heads, softmax_scale, out, workspace, pl, stream);
}

}  // extern "C"

namespace {
// The decode's launches once every argument has been checked.
int attend_decode_impl(const kvq_layout *L, const kvq_store *K, const kvq_store *V, const uint16_t *rope,
                       int32_t rope_dim, const uint16_t *q, int32_t n_q_heads, float softmax_scale, float *out,
                       void *workspace, const Plan &pl, void *stream, const RopeMap *rm)
{
    float *part = static_cast<float *>(workspace);

    if (V && rope_dim == 0 && decode_gqa_supported(L->head_dim)) {
        DecodeArgs d{};
        d.t = tables(L);
        d.k = store(K);
        d.v = store(V);
        d.q = q;
        d.out = out;
        d.part = part;
        d.Hq = n_q_heads;
        d.G = n_q_heads / L->n_heads;
        d.SB = pl.sb;
        d.n_splits = pl.dec_splits;
        d.c = softmax_scale * 1.4426950408889634f;
        hipStream_t hs = static_cast<hipStream_t>(stream);
        if (decode_g4_supported(L->head_dim, d.G)) {
            d.SB = pl.g4_sb;
            d.n_splits = pl.g4_splits;
            return hip_status(launch_decode_g4(d, hs));
        }
        return hip_status(launch_decode_gqa(d, hs));
    }

    if (!V && mla_supported(L->head_dim, L->n_heads, n_q_heads / L->n_heads, rope_dim)) {
        DecodeArgs d{};
        d.t = tables(L);
        d.k = store(K);
        d.v = store(K);
        d.q = q;
        d.out = out;
        d.part = part;
        d.Hq = n_q_heads;
        d.G = n_q_heads;
        d.SB = pl.mla_sb;
        d.n_splits = pl.mla_splits;
        d.c = softmax_scale * 1.4426950408889634f;
        int64_t rope_tokens = (int64_t)L->max_blocks * 64 + L->window_cap;
        if (rm && rope_dim) {
            d.rope_map = rm->map;
            d.rope_nb = rm->nb;
            d.rope_max_blocks = rm->max_blocks;
            rope_tokens = rm->tokens;
        }
        return hip_status(launch_mla(d, rope, rope_dim, rope_tokens, static_cast<hipStream_t>(stream)));
    }

    AttnArgs a{};
    a.t = tables(L);
    a.k = store(K);
    a.v = V ? store(V) : store(K);
    a.v_is_k = V == nullptr;
    a.rope = rope;
    a.rope_dim = rope_dim;
    a.rope_tokens = (int64_t)L->max_blocks * 64 + L->window_cap;
    a.q = q;
    a.n_new = 0;
    a.n_qtok = 1;
    a.Hq = n_q_heads;
    a.G = n_q_heads / L->n_heads;
    a.Dk = L->head_dim + rope_dim;
    a.Dv = L->head_dim;
    a.scale = softmax_scale;
    a.tok_per_tile = pl.tok_per_tile;
    a.n_row_tiles = pl.n_row_tiles;
    a.split_keys = pl.split_keys;
    a.n_splits = pl.n_splits;
    a.part = part;
    a.out = out;
    return hip_status(launch_attend_generic(a, static_cast<hipStream_t>(stream)));
}

// Scratch of kvq_attend_decode_static: the split partials live in this
// file-scope device array (one copy per GPU, held until the process ends).
// Host code never uses its name as an address: the address of each
// device's copy comes from hipGetSymbolAddress, taken once per device.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Address of the current device's scratch, or null on a HIP error.
void *static_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int kvq_attend_decode_static(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                             const uint16_t *rope, int32_t rope_dim, const uint16_t *q,
                             int32_t n_q_heads, float softmax_scale, float *out, void *stream)
{
    Plan pl;
    int st = check_decode(L, K, V, rope, rope_dim, q, n_q_heads, softmax_scale, out, &pl);
    if (st) return st;
    if (pl.ws_bytes > kStaticScratchBytes) return KVQ_ENOSPC;
    void *ws = static_scratch();
    if (!ws) return KVQ_EHIP;
    return attend_decode_impl(L, K, V, rope, rope_dim, q, n_q_heads, softmax_scale, out, ws, pl, stream);
}

namespace {
// Workspace of a top-K call: the decode's own workspace first, then the
// selection tables.
struct TopkWs {
    size_t scores, n_sel, sel_idx, sel_bits, sel_koff, sel_voff, rope_sel, dec, total;
    kvq_layout L2;                            // pointers filled in at call time
    size_t dec_bytes;
};

static int topk_plan(const kvq_layout *L, int32_t n_q_heads, int32_t rope_dim, int32_t top_k, TopkWs *w)
{
    int st = check_layout(L);
    if (st) return st;
    if (top_k < 1 || n_q_heads < 1 || n_q_heads % L->n_heads) return KVQ_EINVAL;
    if (rope_dim != 0 && rope_dim != 64) return KVQ_EUNSUPPORTED;
    if (!topk_supported(L->max_blocks, n_q_heads / L->n_heads, L->head_dim, rope_dim)) return KVQ_EUNSUPPORTED;
    // kept blocks per sequence (0 for a window-only layout); arrays hold at least one entry
    const int k = top_k < L->max_blocks ? top_k : L->max_blocks;
    const size_t ka = (size_t)(k > 0 ? k : 1);
    const size_t A = (size_t)L->n_seqs;
    w->L2 = *L;
    w->L2.max_blocks = k;
    size_t dec = 0;
    if ((st = kvq_decode_workspace(&w->L2, n_q_heads, rope_dim, &dec))) return st;
    w->dec = 0;
    w->dec_bytes = dec;
    size_t pos = round256(dec);
    w->scores = pos;   pos += round256(A * (size_t)(L->max_blocks > 0 ? L->max_blocks : 1) * L->n_heads * 4);
    w->n_sel = pos;    pos += round256(A * 4);
    w->sel_idx = pos;  pos += round256(A * ka * 4);
    w->sel_bits = pos; pos += round256(A * ka);
    w->sel_koff = pos; pos += round256(A * ka * 8);
    w->sel_voff = pos; pos += round256(A * ka * 8);
    w->rope_sel = pos;
    pos += round256(A * ((size_t)64 * ka + L->window_cap) * L->n_heads * rope_dim * 2);
    w->total = pos;
    return KVQ_OK;
}
}  // namespace

int kvq_topk_workspace(const kvq_layout *L, int32_t n_q_heads, int32_t rope_dim, int32_t top_k, size_t *bytes)
{
    if (!bytes) return KVQ_EINVAL;
    TopkWs w;
    int st = topk_plan(L, n_q_heads, rope_dim, top_k, &w);
    if (st) return st;
    *bytes = w.total;
    return KVQ_OK;
}

int kvq_attend_decode_topk(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                           const uint16_t *rope, int32_t rope_dim, const uint16_t *q,
                           int32_t n_q_heads, float softmax_scale, int32_t top_k, float *out,
                           int32_t *selected, void *workspace, size_t workspace_bytes, void *stream)
{
    TopkWs w;
    int st = topk_plan(L, n_q_heads, rope_dim, top_k, &w);
    if (st) return st;
    if ((st = check_store(L, K))) return st;
    if (V && (st = check_store(L, V))) return st;
    if ((rope_dim > 0) != (rope != nullptr)) return KVQ_EINVAL;
    if (rope && !aligned(rope, 16)) return KVQ_EINVAL;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return KVQ_EINVAL;
    if (selected && !aligned(selected, 4)) return KVQ_EINVAL;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return KVQ_EINVAL;
    if (workspace_bytes < w.total) return KVQ_ENOSPC;
    if (!workspace || !aligned(workspace, 256)) return KVQ_EINVAL;
    const int k = w.L2.max_blocks;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    TopkArgs p{};
    p.t = tables(L);
    p.k = store(K);
    if (V) p.v = store(V);
    p.q = q;
    p.rope = rope;
    p.rope_dim = rope_dim;
    p.Hq = n_q_heads;
    p.G = n_q_heads / L->n_heads;
    p.scale = softmax_scale;
    p.top_k = k;
    p.scores = reinterpret_cast<float *>(ws + w.scores);
    p.n_sel = reinterpret_cast<int32_t *>(ws + w.n_sel);
    p.sel_idx = reinterpret_cast<int32_t *>(ws + w.sel_idx);
    p.sel_bits = ws + w.sel_bits;
    p.sel_koff = reinterpret_cast<uint64_t *>(ws + w.sel_koff);
    p.sel_voff = V ? reinterpret_cast<uint64_t *>(ws + w.sel_voff) : nullptr;
    p.rope_sel = rope_dim ? reinterpret_cast<uint16_t *>(ws + w.rope_sel) : nullptr;
    p.selected = selected;
    p.sel_stride = top_k;
    p.score_stride = 1;
    // The decode over the compacted tables, validated before anything runs.
    kvq_layout L2 = w.L2;
    L2.n_blocks = p.n_sel;
    L2.bits = p.sel_bits;
    kvq_store K2 = *K;
    K2.offset = p.sel_koff;
    kvq_store V2{};
    if (V) {
        V2 = *V;
        V2.offset = p.sel_voff;
    }
    if ((st = check_layout(&L2)) || (st = check_store(&L2, &K2)) || (V && (st = check_store(&L2, &V2))))
        return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    DecodeArgs g4{};
    const bool use_g4 = rope_dim == 0 && decode_g4_supported(L->head_dim, p.G);
    if (use_g4) {
        g4.t = tables(L);
        g4.k = store(K);
        g4.q = q;
        g4.Hq = n_q_heads;
        g4.G = p.G;
        int splits = 0;
        decode_g4_plan(L->n_seqs, L->n_heads, L->head_dim, L->max_blocks, 0, &g4.SB, &splits);
        // scores need no merge, so shorter runs of blocks per wave than the
        // decode's (measured: 4 against the decode's 16 on 10 x 32 768 tokens,
        // 2 against 1 on 10 x 4 096)
        if (g4.SB > 2) g4.SB = g4.SB / 4 > 2 ? g4.SB / 4 : 2;
        p.score_stride = L->n_heads;
    }
    // The latent kernel reads the kept blocks' rope rows in place (through
    // the selection's block indices); other decodes read a compacted copy.
    // Everything the decode checks is checked before the first launch.
    const bool mla_route = !V && rope_dim > 0 && mla_supported(L->head_dim, L->n_heads, p.G, rope_dim);
    Plan mpl;
    if (mla_route) {
        if ((st = check_decode(&L2, &K2, nullptr, rope, rope_dim, q, n_q_heads, softmax_scale, out, &mpl)))
            return st;
        if (w.dec_bytes < mpl.ws_bytes) return KVQ_ENOSPC;
    }
    if (launch_topk_select(p, use_g4 ? &g4 : nullptr, !mla_route, hs) != hipSuccess) return KVQ_EHIP;
    if (mla_route) {
        const RopeMap rm{p.sel_idx, L->n_blocks, L->max_blocks, (int64_t)L->max_blocks * 64 + L->window_cap};
        return attend_decode_impl(&L2, &K2, nullptr, rope, rope_dim, q, n_q_heads, softmax_scale, out, ws + w.dec,
                                  mpl, stream, &rm);
    }
    return kvq_attend_decode(&L2, &K2, V ? &V2 : nullptr, p.rope_sel, rope_dim, q, n_q_heads, softmax_scale, out,
                             ws + w.dec, w.dec_bytes, stream);
}

int kvq_chunk_workspace(const kvq_layout *L, int32_t n_q_heads, int32_t n_new, size_t *bytes)
{
    if (!bytes) return KVQ_EINVAL;
    if (n_new < 0) return KVQ_EINVAL;
    Plan pl;
    int st = plan_attention(L, n_q_heads, 0, n_new, &pl);
    if (st) return st;
    *bytes = n_new ? pl.ws_bytes : 0;
    return KVQ_OK;
}

int kvq_attend_chunk(const kvq_layout *L, const kvq_store *K, const kvq_store *V,
                     const uint16_t *q_new, const uint16_t *k_new, const uint16_t *v_new,
                     int32_t n_new, int32_t n_q_heads, float softmax_scale, float *out,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    if (n_new < 0) return KVQ_EINVAL;
    Plan pl;
    int st = plan_attention(L, n_q_heads, 0, n_new, &pl);
    if (st) return st;
    if ((st = check_store(L, K))) return st;
    if (!V) return KVQ_EUNSUPPORTED;
    if ((st = check_store(L, V))) return st;
    if (!q_new || !k_new || !v_new || !out) return KVQ_EINVAL;
    if (!aligned(q_new, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16))
        return KVQ_EINVAL;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return KVQ_EINVAL;
    if (n_new == 0) return KVQ_OK;
    if (workspace_bytes < pl.ws_bytes) return KVQ_ENOSPC;
    if (!workspace || !aligned(workspace, 256)) return KVQ_EINVAL;

    if (pl.ch_ok) {
        ChunkArgs c{};
        c.t = tables(L);
        c.k = store(K);
        c.v = store(V);
        c.q_new = q_new;
        c.k_new = k_new;
        c.v_new = v_new;
        c.n_new = n_new;
        c.Hq = n_q_heads;
        c.G = n_q_heads / L->n_heads;
        c.c = softmax_scale * 1.4426950408889634f;
        c.n_row_tiles = pl.ch_row_tiles;
        c.n_splits = pl.ch_splits;
        c.split_tiles = pl.ch_split_tiles;
        c.part = static_cast<float *>(workspace);
        c.out = out;
        return hip_status(launch_chunk(c, static_cast<hipStream_t>(stream)));
    }

    AttnArgs a{};
    a.t = tables(L);
    a.k = store(K);
    a.v = store(V);
    a.v_is_k = 0;
    a.rope = nullptr;
    a.rope_dim = 0;
    a.rope_tokens = 0;
    a.q = q_new;
    a.k_new = k_new;
    a.v_new = v_new;
    a.n_new = n_new;
    a.n_qtok = n_new;
    a.Hq = n_q_heads;
    a.G = n_q_heads / L->n_heads;
    a.Dk = L->head_dim;
    a.Dv = L->head_dim;
    a.scale = softmax_scale;
    a.tok_per_tile = pl.tok_per_tile;
    a.n_row_tiles = pl.n_row_tiles;
    a.split_keys = pl.split_keys;
    a.n_splits = pl.n_splits;
    a.part = static_cast<float *>(workspace);
    a.out = out;
    return hip_status(launch_attend_generic(a, static_cast<hipStream_t>(stream)));
}

const char *kvq_strerror(int status)
{
    switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument (null pointer, bad size or misalignment)";
    case KVQ_ENOSPC: return "workspace too small";
    case KVQ_EUNSUPPORTED: return "unsupported shape or option";
    case KVQ_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

}  // extern "C"
