// Top-K block selection for sparse decode over the quantized cache.
//
// What it computes (Reasoning-Aware Error-Bounded KV-Cache Compression and
// Sparse Attention for Long-Context LLMs, section 2C: the active set is the
// top-K entries by a query-aware score built on the instantaneous query-key
// compatibility; section 2B: the output error is bounded by twice the
// largest value norm times the attention mass left out).  Here an entry is a
// 64-token quantized block of a sequence, its score the largest scaled
// query-key product over its tokens and over all of the sequence's query
// heads, computed from the restored keys (plus raw rope dims).  The top-K
// blocks (ties to the lower index) are compacted, in block order, into
// tables that the ordinary decode kernels then read; the bf16 window is
// always active.
#include "kvq_internal.h"
#include "unpack.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int MAXQ = 16 * (512 + 64);                 // G <= 16 rows of D + rope <= 576

// Scores on matrix cores: one wave per (block j, sequence a) computes
// S^T[key][head] for the block's 64 keys (four 16-key tiles) and the query
// heads of every KV head, on exact codes: per 64-dim group g,
// T_g = sum_{d in g} q_d c_d on v_mfma_f32_16x16x32_f16 (every 32-dim K-step
// lies in one group), then sum_g (s_g T_g + b_g Q_g) in fp32 with the key's
// (scale, bias) and Q_g the group's sum of the fp16 query; the rope dims
// (bf16, exact in fp16) add two K-steps.  The block's score is the largest
// over its keys and the heads, times the softmax scale.
template <int B, int NG, int R>
__device__ __forceinline__ float block_tiles(const TopkArgs &p, const uint8_t *blk, int a, int j, int g,
                                             const h8 *qop, const float *qsum)
{
    constexpr int CODE_ROW = 8 * NG * B, ND = GRow<B>::NDW;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    const int H = p.t.H;
    const size_t rope_tokens = (size_t)64 * p.t.max_blocks + p.t.window_cap;
    const uint32_t *meta = reinterpret_cast<const uint32_t *>(blk + (size_t)H * 64 * CODE_ROW);
    float best = -INFINITY;
    // two 16-key tiles' code rows and rope rows are loaded before their
    // products (two memory round trips per block instead of four)
#pragma unroll 1
    for (int hf = 0; hf < 2; hf++) {
        uint32_t w[2][NG][ND];
        uint4 rq[2][R > 0 ? R / 32 : 1];
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
            const int tau = 2 * hf + tt;
            const int key = 16 * tau + m;
            const uint8_t *row = blk + ((size_t)g * 64 + key) * CODE_ROW;
#pragma unroll
            for (int gg = 0; gg < NG; gg++) GRow<B>::load(w[tt][gg], row + 8 * B * gg, q);
            if constexpr (R > 0) {
                const uint16_t *rr = p.rope + (((size_t)a * rope_tokens + (size_t)64 * j + key) * H + g) * R;
#pragma unroll
                for (int r = 0; r < R / 32; r++) rq[tt][r] = *reinterpret_cast<const uint4 *>(rr + 32 * r + 8 * q);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
            const int tau = 2 * hf + tt;
            f4 T[NG], Tr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int gg = 0; gg < NG; gg++) {
                f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 2; u++)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand(GRow<B>::chunk(w[tt][gg], q, u)),
                                                                 qop[2 * gg + u], acc, 0, 0, 0);
                T[gg] = acc;
            }
            if constexpr (R > 0) {
#pragma unroll
                for (int r = 0; r < R / 32; r++)
                    Tr = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand(bf16_pairs(rq[tt][r])), qop[2 * NG + r], Tr, 0,
                                                                0, 0);
            }
            // lane (head m, q) holds keys 16 tau + 4q + i, i = 0..3; their NG
            // metadata words are contiguous (16-byte loads when NG % 4 == 0)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t *km = meta + ((size_t)g * 64 + 16 * tau + 4 * q + i) * NG;
                uint32_t kmv[NG];
                if constexpr (NG % 4 == 0) {
#pragma unroll
                    for (int c = 0; c < NG / 4; c++) {
                        const uint4 v = reinterpret_cast<const uint4 *>(km)[c];
                        kmv[4 * c] = v.x; kmv[4 * c + 1] = v.y; kmv[4 * c + 2] = v.z; kmv[4 * c + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int gg = 0; gg < NG; gg++) kmv[gg] = km[gg];
                }
                float sc = Tr[i];
#pragma unroll
                for (int gg = 0; gg < NG; gg++) {
                    const h2 sb = as_h2(kmv[gg]);
                    sc = __builtin_fmaf((float)sb[0], T[gg][i], __builtin_fmaf((float)sb[1], qsum[gg], sc));
                }
                best = fmaxf(best, sc);
            }
        }
    }
    return best;
}

template <int NG, int R>
__global__ __launch_bounds__(64) void block_scores_mfma(TopkArgs p)
{
    constexpr int D = 64 * NG, KS = 2 * NG + R / 32;
    const int j = blockIdx.x, a = blockIdx.y;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    const int H = p.t.H, G = p.G;
    int nb = p.t.n_blocks[a];
    nb = nb < 0 ? 0 : (nb > p.t.max_blocks ? p.t.max_blocks : nb);
    if (j >= nb) {
        if (lane == 0) p.scores[(size_t)a * p.t.max_blocks + j] = -INFINITY;
        return;
    }
    const size_t e = (size_t)a * p.t.max_blocks + j;
    const int B = p.t.bits[e];
    const uint8_t *blk = p.k.pool + p.k.offset[e];
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    float best = -INFINITY;
    for (int g = 0; g < H; g++) {
        // the G query rows of KV head g as B operands (heads past G are zero)
        const bool hv = m < G;
        const uint16_t *qrow = p.q + ((size_t)a * p.Hq + (size_t)g * G + (hv ? m : 0)) * (D + R);
        h8 qop[KS];
        float qsum[NG];
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
            float qs = 0.0f;
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const int c = 8 * gg + 2 * q + u;
                h8 o = operand(bf16_pairs(*reinterpret_cast<const uint4 *>(qrow + 8 * c)));
                if (!hv) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
                qop[2 * gg + u] = o;
#pragma unroll
                for (int i = 0; i < 4; i++) qs = __builtin_amdgcn_fdot2(h2{o[2 * i], o[2 * i + 1]}, ones, qs, false);
            }
            qs += __shfl_xor(qs, 16);
            qs += __shfl_xor(qs, 32);
            qsum[gg] = qs;
        }
#pragma unroll
        for (int r = 0; r < R / 32; r++) {
            h8 o = operand(bf16_pairs(*reinterpret_cast<const uint4 *>(qrow + D + 32 * r + 8 * q)));
            if (!hv) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
            qop[2 * NG + r] = o;
        }
        float t;
        switch (B) {
        case 2: t = block_tiles<2, NG, R>(p, blk, a, j, g, qop, qsum); break;
        case 3: t = block_tiles<3, NG, R>(p, blk, a, j, g, qop, qsum); break;
        case 4: t = block_tiles<4, NG, R>(p, blk, a, j, g, qop, qsum); break;
        default: t = block_tiles<8, NG, R>(p, blk, a, j, g, qop, qsum); break;
        }
        if (hv) best = fmaxf(best, t);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = fmaxf(best, __shfl_xor(best, o));
    if (lane == 0) p.scores[e] = p.scale * best;
}

// Selection: one workgroup per sequence.  Block i is kept when fewer than
// Kk = min(top_k, nb) blocks rank above it (higher score, or equal score and
// lower index); kept blocks are compacted in block order.  The Kk-th largest
// score comes from a radix select over order-preserving 32-bit keys (four
// 8-bit digits, an LDS histogram per digit), so the cost is linear in nb;
// blocks with exactly that score are taken in index order.
constexpr int MAXB = 16384;

// Key of a finite score: unsigned order equals float order (-0 is made +0
// first, so equal scores give equal keys).
__device__ __forceinline__ uint32_t score_key(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum of one value per thread over the 256 threads, in
// thread order; *total gets the sum.  wsum: 4 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int *wsum, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const int x = wsum[w];
        off += w < wave ? x : 0;
        tot += x;
    }
    *total = tot;
    __syncthreads();
    return off + incl - v;
}

__global__ __launch_bounds__(256) void select_blocks(TopkArgs p)
{
    __shared__ uint32_t key[MAXB];
    __shared__ int hist[256];
    __shared__ int wsum[4];
    __shared__ int sel[2];                              // digit, candidates above it
    const int a = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    int nb = p.t.n_blocks[a];
    nb = nb < 0 ? 0 : (nb > p.t.max_blocks ? p.t.max_blocks : nb);
    const int Kk = nb < p.top_k ? nb : p.top_k;
    // Each thread owns a contiguous run of blocks [b0, b1); the table
    // entries of its first PF blocks are loaded now, beside the scores, so
    // the compaction at the end waits on no load.
    constexpr int PF = 4;
    const int per = (nb + 255) / 256, b0 = min(tid * per, nb), b1 = min(b0 + per, nb);
    const size_t in = (size_t)a * p.t.max_blocks, out = (size_t)a * p.top_k;
    uint8_t pbits[PF];
    uint64_t pko[PF], pvo[PF];
#pragma unroll
    for (int k = 0; k < PF; k++) {
        pbits[k] = 0;
        pko[k] = pvo[k] = 0;
        if (nb > 0) {                                   // window-only tables may be empty (or null)
            const int i = min(b0 + k, nb - 1);
            pbits[k] = p.t.bits[in + i];
            pko[k] = p.k.offset[in + i];
            pvo[k] = p.sel_voff ? p.v.offset[in + i] : 0;
        }
    }
    // a block's score: the max over its score_stride entries (the first 16
    // loads are independent of each other)
    const int S = p.score_stride;
    const float *sp = p.scores + (size_t)a * p.t.max_blocks * S;
    for (int i = tid; i < nb; i += 256) {
        const float *r = sp + (size_t)i * S;
        float m = r[0];
#pragma unroll
        for (int e = 1; e < 16; e++)
            if (e < S) m = fmaxf(m, r[e]);
        for (int e = 16; e < S; e++) m = fmaxf(m, r[e]);
        key[i] = score_key(m);
    }
    // Radix select, most significant digit first: T = the Kk-th largest key;
    // `need` ends as the number of keys equal to T that are kept.
    uint32_t prefix = 0, mask = 0;
    int need = Kk;
    if (Kk > 0 && nb <= 256) {
        // One block per thread: its rank (larger keys, then equal keys at lower
        // indices) by counting over the LDS keys; the block of rank Kk - 1
        // gives T and the number of keys above it.
        __syncthreads();
        if (tid < nb) {
            const uint32_t u = key[tid];
            int gt = 0, eqb = 0;
            for (int j = 0; j < nb; j++) {
                const uint32_t w = key[j];
                gt += w > u;
                eqb += (w == u) & (j < tid);
            }
            if (gt + eqb == Kk - 1) {
                sel[0] = (int)u;
                sel[1] = gt;
            }
        }
        __syncthreads();
        prefix = (uint32_t)sel[0];
        need = Kk - sel[1];
    } else if (Kk > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            hist[tid] = 0;
            __syncthreads();
            for (int i = tid; i < nb; i += 256) {
                const uint32_t u = key[i];
                if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
            }
            __syncthreads();
            if (tid < 64) {
                // lane l holds digits 255-4l .. 252-4l, largest first
                int c[4], sum = 0;
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    c[k] = hist[255 - 4 * lane - k];
                    sum += c[k];
                }
                int above = wave_incl_scan(sum) - sum;      // candidates with a larger digit
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    if (above < need && above + c[k] >= need) {
                        sel[0] = 255 - 4 * lane - k;
                        sel[1] = above;
                    }
                    above += c[k];
                }
            }
            __syncthreads();
            need -= sel[1];
            prefix |= (uint32_t)sel[0] << shift;
            mask |= 255u << shift;
        }
    }
    __syncthreads();
    const uint32_t T = prefix;
    // ties (key == T) ranked in index order, then the kept flags, then their
    // compaction, over each thread's run
    int ties = 0;
    for (int i = b0; i < b1; i++) ties += (Kk > 0 && key[i] == T);
    int tot;
    int tie_rank = block_exclusive_scan(ties, wsum, &tot);
    int kept = 0;
    for (int i = b0; i < b1; i++) {
        const uint32_t u = key[i];
        bool k = false;
        if (Kk > 0) {
            if (u > T) k = true;
            else if (u == T) k = tie_rank++ < need;
        }
        kept += k;
    }
    // second walk with the kept positions
    int pos = block_exclusive_scan(kept, wsum, &tot);
    tie_rank -= ties;                                   // back to this run's first tie rank
    int32_t *user = p.selected ? p.selected + (size_t)a * p.sel_stride : nullptr;
    for (int i = b0; i < b1; i++) {
        const uint32_t u = key[i];
        bool k = false;
        if (Kk > 0) {
            if (u > T) k = true;
            else if (u == T) k = tie_rank++ < need;
        }
        if (!k) continue;
        const int r = i - b0;
        uint8_t bw;
        uint64_t ko, vo;
        if (r < PF) {
            bw = r == 0 ? pbits[0] : r == 1 ? pbits[1] : r == 2 ? pbits[2] : pbits[3];
            ko = r == 0 ? pko[0] : r == 1 ? pko[1] : r == 2 ? pko[2] : pko[3];
            vo = r == 0 ? pvo[0] : r == 1 ? pvo[1] : r == 2 ? pvo[2] : pvo[3];
        } else {
            bw = p.t.bits[in + i];
            ko = p.k.offset[in + i];
            vo = p.sel_voff ? p.v.offset[in + i] : 0;
        }
        p.sel_idx[out + pos] = i;
        if (user) user[pos] = i;
        p.sel_bits[out + pos] = bw;
        p.sel_koff[out + pos] = ko;
        if (p.sel_voff) p.sel_voff[out + pos] = vo;
        pos++;
    }
    for (int q = Kk + tid; q < p.top_k; q += 256) {
        p.sel_idx[out + q] = -1;
        p.sel_bits[out + q] = 4;
        p.sel_koff[out + q] = 0;
        if (p.sel_voff) p.sel_voff[out + q] = 0;
    }
    if (user)
        for (int q = Kk + tid; q < p.sel_stride; q += 256) user[q] = -1;
    if (tid == 0) p.n_sel[a] = Kk;
}

// Rope rows of the compacted layout: block slot q takes the rows of block
// sel_idx[q]; the window rows follow the last kept block.
__global__ __launch_bounds__(256) void compact_rope(TopkArgs p)
{
    const int x = blockIdx.x, a = blockIdx.y;
    const int H = p.t.H, R = p.rope_dim;
    int nb = p.t.n_blocks[a];
    nb = nb < 0 ? 0 : (nb > p.t.max_blocks ? p.t.max_blocks : nb);
    int W = p.t.n_window ? p.t.n_window[a] : 0;
    W = W < 0 ? 0 : (W > p.t.window_cap ? p.t.window_cap : W);
    const int Kk = nb < p.top_k ? nb : p.top_k;
    const size_t src_tokens = (size_t)64 * p.t.max_blocks + p.t.window_cap;
    const size_t dst_tokens = (size_t)64 * p.top_k + p.t.window_cap;
    const uint16_t *src = p.rope + (size_t)a * src_tokens * H * R;
    uint16_t *dst = p.rope_sel + (size_t)a * dst_tokens * H * R;
    int s0, d0, n;                                    // rows
    if (x < p.top_k) {
        if (x >= Kk) return;
        s0 = 64 * p.sel_idx[(size_t)a * p.top_k + x];
        d0 = 64 * x;
        n = 64;
    } else {
        const int c = x - p.top_k;                    // 64-row chunks of the window
        if (64 * c >= W) return;
        s0 = 64 * nb + 64 * c;
        d0 = 64 * Kk + 64 * c;
        n = min(64, W - 64 * c);
    }
    const int pieces = n * H * R / 8;                 // 16-byte pieces
    const uint4 *sp = reinterpret_cast<const uint4 *>(src + (size_t)s0 * H * R);
    uint4 *dp = reinterpret_cast<uint4 *>(dst + (size_t)d0 * H * R);
    for (int i = threadIdx.x; i < pieces; i += 256) dp[i] = sp[i];
}

}  // namespace

bool topk_supported(int max_blocks, int G, int head_dim, int rope_dim)
{
    return max_blocks <= MAXB && G * (head_dim + rope_dim) <= MAXQ;
}

hipError_t launch_topk_select(const TopkArgs &p, const DecodeArgs *g4, bool copy_rope, hipStream_t s)
{
    if (p.t.max_blocks > 0) {
        hipError_t e;
        if (g4) {                                     // per KV head, from the decode's own products
            e = launch_g4_scores(*g4, p.scale, p.scores, s);
        } else {
            const dim3 grid(p.t.max_blocks, p.t.A);
            const int ng = p.t.D / 64;
            if (p.rope_dim == 0) {
                switch (ng) {
                case 1: block_scores_mfma<1, 0><<<grid, 64, 0, s>>>(p); break;
                case 2: block_scores_mfma<2, 0><<<grid, 64, 0, s>>>(p); break;
                case 3: block_scores_mfma<3, 0><<<grid, 64, 0, s>>>(p); break;
                case 4: block_scores_mfma<4, 0><<<grid, 64, 0, s>>>(p); break;
                case 5: block_scores_mfma<5, 0><<<grid, 64, 0, s>>>(p); break;
                case 6: block_scores_mfma<6, 0><<<grid, 64, 0, s>>>(p); break;
                case 7: block_scores_mfma<7, 0><<<grid, 64, 0, s>>>(p); break;
                default: block_scores_mfma<8, 0><<<grid, 64, 0, s>>>(p); break;
                }
            } else {
                switch (ng) {
                case 1: block_scores_mfma<1, 64><<<grid, 64, 0, s>>>(p); break;
                case 2: block_scores_mfma<2, 64><<<grid, 64, 0, s>>>(p); break;
                case 3: block_scores_mfma<3, 64><<<grid, 64, 0, s>>>(p); break;
                case 4: block_scores_mfma<4, 64><<<grid, 64, 0, s>>>(p); break;
                case 5: block_scores_mfma<5, 64><<<grid, 64, 0, s>>>(p); break;
                case 6: block_scores_mfma<6, 64><<<grid, 64, 0, s>>>(p); break;
                case 7: block_scores_mfma<7, 64><<<grid, 64, 0, s>>>(p); break;
                default: block_scores_mfma<8, 64><<<grid, 64, 0, s>>>(p); break;
                }
            }
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    select_blocks<<<p.t.A, 256, 0, s>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.rope_dim || !copy_rope) return e;
    const int wchunks = (p.t.window_cap + 63) / 64;
    compact_rope<<<dim3(p.top_k + wchunks, p.t.A), 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace kvq
