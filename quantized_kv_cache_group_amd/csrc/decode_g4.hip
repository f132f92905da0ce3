// Batched split-K decode for grouped-query attention with at most 4 query
// heads per KV head (gfx950, 4x4x4 matrix-core blocks).
//
// What it computes (Agent Memory Below the Prompt, arXiv 2603.04428,
// Abstract: batched inference over several agents' quantized caches restored
// directly into the attention layer; QKVShare, Metodologia: the fused
// quantized attention kernel): for sequence a and query head h, softmax
// attention of q[a][h] over the 64*n_blocks[a] quantized tokens and the
// n_window[a] bf16 tokens of KV head h / G.
//
// Why 4x4x4 blocks: with G <= 4 query heads per KV head, a 16x16 tile would
// leave 12 of its 16 head rows empty, and every score would cost 4x the
// vector work.  v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4x4x4 products,
// so a wave of 64 lanes maps lane l to token l of a 64-token block:
//   Q.K^T  block b = tokens 4b..4b+3; A = K rows (lane = token, 4 dims per
//          instruction), B = the G query rows (read from LDS), so lane (b, j)
//          ends with the scores of tokens 4b..4b+3 for head j;
//   P.V    for each 4-token slice s, A = P[heads][tokens 4s..4s+3], which is
//          exactly what the lanes of block s hold after the softmax, broadcast
//          to all 16 blocks by the instruction's CBSZ/ABID fields; B = V rows
//          of those 4 tokens for 4 output dims per block: each lane writes its
//          dequantized V row to LDS and ds_read_b64_tr_b16 hands lane l dim
//          l of four consecutive tokens.  No lane shuffles move probabilities.
// Codes become fp16 with an and_or magic-exponent unpack and two packed
// fmas (exact code, then code*scale+bias).  The softmax runs in fp32 (exp2);
// probabilities rounded to fp16 feed P.V and the running sum adds those same
// rounded values.
//
// Work decomposition: one wave per (key split, KV head, sequence); a split is
// SB 64-token blocks or the bf16 window; many small waves per SIMD hide the
// load latency.  The split's widths and pool offsets sit one per lane
// (v_readlane), so no block's loads wait on a scalar load.  Partials (max,
// sum, unnormalised output) are combined by the decode merge kernel.
#include "kvq_internal.h"
#include "unpack.h"

namespace kvq {
namespace {

using namespace dev;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

// A lane's full token row of codes: D*B/8 bytes as dwords (sized for 8 bits).
template <int B, int NG>
struct FullRow {
    static constexpr int BYTES = 8 * NG * B;
    static constexpr int NDW = BYTES / 4;

    __device__ static __forceinline__ void load(uint32_t *w, const uint8_t *row)
    {
        if constexpr (BYTES % 16 == 0) {
#pragma unroll
            for (int i = 0; i < BYTES / 16; i++) {
                const uint4 v = reinterpret_cast<const uint4 *>(row)[i];
                w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < BYTES / 8; i++) {
                const uint2 v = reinterpret_cast<const uint2 *>(row)[i];
                w[2 * i] = v.x; w[2 * i + 1] = v.y;
            }
        }
    }

    // Exact codes of chunk c (dims 8c..8c+7) as fp16 pairs.
    __device__ static __forceinline__ Pairs chunk(const uint32_t *w, int c)
    {
        if constexpr (B == 4) {
            return Unpack<4>::run(w[c]);
        } else if constexpr (B == 2) {
            const uint32_t d = w[c >> 1];
            return Unpack<2>::run((c & 1) ? (d >> 16) : (d & 0xffffu));
        } else if constexpr (B == 8) {
            return Unpack<8>::run2(w[2 * c], w[2 * c + 1]);
        } else {
            const int o = 3 * c, i = o >> 2;
            return Unpack<3>::run3(w[i], w[(i + 1 < NDW) ? i + 1 : i], o & 3);
        }
    }
};

template <int NG>
struct State {
    static constexpr int NH = NG;             // 64-dim output sets
    f4 o[NH];                                 // lane (b, j): O[head i][64*hh + 4b + j] in o[hh][i]
    float m_run;                              // running max (log2 domain) of head j
    float l_lane;                             // this lane's share of head j's running sum
};

// Q.K^T of the 64 rows held by the lanes: kdeq(c) yields the dequantized
// fp16 pairs of chunk c of the lane's key row.
template <int NG, typename KF>
__device__ __forceinline__ f4 scores(const h4 (*qs)[4], KF kdeq)
{
    const int j = threadIdx.x & 3;
    f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8 * NG; c++) {
        const Pairs pr = kdeq(c);
        const h4 a0 = {pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1]};
        const h4 a1 = {pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
        s = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, qs[2 * c][j], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, qs[2 * c + 1][j], s, 0, 0, 0);
    }
    return s;
}

// Online softmax on the scores of one 64-token round (lane (b, j): tokens
// 4b..4b+3 of head j), then O += P.V for every 64-dim output set; vdeq(c)
// yields the dequantized pairs of chunk c of the lane's value row.  V rows go
// to LDS in chunk order (position k of a chunk holds dim (k>>1) + 4(k&1)),
// so lane l accumulates output dim 64hh + that permutation of l.
template <int NG, typename VF>
__device__ __forceinline__ void softmax_pv(State<NG> &st, f4 s, int n_valid, float c,
                                           _Float16 *vr, VF vdeq)
{
    constexpr int VS = 64 + 8;                // LDS row stride of one 64-dim set (halves)
    const int lane = threadIdx.x, b = lane >> 2, j = lane & 3;
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) sc[i] = (4 * b + i < n_valid) ? s[i] * c : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.m_run = m_new;
    const h2 p01 = __builtin_convertvector(f2{__builtin_amdgcn_exp2f(sc[0] - m_new),
                                              __builtin_amdgcn_exp2f(sc[1] - m_new)}, h2);
    const h2 p23 = __builtin_convertvector(f2{__builtin_amdgcn_exp2f(sc[2] - m_new),
                                              __builtin_amdgcn_exp2f(sc[3] - m_new)}, h2);
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    st.l_lane = __builtin_amdgcn_fdot2(p23, ones, __builtin_amdgcn_fdot2(p01, ones, st.l_lane * alpha, false), false);
    // alpha of each head, for the output rows this lane holds
    if (__any(alpha != 1.0f)) {
        const int base = lane & ~3;
        const float a0 = __shfl(alpha, base), a1 = __shfl(alpha, base + 1);
        const float a2 = __shfl(alpha, base + 2), a3 = __shfl(alpha, base + 3);
#pragma unroll
        for (int hh = 0; hh < NG; hh++) {
            st.o[hh][0] *= a0; st.o[hh][1] *= a1; st.o[hh][2] *= a2; st.o[hh][3] *= a3;
        }
    }
    const h4 pa = {p01[0], p01[1], p23[0], p23[1]};   // A operand: head j, tokens 4b..4b+3

    // Per 64-dim set: the lane's V row (token = lane) into LDS, then 16
    // slices of 4 tokens.  One wave owns the buffer: its LDS instructions
    // execute in order, so only the compiler needs a barrier between the
    // writes and the reads (and before the next set's writes).
    // Transposed read for slice S: lane i of each 16-lane group addresses
    // token 4S + i/4, positions 16(l/16) + 4(i%4)..+3 of the set.
    const _Float16 *vb = vr + ((lane & 15) >> 2) * VS + 16 * (lane >> 4) + 4 * (lane & 3);
#pragma unroll
    for (int hh = 0; hh < NG; hh++) {
#pragma unroll
        for (int cc = 0; cc < 8; cc++) {
            const Pairs pr = vdeq(8 * hh + cc);
            *reinterpret_cast<h8 *>(vr + lane * VS + 8 * cc) =
                h8{pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1], pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f4 acc = st.o[hh];
#define KVQ_PV(S)                                                                                     \
    acc = __builtin_amdgcn_mfma_f32_4x4x4f16(                                                         \
        pa,                                                                                           \
        __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(                               \
                                   (__attribute__((address_space(3))) s4 *)(vb + 4 * (S) * VS))),   \
        acc, 4, S, 0)
        KVQ_PV(0); KVQ_PV(1); KVQ_PV(2); KVQ_PV(3); KVQ_PV(4); KVQ_PV(5); KVQ_PV(6); KVQ_PV(7);
        KVQ_PV(8); KVQ_PV(9); KVQ_PV(10); KVQ_PV(11); KVQ_PV(12); KVQ_PV(13); KVQ_PV(14); KVQ_PV(15);
#undef KVQ_PV
        st.o[hh] = acc;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// Widths and pool offsets of up to 64 consecutive blocks, one per lane, so
// a block's loads never wait on a dependent scalar load.
struct SplitMeta {
    int base, bits;
    uint32_t klo, khi, vlo, vhi;
};

__device__ __forceinline__ void split_meta(SplitMeta &sm, const DecodeArgs &p, int a, int j0, int j1)
{
    const int jb = j0 + (int)threadIdx.x;
    sm.base = j0;
    sm.bits = 0;
    sm.klo = sm.khi = sm.vlo = sm.vhi = 0;
    if (jb < j1) {
        const size_t e = (size_t)a * p.t.max_blocks + jb;
        sm.bits = p.t.bits[e];
        const uint64_t ko = p.k.offset[e], vo = p.v.offset[e];
        sm.klo = (uint32_t)ko; sm.khi = (uint32_t)(ko >> 32);
        sm.vlo = (uint32_t)vo; sm.vhi = (uint32_t)(vo >> 32);
    }
}

template <int B, int NG>
__device__ __forceinline__ void round_block(State<NG> &st, const h4 (*qs)[4], const uint8_t *kblk,
                                            const uint8_t *vblk, int H, int g, float c, _Float16 *vr)
{
    constexpr uint32_t CODE_ROW = 8 * NG * B;
    constexpr int NDW = FullRow<B, NG>::NDW;
    const uint32_t row = (uint32_t)g * 64 + threadIdx.x;
    const uint32_t moff = (uint32_t)H * 64 * CODE_ROW + 4 * NG * row;
    uint32_t kw[NDW], vw[NDW], km[NG], vm[NG];
    FullRow<B, NG>::load(kw, kblk + row * CODE_ROW);
    FullRow<B, NG>::load(vw, vblk + row * CODE_ROW);
#pragma unroll
    for (int i = 0; i < NG; i++) {
        km[i] = reinterpret_cast<const uint32_t *>(kblk + moff)[i];
        vm[i] = reinterpret_cast<const uint32_t *>(vblk + moff)[i];
    }
    const f4 s = scores<NG>(qs, [&](int cidx) {
        Pairs pr = FullRow<B, NG>::chunk(kw, cidx);
        dequant(pr, km[cidx >> 3]);
        return pr;
    });
    softmax_pv<NG>(st, s, 64, c, vr, [&](int cidx) {
        Pairs pr = FullRow<B, NG>::chunk(vw, cidx);
        dequant(pr, vm[cidx >> 3]);
        return pr;
    });
}

// 64 window tokens w0 .. w0+63 (rows past nw read row nw-1 and are masked).
template <int NG>
__device__ __forceinline__ void round_window(State<NG> &st, const h4 (*qs)[4], const uint16_t *kw,
                                             const uint16_t *vw, int H, int g, int w0, int nw,
                                             float c, _Float16 *vt)
{
    constexpr int D = 64 * NG;
    const int t = min(w0 + (int)threadIdx.x, nw - 1);
    const uint4 *kr = reinterpret_cast<const uint4 *>(kw + ((size_t)t * H + g) * D);
    const uint4 *vr = reinterpret_cast<const uint4 *>(vw + ((size_t)t * H + g) * D);
    const f4 s = scores<NG>(qs, [&](int cidx) { return bf16_pairs(kr[cidx]); });
    softmax_pv<NG>(st, s, nw - w0, c, vt, [&](int cidx) { return bf16_pairs(vr[cidx]); });
}

template <int NG>
__global__ __launch_bounds__(64) void decode_g4_split(DecodeArgs p)
{
    constexpr int D = 64 * NG, NCH = 8 * NG;
    __shared__ __attribute__((aligned(16))) h4 qs[2 * NCH][4];      // [slice][head], permuted dims
    __shared__ __attribute__((aligned(16))) _Float16 vt[64 * 72];  // V rows, one 64-dim set
    const int s = blockIdx.x, g = blockIdx.y, a = blockIdx.z;
    const int lane = threadIdx.x, b = lane >> 2, j = lane & 3;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int nsb = (nb + p.SB - 1) / p.SB;
    const bool win = (s == nsb) && nw > 0;
    if (s > nsb || (s == nsb && !win)) return;

    // Query rows of the G heads, fp16, in the unpack order of the key chunks.
    for (int e = lane; e < 4 * NCH; e += 64) {
        const int h = e / NCH, cc = e % NCH;
        Pairs pr;
        if (h < p.G) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p.q + ((size_t)a * p.Hq + g * p.G + h) * D + 8 * cc);
            pr = bf16_pairs(v);
        } else {
            pr.p[0] = pr.p[1] = pr.p[2] = pr.p[3] = h2{(_Float16)0.0f, (_Float16)0.0f};
        }
        qs[2 * cc][h] = h4{pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1]};
        qs[2 * cc + 1][h] = h4{pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
    }
    __syncthreads();

    State<NG> st;
#pragma unroll
    for (int hh = 0; hh < NG; hh++) st.o[hh] = f4{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_lane = 0.0f;

    if (!win) {
        const int j0 = s * p.SB, j1 = min(j0 + p.SB, nb);
        SplitMeta sm;
        sm.base = -(1 << 20);
        for (int jb = j0; jb < j1; jb++) {
            if (jb - sm.base >= 64) split_meta(sm, p, a, jb, j1);   // blocks are visited in order
            const int i = jb - sm.base;
            const int bw = __builtin_amdgcn_readlane(sm.bits, i);
            const uint8_t *kb = p.k.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sm.khi, i) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane(sm.klo, i));
            const uint8_t *vb = p.v.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sm.vhi, i) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane(sm.vlo, i));
            switch (bw) {
            case 2: round_block<2, NG>(st, qs, kb, vb, p.t.H, g, p.c, vt); break;
            case 3: round_block<3, NG>(st, qs, kb, vb, p.t.H, g, p.c, vt); break;
            case 4: round_block<4, NG>(st, qs, kb, vb, p.t.H, g, p.c, vt); break;
            default: round_block<8, NG>(st, qs, kb, vb, p.t.H, g, p.c, vt); break;
            }
        }
    } else {
        const uint16_t *kw = p.k.window + (size_t)a * p.t.window_cap * p.t.H * D;
        const uint16_t *vw = p.v.window + (size_t)a * p.t.window_cap * p.t.H * D;
        for (int w0 = 0; w0 < nw; w0 += 64) round_window<NG>(st, qs, kw, vw, p.t.H, g, w0, nw, p.c, vt);
    }

    // Head j's sum over the 16 lanes that hold it; outputs of heads < G.
    float l = st.l_lane;
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) l += __shfl_xor(l, o);
    const size_t stride = (size_t)(D + 2);
    const size_t rbase = (size_t)a * p.Hq + (size_t)g * p.G;
    if (b == 0 && j < p.G) {
        float *pr = p.part + ((rbase + j) * p.n_splits + s) * stride;
        pr[0] = st.m_run;
        pr[1] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (i < p.G) {
            float *pr = p.part + ((rbase + i) * p.n_splits + s) * stride + 2;
            // lane l holds dim 64hh + (chunk-order position l)
            const int d = ((4 * b + j) & ~7) | (((4 * b + j) & 7) >> 1) | (((4 * b + j) & 1) << 2);
#pragma unroll
            for (int hh = 0; hh < NG; hh++) pr[64 * hh + d] = st.o[hh][i];
        }
    }
}

}  // namespace

bool decode_g4_supported(int D, int G) { return G <= 4 && (D == 64 || D == 128 || D == 256); }

void decode_g4_plan(int A, int H, int max_blocks, int window_cap, int *SB, int *n_splits)
{
    // Longest splits that still give about KVQ_G4_WAVES waves (latency is
    // hidden by waves in flight; longer splits keep the merge's partials small).
#ifndef KVQ_G4_WAVES
#define KVQ_G4_WAVES 2048
#endif
    int sb = 64;
    while (sb > 1 && (long)A * H * ((max_blocks + sb - 1) / sb) < KVQ_G4_WAVES) sb >>= 1;
    while ((max_blocks + sb - 1) / sb + 1 > 512) sb <<= 1;     // merge limit on splits
    *SB = sb;
    *n_splits = (max_blocks + sb - 1) / sb + (window_cap > 0 ? 1 : 0);
    if (*n_splits < 1) *n_splits = 1;
}

hipError_t launch_decode_g4(const DecodeArgs &p, hipStream_t s)
{
    dim3 grid(p.n_splits, p.t.H, p.t.A);
    switch (p.t.D) {
    case 64: decode_g4_split<1><<<grid, 64, 0, s>>>(p); break;
    case 128: decode_g4_split<2><<<grid, 64, 0, s>>>(p); break;
    case 256: decode_g4_split<4><<<grid, 64, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
