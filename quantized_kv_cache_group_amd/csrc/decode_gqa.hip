// Batched split-K decode over quantized K/V blocks, grouped-query attention
// (gfx950, matrix cores).
//
// What it computes (Agent Memory Below the Prompt, arXiv 2603.04428,
// Abstract: batched inference over several agents' quantized caches restored
// directly into the attention layer; QKVShare, Metodologia: the fused
// quantized attention kernel): for sequence a and query head h, softmax
// attention of q[a][h] over the 64*n_blocks[a] quantized tokens and the
// n_window[a] bf16 tokens of KV head h / G.
//
// Work decomposition: one wave64 per (key split, KV head, sequence).  A split
// is SB whole 64-token blocks, or the bf16 window.  The wave walks its split
// in steps of 32 tokens:
//   1. K rows are the A operand of v_mfma_f32_16x16x32_f16 (16 tokens x 32
//      dims), the G query heads (padded to 16) the B operand, so one MFMA
//      tile gives S^T[16 tokens][16 heads].  Every 32-dim K-step lies in one
//      64-dim group: lane q of a token row holds codes 16q..16q+15 of each
//      group, turned into exact fp16 integers (one and_or per pair with the
//      1024.0 magic exponent, one packed fma to remove it).  Each group's
//      products accumulate on their own, and the score is
//      sum_g (s_tg T_tg + b_tg Q_g) in fp32, T_tg = sum_{d in g} q_d c_td,
//      Q_g = sum_{d in g} q_d, with each token's (scale, bias) read from LDS.
//   2. V codes, also exact, are written transposed into LDS (V^T[d][token]),
//      the A operand of the P.V MFMA; the B operand of a 16-dim output tile
//      is fp16(p_t s_tg) for the tile's group g, and sum_t p_t b_tg is added
//      in fp32.  No restored value is rounded to fp16, so the output error
//      is the rounding of p s, not of the values themselves.
//   3. Online softmax in fp32 on the S^T tile (exp2, running max per head);
//      the probabilities are rounded to fp16 once, and both the running sum
//      and the products use those rounded values.
// Each split writes (max, sum, unnormalised output) for its rows; the merge
// kernel combines splits.
//
// Rows of the S^T tile are ordered so that lane (head, q) ends up holding
// tokens 8q..8q+7 of the step, which is exactly the B-operand layout P.V
// needs; no shuffles move probabilities between lanes.
#include "kvq_internal.h"
#include "unpack.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int VT_PAD = 8;                  // LDS row padding (halves)
constexpr int STEP = 32;                   // tokens per step

// Local token (0..31) of row m of S^T tile tau within a step: lane (head, q)
// of the accumulator then holds tokens 8q + 4*tau + j.
__device__ __forceinline__ int tile_token(int m, int tau) { return 8 * (m >> 2) + 4 * tau + (m & 3); }

template <int NG>
struct DecodeState {
    static constexpr int D = 64 * NG;
    static constexpr int KS = 2 * NG;        // K-steps of 32 dims (two per group)
    static constexpr int NT = D / 16;        // output tiles of 16 dims
    h8 qop[KS];                              // B operand of Q.K^T
    float qsum[NG];                          // Q_g of the lane's head
    f4 acc[NT];                              // O^T tiles: [d = 16nt + 4q + j][head], sum p s c
    float bacc[NG];                          // the lane's share of sum_t p_t b_tg
    float m_run, l_run;                      // log2-domain running max, running sum
};

// Per-step (scale, bias) of every token and group, K then V, written by the
// lanes that load them (lane q < NG loads group q of its rows).
template <int NG>
struct StepMeta {
    uint32_t k[NG][STEP], v[NG][STEP];
};

// Registers of one 32-token step of a quantized block, loaded ahead of use.
// Sized for widths up to 4 bits; 8-bit blocks load at compute time instead.
template <int NG>
struct Raw {
    static constexpr int KW = 2 * NG;        // dwords per (tensor, tile) at 4 bits
    uint32_t k[2][KW], v[2][KW];
    uint32_t km[2], vm[2];
};

__device__ __forceinline__ size_t step_row(int g, int half, int m, int tau)
{
    return (size_t)g * 64 + 32 * half + tile_token(m, tau);
}

template <int B, int NG, int W>
__device__ __forceinline__ void load_rows(uint32_t (&kw)[2][W], uint32_t (&vw)[2][W], uint32_t km[2],
                                          uint32_t vm[2], const uint8_t *kblk, const uint8_t *vblk, int H,
                                          int g, int half)
{
    constexpr int CODE_ROW = 64 * NG * B / 8, GB = 8 * B, ND = GRow<B>::NDW;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    const size_t meta0 = (size_t)H * 64 * CODE_ROW;
    const int grp = q < NG ? q : 0;
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const size_t row = step_row(g, half, m, tau);
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
            GRow<B>::load(kw[tau] + ND * gg, kblk + row * CODE_ROW + GB * gg, q);
            GRow<B>::load(vw[tau] + ND * gg, vblk + row * CODE_ROW + GB * gg, q);
        }
        km[tau] = reinterpret_cast<const uint32_t *>(kblk + meta0)[row * NG + grp];
        vm[tau] = reinterpret_cast<const uint32_t *>(vblk + meta0)[row * NG + grp];
    }
}

template <int B, int NG>
__device__ __forceinline__ void load_step(Raw<NG> &r, const uint8_t *kblk, const uint8_t *vblk, int H, int g,
                                          int half)
{
    load_rows<B, NG, Raw<NG>::KW>(r.k, r.v, r.km, r.vm, kblk, vblk, H, g, half);
}

// Per-group S^T tiles of the step into T[tau][group]; V^T codes of the step
// and the step's (scale, bias) words into LDS.
template <int B, int NG, int W>
__device__ __forceinline__ void compute_rows(const DecodeState<NG> &st, const uint32_t (&kw)[2][W],
                                             const uint32_t (&vw)[2][W], const uint32_t km[2],
                                             const uint32_t vm[2], _Float16 *vt, StepMeta<NG> &sm,
                                             f4 (&T)[2][NG])
{
    constexpr int ND = GRow<B>::NDW;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 2; u++)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand(GRow<B>::chunk(kw[tau] + ND * gg, q, u)),
                                                             st.qop[2 * gg + u], acc, 0, 0, 0);
            T[tau][gg] = acc;
        }
    }
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const int t = tile_token(m, tau);
        if (q < NG) {
            sm.k[q][t] = km[tau];
            sm.v[q][t] = vm[tau];
        }
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const Pairs pr = GRow<B>::chunk(vw[tau] + ND * gg, q, u);
                const int d0 = 8 * (8 * gg + 2 * q + u);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    vt[(d0 + i) * (STEP + VT_PAD) + t] = pr.p[i][0];
                    vt[(d0 + i + 4) * (STEP + VT_PAD) + t] = pr.p[i][1];
                }
            }
        }
    }
}

// 8-bit blocks: load and compute in place (no prefetch registers).
template <int NG>
__device__ __forceinline__ void step_block8(const DecodeState<NG> &st, const uint8_t *kblk,
                                            const uint8_t *vblk, int H, int g, int half,
                                            _Float16 *vt, StepMeta<NG> &sm, f4 (&T)[2][NG])
{
    constexpr int W = 4 * NG;
    uint32_t kw[2][W], vw[2][W], km[2], vm[2];
    load_rows<8, NG, W>(kw, vw, km, vm, kblk, vblk, H, g, half);
    compute_rows<8, NG, W>(st, kw, vw, km, vm, vt, sm, T);
}


// One 32-token step of the bf16 window, tokens t0 .. t0+31 (rows past nw are
// read from row nw-1 and masked by the caller): values straight into the
// products (scale 1, bias 0).
template <int NG>
__device__ __forceinline__ void step_window(const DecodeState<NG> &st, const uint16_t *kw,
                                            const uint16_t *vw, int H, int g, int t0, int nw,
                                            _Float16 *vt, f4 (&T)[2][NG])
{
    constexpr int D = 64 * NG;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    uint4 kr[2][2 * NG], vr[2][2 * NG];
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const int t = min(t0 + tile_token(m, tau), nw - 1);
        const uint16_t *kp = kw + ((size_t)t * H + g) * D;
        const uint16_t *vp = vw + ((size_t)t * H + g) * D;
#pragma unroll
        for (int k = 0; k < 2 * NG; k++) {
            const int c = 8 * (k >> 1) + 2 * q + (k & 1);      // chunk of K-step k
            kr[tau][k] = *reinterpret_cast<const uint4 *>(kp + 8 * c);
            vr[tau][k] = *reinterpret_cast<const uint4 *>(vp + 8 * c);
        }
    }
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 2; u++)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand(bf16_pairs(kr[tau][2 * gg + u])),
                                                             st.qop[2 * gg + u], acc, 0, 0, 0);
            T[tau][gg] = acc;
        }
    }
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const int t = tile_token(m, tau);
#pragma unroll
        for (int k = 0; k < 2 * NG; k++) {
            const Pairs pr = bf16_pairs(vr[tau][k]);
            const int d0 = 8 * (8 * (k >> 1) + 2 * q + (k & 1));
#pragma unroll
            for (int i = 0; i < 4; i++) {
                vt[(d0 + i) * (STEP + VT_PAD) + t] = pr.p[i][0];
                vt[(d0 + i + 4) * (STEP + VT_PAD) + t] = pr.p[i][1];
            }
        }
    }
}

// Online softmax on the step's scores, then O^T += V^T . P'^T per 16-dim
// tile.  WIN: window step (scores are the plain sums, values carry no scale
// or bias).  n_valid: tokens of the step that exist (32 except in the last
// window step).
template <int NG, bool WIN>
__device__ __forceinline__ void softmax_pv(DecodeState<NG> &st, const f4 (&T)[2][NG], int n_valid,
                                           const _Float16 *vt, const StepMeta<NG> &sm, float c)
{
    constexpr int NT = 4 * NG;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    __syncthreads();                          // V^T and the step's meta are in LDS
    float sc[8];
    if constexpr (WIN) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float v = 0.0f;
#pragma unroll
            for (int gg = 0; gg < NG; gg++) v += T[i >> 2][gg][i & 3];
            sc[i] = v;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) sc[i] = 0.0f;
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
            const uint4 m0 = *reinterpret_cast<const uint4 *>(&sm.k[gg][8 * q]);
            const uint4 m1 = *reinterpret_cast<const uint4 *>(&sm.k[gg][8 * q + 4]);
            const uint32_t mw[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const h2 sb = as_h2(mw[i]);
                sc[i] = __builtin_fmaf((float)sb[0], T[i >> 2][gg][i & 3],
                                       __builtin_fmaf((float)sb[1], st.qsum[gg], sc[i]));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) sc[i] = (8 * q + i < n_valid) ? sc[i] * c : -INFINITY;
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mx = fmaxf(mx, sc[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    h2 ph[4];
    float pf[8];
    float lsum = 0.0f;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const f2 pv = {__builtin_amdgcn_exp2f(sc[2 * k] - m_new), __builtin_amdgcn_exp2f(sc[2 * k + 1] - m_new)};
        ph[k] = __builtin_convertvector(pv, h2);
        pf[2 * k] = (float)ph[k][0];
        pf[2 * k + 1] = (float)ph[k][1];
        lsum = __builtin_amdgcn_fdot2(ph[k], ones, lsum, false);
    }
    st.l_run = st.l_run * alpha + lsum;
    st.m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) st.acc[nt] *= alpha;
#pragma unroll
        for (int gg = 0; gg < NG; gg++) st.bacc[gg] *= alpha;
    }
    h8 pb[NG];
    if constexpr (WIN) {
        h8 o;
#pragma unroll
        for (int k = 0; k < 4; k++) { o[2 * k] = ph[k][0]; o[2 * k + 1] = ph[k][1]; }
#pragma unroll
        for (int gg = 0; gg < NG; gg++) pb[gg] = o;
    } else {
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
            const uint4 m0 = *reinterpret_cast<const uint4 *>(&sm.v[gg][8 * q]);
            const uint4 m1 = *reinterpret_cast<const uint4 *>(&sm.v[gg][8 * q + 4]);
            const uint32_t mw[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            float bsum = 0.0f;
            h8 o;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const h2 sb = as_h2(mw[i]);
                o[i] = (_Float16)(pf[i] * (float)sb[0]);
                bsum = __builtin_fmaf(pf[i], (float)sb[1], bsum);
            }
            pb[gg] = o;
            st.bacc[gg] += bsum;
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const h8 a = *reinterpret_cast<const h8 *>(vt + (16 * nt + m) * (STEP + VT_PAD) + 8 * q);
        st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[nt >> 2], st.acc[nt], 0, 0, 0);
    }
    __syncthreads();                          // reads done before the next step writes
}


template <int NG>
__global__ __launch_bounds__(64) void decode_gqa_split(DecodeArgs p)
{
    constexpr int D = 64 * NG, NT = 4 * NG;
    __shared__ __attribute__((aligned(16))) _Float16 vt[D * (STEP + VT_PAD)];
    __shared__ __attribute__((aligned(16))) StepMeta<NG> sm;
    const int s = blockIdx.x, g = blockIdx.y, a = blockIdx.z;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int nsb = (nb + p.SB - 1) / p.SB;
    const bool win = (s == nsb) && nw > 0;
    if (s > nsb || (s == nsb && !win)) return;

    DecodeState<NG> st;
    const int h = g * p.G + m;
    const bool hv = m < p.G;
    const uint16_t *qrow = p.q + ((size_t)a * p.Hq + (hv ? h : 0)) * D;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int gg = 0; gg < NG; gg++) {
        float qs = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int c = 8 * gg + 2 * q + u;                 // chunk of K-step 2gg + u
            const uint4 v = *reinterpret_cast<const uint4 *>(qrow + 8 * c);
            const Pairs pr = bf16_pairs(v);
            h8 o = operand(pr);
            if (!hv) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
            st.qop[2 * gg + u] = o;
#pragma unroll
            for (int i = 0; i < 4; i++) qs = __builtin_amdgcn_fdot2(h2{o[2 * i], o[2 * i + 1]}, ones, qs, false);
        }
        qs += __shfl_xor(qs, 16);
        qs += __shfl_xor(qs, 32);
        st.qsum[gg] = qs;
        st.bacc[gg] = 0.0f;
    }
#pragma unroll
    for (int nt = 0; nt < NT; nt++) st.acc[nt] = f4{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_run = 0.0f;

    if (!win) {
        const int j0 = s * p.SB;
        const int n_steps = 2 * (min(j0 + p.SB, nb) - j0);
        const uint8_t *kbase = p.k.pool, *vbase = p.v.pool;
        const size_t e0 = (size_t)a * p.t.max_blocks + j0;
        const int H = p.t.H;
        Raw<NG> ra, rb;
        auto issue = [&](Raw<NG> &r, int i) {
            const size_t e = e0 + (i >> 1);
            const int b = p.t.bits[e];
            const uint8_t *kb = kbase + p.k.offset[e], *vb = vbase + p.v.offset[e];
            switch (b) {
            case 2: load_step<2, NG>(r, kb, vb, H, g, i & 1); break;
            case 3: load_step<3, NG>(r, kb, vb, H, g, i & 1); break;
            case 4: load_step<4, NG>(r, kb, vb, H, g, i & 1); break;
            default: break;                       // 8-bit: loaded at compute time
            }
        };
        auto run = [&](const Raw<NG> &r, int i) {
            const size_t e = e0 + (i >> 1);
            const int b = p.t.bits[e];
            f4 T[2][NG];
            switch (b) {
            case 2: compute_rows<2, NG, Raw<NG>::KW>(st, r.k, r.v, r.km, r.vm, vt, sm, T); break;
            case 3: compute_rows<3, NG, Raw<NG>::KW>(st, r.k, r.v, r.km, r.vm, vt, sm, T); break;
            case 4: compute_rows<4, NG, Raw<NG>::KW>(st, r.k, r.v, r.km, r.vm, vt, sm, T); break;
            default:
                step_block8<NG>(st, kbase + p.k.offset[e], vbase + p.v.offset[e], H, g, i & 1, vt, sm, T);
                break;
            }
            softmax_pv<NG, false>(st, T, STEP, vt, sm, p.c);
        };
        if (n_steps > 0) issue(ra, 0);
        for (int i = 0; i < n_steps; i += 2) {
            issue(rb, i + 1);                     // every block has two steps
            run(ra, i);
            if (i + 2 < n_steps) issue(ra, i + 2);
            run(rb, i + 1);
        }
    } else {
        const uint16_t *kw = p.k.window + (size_t)a * p.t.window_cap * p.t.H * D;
        const uint16_t *vw = p.v.window + (size_t)a * p.t.window_cap * p.t.H * D;
        for (int t0 = 0; t0 < nw; t0 += STEP) {
            f4 T[2][NG];
            step_window<NG>(st, kw, vw, p.t.H, g, t0, nw, vt, T);
            softmax_pv<NG, true>(st, T, nw - t0, vt, sm, p.c);
        }
    }

    float l = st.l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float bt[NG];
#pragma unroll
    for (int gg = 0; gg < NG; gg++) {
        bt[gg] = st.bacc[gg];
        bt[gg] += __shfl_xor(bt[gg], 16);
        bt[gg] += __shfl_xor(bt[gg], 32);
    }
    if (hv) {
        float *pr = p.part + ((size_t)(a * p.Hq + h) * p.n_splits + s) * (D + 2);
        if (q == 0) { pr[0] = st.m_run; pr[1] = l; }
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int j = 0; j < 4; j++) pr[2 + 16 * nt + 4 * q + j] = st.acc[nt][j] + bt[nt >> 2];
    }
}

// Combine the splits of one (sequence, query head): max-rescaled sums in the
// log2 domain of the split kernel.  One wave per row and 64-dim slice
// (grid.y).  Up to 64 splits, lane s reads split s's (max, sum) and every
// lane reads its dim of all the partial outputs, all before the first use,
// so the row costs one memory round trip; longer rows keep the split weights
// in LDS and stream the partials.
constexpr int MERGE_ROWS = 4;
constexpr int MAX_SPLITS = 512;

__global__ __launch_bounds__(64 * MERGE_ROWS) void decode_gqa_merge(DecodeArgs p)
{
    __shared__ float wsh[MERGE_ROWS][MAX_SPLITS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x * MERGE_ROWS + wave;
    if (row >= p.t.A * p.Hq) return;
    const int a = row / p.Hq;
    const int D = p.t.D;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int ns = (nb + p.SB - 1) / p.SB + (nw > 0 ? 1 : 0);
    const size_t stride = (size_t)(D + 2);
    const float *pr = p.part + (size_t)row * p.n_splits * stride;
    float *o = p.out + (size_t)row * D;
    const int d = 64 * blockIdx.y + lane;
    if (ns <= 64) {
        if (ns == 0) {
            if (d < D) o[d] = 0.0f;
            return;
        }
        const int sl = min(lane, ns - 1), dd = min(d, D - 1);
        const float mv = pr[sl * stride], lv = pr[sl * stride + 1];
        float v[64];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            if (16 * c < ns) {
#pragma unroll
                for (int u = 0; u < 16; u++) v[16 * c + u] = pr[min(16 * c + u, ns - 1) * stride + 2 + dd];
            }
        }
        float M = lane < ns ? mv : -INFINITY;
#pragma unroll
        for (int x = 32; x > 0; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
        const float w = (lane < ns && M > -INFINITY) ? __builtin_amdgcn_exp2f(mv - M) : 0.0f;
        float L = w * lv;
#pragma unroll
        for (int x = 32; x > 0; x >>= 1) L += __shfl_xor(L, x);
        float ax = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            if (16 * c < ns) {
#pragma unroll
                for (int u = 0; u < 16; u++)
                    ax = __builtin_fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), 16 * c + u)),
                                        v[16 * c + u], ax);
            }
        }
        if (d < D) o[d] = L > 0.0f ? ax * (1.0f / L) : 0.0f;
        return;
    }
    float M = -INFINITY;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, pr[s * stride]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.0f;
    for (int s = lane; s < ns; s += 64) {
        const float w = __builtin_amdgcn_exp2f(pr[s * stride] - M);
        wsh[wave][s] = w;
        L += w * pr[s * stride + 1];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (d < D) {
        float ax = 0.0f;
        int s = 0;
        for (; s + 8 <= ns; s += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) v[u] = pr[(s + u) * stride + 2 + d];
#pragma unroll
            for (int u = 0; u < 8; u++) ax += wsh[wave][s + u] * v[u];
        }
        for (; s < ns; s++) ax += wsh[wave][s] * pr[s * stride + 2 + d];
        o[d] = ax * inv;
    }
}

}  // namespace

void decode_gqa_plan(int A, int H, int max_blocks, int window_cap, int *SB, int *n_splits)
{
    int sb = 16;
    while (sb > 1 && (long)A * H * ((max_blocks + sb - 1) / sb) < 2048) sb >>= 1;
#ifdef KVQ_DECODE_SB
    sb = KVQ_DECODE_SB;                     // build-time tuning override
#endif
    while ((max_blocks + sb - 1) / sb + 1 > MAX_SPLITS) sb <<= 1;
    *SB = sb;
    *n_splits = (max_blocks + sb - 1) / sb + (window_cap > 0 ? 1 : 0);
    if (*n_splits < 1) *n_splits = 1;
}

bool decode_gqa_supported(int D) { return D == 64 || D == 128 || D == 256; }

hipError_t launch_decode_gqa(const DecodeArgs &p, hipStream_t s)
{
    dim3 grid(p.n_splits, p.t.H, p.t.A);
    switch (p.t.D) {
    case 64: decode_gqa_split<1><<<grid, 64, 0, s>>>(p); break;
    case 128: decode_gqa_split<2><<<grid, 64, 0, s>>>(p); break;
    case 256: decode_gqa_split<4><<<grid, 64, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_merge(p, s);
}

hipError_t launch_decode_merge(const DecodeArgs &p, hipStream_t s)
{
    decode_gqa_merge<<<dim3((p.t.A * p.Hq + MERGE_ROWS - 1) / MERGE_ROWS, (p.t.D + 63) / 64), 64 * MERGE_ROWS, 0,
                       s>>>(p);
    return hipGetLastError();
}

}  // namespace kvq
