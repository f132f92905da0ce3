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
//      tile gives S^T[16 tokens][16 heads].  Each lane loads a contiguous
//      run of its token's packed codes, turns 8 codes into fp16 with one
//      and_or per pair (the 1024.0 magic exponent), removes the magic with a
//      packed fma and applies scale/bias with a second packed fma.
//   2. V rows are unpacked the same way and written transposed into LDS
//      (V^T[d][token], fp16), the A operand of the P.V MFMA.
//   3. Online softmax in fp32 on the S^T tile (exp2, running max per head);
//      the probabilities, rounded to fp16, are the B operand of P.V, and the
//      running sum adds those same rounded values (so numerator and
//      denominator use identical weights).
// Each split writes (max, sum, unnormalised output) for its rows; the merge
// kernel combines splits.
//
// Rows of the S^T tile are ordered so that lane (head, q) ends up holding
// tokens 8q..8q+7 of the step, which is exactly the B-operand layout P.V
// needs; no shuffles move probabilities between lanes.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr uint32_t MAGIC = 0x64006400u;   // fp16 1024.0 in both halves
constexpr int VT_PAD = 8;                  // LDS row padding (halves)
constexpr int STEP = 32;                   // tokens per step
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t u32_of(h2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Four fp16 pairs (c0,c4) (c1,c5) (c2,c6) (c3,c7) of one chunk of 8 codes,
// as exact small integers in fp16.  `x` holds 1024 + m*c per half; the
// constants undo the magic and the per-position multiplier m.
struct Pairs {
    h2 p[4];
};

template <int B>
struct Unpack;

template <>
struct Unpack<4> {
    // chunk: one dword, code i at bits 4i.
    __device__ static __forceinline__ Pairs run(uint32_t w)
    {
        const uint32_t w8 = w >> 8;
        const h2 x0 = as_h2((w & 0x000F000Fu) | MAGIC);
        const h2 x1 = as_h2((w & 0x00F000F0u) | MAGIC);
        const h2 x2 = as_h2((w8 & 0x000F000Fu) | MAGIC);
        const h2 x3 = as_h2((w8 & 0x00F000F0u) | MAGIC);
        const h2 one = {(_Float16)1.0f, (_Float16)1.0f}, m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
        const h2 s16 = {(_Float16)0.0625f, (_Float16)0.0625f}, m64 = {(_Float16)-64.0f, (_Float16)-64.0f};
        Pairs r;
        r.p[0] = __builtin_elementwise_fma(x0, one, m1024);
        r.p[1] = __builtin_elementwise_fma(x1, s16, m64);
        r.p[2] = __builtin_elementwise_fma(x2, one, m1024);
        r.p[3] = __builtin_elementwise_fma(x3, s16, m64);
        return r;
    }
};

template <>
struct Unpack<2> {
    // chunk: 16 bits (upper half of v zero), code i at bits 2i.
    __device__ static __forceinline__ Pairs run(uint32_t v)
    {
        const uint32_t y = v | (v << 8);          // hi half: codes 4..7 at bits 0..7
        Pairs r;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const h2 x = as_h2((y & (0x00030003u << (2 * i))) | MAGIC);
            const float inv = 1.0f / (float)(1 << (2 * i));
            const h2 s = {(_Float16)inv, (_Float16)inv};
            const h2 b = {(_Float16)(-1024.0f * inv), (_Float16)(-1024.0f * inv)};
            r.p[i] = __builtin_elementwise_fma(x, s, b);
        }
        return r;
    }
};

template <>
struct Unpack<8> {
    // chunk: two dwords, code i at byte i.
    __device__ static __forceinline__ Pairs run2(uint32_t w0, uint32_t w1)
    {
        const h2 one = {(_Float16)1.0f, (_Float16)1.0f}, m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
        Pairs r;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + i) << 16) | (uint32_t)i;
            r.p[i] = __builtin_elementwise_fma(as_h2(perm(w1, w0, sel) | MAGIC), one, m1024);
        }
        return r;
    }
};

template <>
struct Unpack<3> {
    // chunk: 3 bytes starting at byte r of the 8 bytes {lo, hi}; code i at
    // bits 3i of those 24 bits.
    __device__ static __forceinline__ Pairs run3(uint32_t lo, uint32_t hi, int r)
    {
        const uint32_t z = perm(hi, lo, ((uint32_t)(r + 2) << 24) | ((uint32_t)(r + 1) << 16) |
                                            ((uint32_t)(r + 1) << 8) | (uint32_t)r);
        const uint32_t z2 = perm(hi, lo, 0x0C000000u | ((uint32_t)(r + 2) << 16) |
                                             ((uint32_t)(r + 2) << 8) | (uint32_t)(r + 1));
        const h2 x0 = as_h2((z & 0x00700007u) | MAGIC);                 // c0 x1,  c4 x16
        const h2 x1 = as_h2((z & 0x03800038u) | MAGIC);                 // c1 x8,  c5 x128
        const h2 x2 = as_h2((z & 0x000001C0u) | (z2 & 0x001C0000u) | MAGIC);  // c2 x64, c6 x4
        const h2 x3 = as_h2((z2 & 0x00E0000Eu) | MAGIC);                // c3 x2,  c7 x32
        Pairs o;
        o.p[0] = __builtin_elementwise_fma(x0, h2{(_Float16)1.0f, (_Float16)0.0625f},
                                           h2{(_Float16)-1024.0f, (_Float16)-64.0f});
        o.p[1] = __builtin_elementwise_fma(x1, h2{(_Float16)0.125f, (_Float16)0.0078125f},
                                           h2{(_Float16)-128.0f, (_Float16)-8.0f});
        o.p[2] = __builtin_elementwise_fma(x2, h2{(_Float16)0.015625f, (_Float16)0.25f},
                                           h2{(_Float16)-16.0f, (_Float16)-256.0f});
        o.p[3] = __builtin_elementwise_fma(x3, h2{(_Float16)0.5f, (_Float16)0.03125f},
                                           h2{(_Float16)-512.0f, (_Float16)-32.0f});
        return o;
    }
};

// A lane's share of one token row: chunks [q*2NG, (q+1)*2NG) of 8 codes
// (d in [16*NG*q, 16*NG*(q+1))), loaded as dwords.
template <int B, int NG>
struct RowLoad {
    static constexpr int BYTES = 2 * NG * B;                 // codes bytes of the lane
    static constexpr bool ODD = (B == 3 && NG == 1);         // 6 bytes at offset 6q
    static constexpr int NDW = ODD ? 2 : BYTES / 4;
    uint32_t w[NDW];
    int r0;                                                  // byte offset of chunk 0 in w

    __device__ __forceinline__ void load(const uint8_t *row, int q)
    {
        if constexpr (ODD) {
            const int off = 6 * q;
            const uint32_t *p = reinterpret_cast<const uint32_t *>(row + (off & ~3));
            w[0] = p[0];
            w[1] = p[1];
            r0 = off & 3;
        } else {
            const uint8_t *base = row + q * BYTES;
            if constexpr (BYTES % 16 == 0) {
#pragma unroll
                for (int i = 0; i < BYTES / 16; i++) {
                    const uint4 v = reinterpret_cast<const uint4 *>(base)[i];
                    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
                }
            } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
                for (int i = 0; i < BYTES / 8; i++) {
                    const uint2 v = reinterpret_cast<const uint2 *>(base)[i];
                    w[2 * i] = v.x; w[2 * i + 1] = v.y;
                }
            } else {
#pragma unroll
                for (int i = 0; i < NDW; i++) w[i] = reinterpret_cast<const uint32_t *>(base)[i];
            }
            r0 = 0;
        }
    }

    // Exact codes of chunk c as fp16 pairs.
    __device__ __forceinline__ Pairs chunk(int c) const
    {
        if constexpr (B == 4) {
            return Unpack<4>::run(w[c]);
        } else if constexpr (B == 2) {
            const uint32_t d = w[c >> 1];
            return Unpack<2>::run((c & 1) ? (d >> 16) : (d & 0xffffu));
        } else if constexpr (B == 8) {
            return Unpack<8>::run2(w[2 * c], w[2 * c + 1]);
        } else {
            if constexpr (ODD) {
                const int o = r0 + 3 * c;          // o <= 5
                return Unpack<3>::run3(o >= 4 ? w[1] : w[0], w[1], o & 3);
            } else {
                const int o = 3 * c;
                const int i = o >> 2;
                const uint32_t lo = w[i];
                const uint32_t hi = (i + 1 < NDW) ? w[i + 1] : w[i];
                return Unpack<3>::run3(lo, hi, o & 3);
            }
        }
    }
};

// Dequantized fp16 values of a chunk: pairs (c0,c4) .. (c3,c7) -> fma(c, s, b).
__device__ __forceinline__ void dequant(Pairs &pr, uint32_t meta)
{
    const h2 sb = as_h2(meta);
    const h2 s = {sb[0], sb[0]}, b = {sb[1], sb[1]};
#pragma unroll
    for (int i = 0; i < 4; i++) pr.p[i] = __builtin_elementwise_fma(pr.p[i], s, b);
}

__device__ __forceinline__ h8 operand(const Pairs &pr)
{
    h8 v;
    v[0] = pr.p[0][0]; v[1] = pr.p[0][1];
    v[2] = pr.p[1][0]; v[3] = pr.p[1][1];
    v[4] = pr.p[2][0]; v[5] = pr.p[2][1];
    v[6] = pr.p[3][0]; v[7] = pr.p[3][1];
    return v;
}

// Local token (0..31) of row m of S^T tile tau within a step: lane (head, q)
// of the accumulator then holds tokens 8q + 4*tau + j.
__device__ __forceinline__ int tile_token(int m, int tau) { return 8 * (m >> 2) + 4 * tau + (m & 3); }

template <int NG>
struct DecodeState {
    static constexpr int D = 64 * NG;
    static constexpr int KS = 2 * NG;        // K-steps of 32 dims
    static constexpr int NT = D / 16;        // output tiles of 16 dims
    h8 qop[KS];                              // B operand of Q.K^T
    f4 acc[NT];                              // O^T tiles: [d = 16nt + 4q + j][head]
    float m_run, l_run;                      // log2-domain running max, running sum
};

// One 32-token step of a quantized block (half = which 32 tokens of the 64):
// S^T tiles into s[0..1], V^T rows into LDS.
template <int B, int NG>
__device__ __forceinline__ void step_block(const DecodeState<NG> &st, const uint8_t *kblk,
                                           const uint8_t *vblk, int H, int g, int half,
                                           _Float16 *vt, f4 s[2])
{
    constexpr int D = 64 * NG, KS = 2 * NG;
    constexpr int CODE_ROW = D * B / 8;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    const size_t meta0 = (size_t)H * 64 * CODE_ROW;
    const int grp = (NG * q) >> 2;           // group of the lane's dims [16*NG*q, 16*NG*(q+1))

    RowLoad<B, NG> kl[2], vl[2];
    uint32_t km[2], vm[2];
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const size_t row = (size_t)g * 64 + 32 * half + tile_token(m, tau);
        kl[tau].load(kblk + row * CODE_ROW, q);
        vl[tau].load(vblk + row * CODE_ROW, q);
        km[tau] = reinterpret_cast<const uint32_t *>(kblk + meta0)[row * NG + grp];
        vm[tau] = reinterpret_cast<const uint32_t *>(vblk + meta0)[row * NG + grp];
    }
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; k++) {
            Pairs pr = kl[tau].chunk(k);
            dequant(pr, km[tau]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand(pr), st.qop[k], acc, 0, 0, 0);
        }
        s[tau] = acc;
    }
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const int t = tile_token(m, tau);
#pragma unroll
        for (int k = 0; k < KS; k++) {
            Pairs pr = vl[tau].chunk(k);
            dequant(pr, vm[tau]);
            const int d0 = 8 * (q * KS + k);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                vt[(d0 + i) * (STEP + VT_PAD) + t] = pr.p[i][0];
                vt[(d0 + i + 4) * (STEP + VT_PAD) + t] = pr.p[i][1];
            }
        }
    }
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Pairs (e0,e4) (e1,e5) (e2,e6) (e3,e7) of 8 bf16 values, as fp16.
__device__ __forceinline__ Pairs bf16_pairs(uint4 v)
{
    Pairs r;
    r.p[0] = __builtin_convertvector(f2{bf_lo(v.x), bf_lo(v.z)}, h2);
    r.p[1] = __builtin_convertvector(f2{bf_hi(v.x), bf_hi(v.z)}, h2);
    r.p[2] = __builtin_convertvector(f2{bf_lo(v.y), bf_lo(v.w)}, h2);
    r.p[3] = __builtin_convertvector(f2{bf_hi(v.y), bf_hi(v.w)}, h2);
    return r;
}

// One 32-token step of the bf16 window, tokens t0 .. t0+31 (rows past nw are
// read from row nw-1 and masked by the caller).
template <int NG>
__device__ __forceinline__ void step_window(const DecodeState<NG> &st, const uint16_t *kw,
                                            const uint16_t *vw, int H, int g, int t0, int nw,
                                            _Float16 *vt, f4 s[2])
{
    constexpr int D = 64 * NG, KS = 2 * NG;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    uint4 kr[2][KS], vr[2][KS];
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const int t = min(t0 + tile_token(m, tau), nw - 1);
        const uint4 *kp = reinterpret_cast<const uint4 *>(kw + ((size_t)t * H + g) * D + 16 * NG * q);
        const uint4 *vp = reinterpret_cast<const uint4 *>(vw + ((size_t)t * H + g) * D + 16 * NG * q);
#pragma unroll
        for (int k = 0; k < KS; k++) { kr[tau][k] = kp[k]; vr[tau][k] = vp[k]; }
    }
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; k++)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand(bf16_pairs(kr[tau][k])), st.qop[k], acc, 0, 0, 0);
        s[tau] = acc;
    }
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const int t = tile_token(m, tau);
#pragma unroll
        for (int k = 0; k < KS; k++) {
            const Pairs pr = bf16_pairs(vr[tau][k]);
            const int d0 = 8 * (q * KS + k);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                vt[(d0 + i) * (STEP + VT_PAD) + t] = pr.p[i][0];
                vt[(d0 + i + 4) * (STEP + VT_PAD) + t] = pr.p[i][1];
            }
        }
    }
}

// Online softmax on the step's S^T tiles, then O^T += V^T . P^T.
// n_valid: tokens of the step that exist (32 except in the last window step).
template <int NG>
__device__ __forceinline__ void softmax_pv(DecodeState<NG> &st, const f4 s[2], int n_valid,
                                           const _Float16 *vt, float c)
{
    constexpr int NT = 4 * NG;
    const int lane = threadIdx.x, m = lane & 15, q = lane >> 4;
    float sc[8];
#pragma unroll
    for (int tau = 0; tau < 2; tau++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            sc[4 * tau + j] = (8 * q + 4 * tau + j < n_valid) ? s[tau][j] * c : -INFINITY;
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mx = fmaxf(mx, sc[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    h2 ph[4];
    float lsum = 0.0f;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const f2 pv = {__builtin_amdgcn_exp2f(sc[2 * k] - m_new), __builtin_amdgcn_exp2f(sc[2 * k + 1] - m_new)};
        ph[k] = __builtin_convertvector(pv, h2);
        lsum = __builtin_amdgcn_fdot2(ph[k], ones, lsum, false);
    }
    st.l_run = st.l_run * alpha + lsum;
    st.m_run = m_new;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) st.acc[nt] *= alpha;
    }
    h8 pb;
#pragma unroll
    for (int k = 0; k < 4; k++) { pb[2 * k] = ph[k][0]; pb[2 * k + 1] = ph[k][1]; }
    __syncthreads();                          // V^T of this step is in LDS
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const h8 a = *reinterpret_cast<const h8 *>(vt + (16 * nt + m) * (STEP + VT_PAD) + 8 * q);
        st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, st.acc[nt], 0, 0, 0);
    }
    __syncthreads();                          // reads done before the next step writes
}

__device__ __forceinline__ int seq_blocks(const Tables &t, int a) { return clampi(t.n_blocks[a], 0, t.max_blocks); }
__device__ __forceinline__ int seq_window(const Tables &t, int a)
{
    return t.n_window ? clampi(t.n_window[a], 0, t.window_cap) : 0;
}

template <int NG>
__global__ __launch_bounds__(64) void decode_gqa_split(DecodeArgs p)
{
    constexpr int D = 64 * NG, KS = 2 * NG, NT = 4 * NG;
    __shared__ __attribute__((aligned(16))) _Float16 vt[D * (STEP + VT_PAD)];
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
#pragma unroll
    for (int k = 0; k < KS; k++) {
        const int d0 = 8 * (q * KS + k);
        const uint4 v = *reinterpret_cast<const uint4 *>(qrow + d0);
        const Pairs pr = bf16_pairs(v);
        h8 o = operand(pr);
        if (!hv) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
        st.qop[k] = o;
    }
#pragma unroll
    for (int nt = 0; nt < NT; nt++) st.acc[nt] = f4{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_run = 0.0f;

    if (!win) {
        const int j1 = min((s + 1) * p.SB, nb);
        for (int j = s * p.SB; j < j1; j++) {
            const size_t e = (size_t)a * p.t.max_blocks + j;
            const int b = p.t.bits[e];
            const uint8_t *kb = p.k.pool + p.k.offset[e];
            const uint8_t *vb = p.v.pool + p.v.offset[e];
#pragma unroll 1
            for (int half = 0; half < 2; half++) {
                f4 sc[2];
                switch (b) {
                case 2: step_block<2, NG>(st, kb, vb, p.t.H, g, half, vt, sc); break;
                case 3: step_block<3, NG>(st, kb, vb, p.t.H, g, half, vt, sc); break;
                case 4: step_block<4, NG>(st, kb, vb, p.t.H, g, half, vt, sc); break;
                default: step_block<8, NG>(st, kb, vb, p.t.H, g, half, vt, sc); break;
                }
                softmax_pv<NG>(st, sc, STEP, vt, p.c);
            }
        }
    } else {
        const uint16_t *kw = p.k.window + (size_t)a * p.t.window_cap * p.t.H * D;
        const uint16_t *vw = p.v.window + (size_t)a * p.t.window_cap * p.t.H * D;
        for (int t0 = 0; t0 < nw; t0 += STEP) {
            f4 sc[2];
            step_window<NG>(st, kw, vw, p.t.H, g, t0, nw, vt, sc);
            softmax_pv<NG>(st, sc, nw - t0, vt, p.c);
        }
    }

    float l = st.l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (hv) {
        float *pr = p.part + ((size_t)(a * p.Hq + h) * p.n_splits + s) * (D + 2);
        if (q == 0) { pr[0] = st.m_run; pr[1] = l; }
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int j = 0; j < 4; j++) pr[2 + 16 * nt + 4 * q + j] = st.acc[nt][j];
    }
}

// Combine the splits of one (sequence, query head): max-rescaled sums in the
// log2 domain of the split kernel.
__global__ __launch_bounds__(64) void decode_gqa_merge(DecodeArgs p)
{
    const int row = blockIdx.x;
    const int a = row / p.Hq;
    const int D = p.t.D;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int ns = (nb + p.SB - 1) / p.SB + (nw > 0 ? 1 : 0);
    const float *pr = p.part + (size_t)row * p.n_splits * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < ns; s++) M = fmaxf(M, pr[(size_t)s * (D + 2)]);
    float L = 0.0f;
    for (int s = 0; s < ns; s++) L += __builtin_amdgcn_exp2f(pr[(size_t)s * (D + 2)] - M) * pr[(size_t)s * (D + 2) + 1];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float *o = p.out + (size_t)row * D;
    for (int d = threadIdx.x; d < D; d += 64) {
        float acc = 0.0f;
        for (int s = 0; s < ns; s++)
            acc += __builtin_amdgcn_exp2f(pr[(size_t)s * (D + 2)] - M) * pr[(size_t)s * (D + 2) + 2 + d];
        o[d] = acc * inv;
    }
}

}  // namespace

void decode_gqa_plan(int A, int H, int max_blocks, int window_cap, int *SB, int *n_splits)
{
    int sb = 16;
    while (sb > 1 && (long)A * H * ((max_blocks + sb - 1) / sb) < 2048) sb >>= 1;
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
    decode_gqa_merge<<<dim3(p.t.A * p.Hq), 64, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace kvq
