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
// Work decomposition: one workgroup per (key split, KV head, sequence); a
// split is SB 64-token blocks or the bf16 window.  Each wave of the workgroup
// owns GW consecutive 64-dim groups of head_dim (a group is the quantizer's
// unit: one scale/bias per token).  For each block a wave loads its groups of
// every token's K and V rows together (lane = token), so a wave keeps 8*GW*b
// bytes per lane of both tensors in flight; when a head spans several waves
// they add their partial scores through LDS in a fixed order, so every wave
// holds the same full scores and runs the same online softmax, and each wave
// accumulates the output dims of its own groups.
//
// Matrix products on the codes themselves.  v_mfma_f32_4x4x4_16b_f16 runs 16
// independent 4x4x4 products, so lane l of a wave is token l of a block:
//   Q.K^T  block b = tokens 4b..4b+3; A = K values (lane = token, 4 dims per
//          instruction), B = the G query rows (read from LDS), so lane (b, j)
//          ends with the scores of tokens 4b..4b+3 for head j;
//   P.V    for each 4-token slice s, A = P[heads][tokens 4s..4s+3], which is
//          exactly what the lanes of block s hold after the softmax, broadcast
//          to all 16 blocks by the instruction's CBSZ/ABID fields; B = V values
//          of those 4 tokens for 4 output dims per block: each lane writes its
//          V values to LDS and ds_read_b64_tr_b16 hands lane l dim l of four
//          consecutive tokens.
// A code c of width b enters the products as the exact fp16 value 1024 + m*c:
// an and_or with the magic exponent 0x6400 places the code at the top of the
// fp16 mantissa (m = 64, 64, 16, 1 for b = 2, 3, 4, 8), so the constant 1024
// is at most ~10 times the code term and the fp32 sums lose almost nothing to
// it.  Per 64-dim group of token t (scale s, bias b; restored value s*c + b):
//   q . K_t  = (s/m) (T_t - 1024 Q) + b Q,   T_t = sum_d q_d (1024 + m c_td),
//              Q = sum_d q_d (fp16 query, fp32 sum);
//   sum_t p_t V_t[d] = ( sum_t p''_t (1024 + m c_td) - 1024 sum_t p''_t ) / 64
//                      + sum_t p_t b_t,   p''_t = fp16(p_t s_t 64/m),
// so the largest term of a sum is at most a few times its result.  The
// factor 64/m keeps p'' in fp16 range for every width (|x| <= 65504 bounds
// s), and the correction sums the same rounded p'' the products used.  The
// softmax runs in fp32 (exp2) with an exact running max, so p <= 1.
//
// Each split writes (max, sum, unnormalised output) of its rows; the decode
// merge kernel combines the splits.
#include "kvq_internal.h"
#include "unpack.h"

namespace kvq {
namespace {

using namespace dev;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

constexpr int VS = 64;                        // LDS row stride of the V tile (halves)
constexpr float FV = 64.0f;                   // probability factor of the V products

// 16-byte chunk c of V row r sits at chunk c ^ vswz(r).  gfx950's LDS serves
// a 16-byte write for 8 lanes per cycle over 32 banks and an 8-byte read for
// 32 lanes over 64 banks; with this swap the row stores (8 consecutive rows,
// one chunk) and the transposed reads (4 consecutive rows x 8 chunks per 32
// lanes) both spread over distinct banks.
__device__ __forceinline__ int vswz(int r) { return ((r & 1) ^ ((r & 2) << 1) ^ ((r >> 1) & 2)) << 3; }

// (x & mask) | magic as one v_and_or_b32 (magic in a vector register from
// opaque_magic(), so the mask may take the one scalar operand slot).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic_v)
{
    return (x & mask) | magic_v;
}

__device__ __forceinline__ uint32_t opaque_magic()
{
    uint32_t m = MAGIC;
    asm("" : "+v"(m));                        // emits nothing; pins the value to a vector register
    return m;
}

// Code multiplier m of width B: where the code sits in the fp16 mantissa.
template <int B> struct CodeMul;
template <> struct CodeMul<2> { static constexpr float M = 64.0f; };   // bits 6..7
template <> struct CodeMul<3> { static constexpr float M = 64.0f; };   // bits 6..8
template <> struct CodeMul<4> { static constexpr float M = 16.0f; };   // bits 4..7
template <> struct CodeMul<8> { static constexpr float M = 1.0f; };    // bits 0..7

// A lane's 64-dim group of one token row: 8*B bytes of codes, as dwords.
template <int B>
struct GroupRow {
    static constexpr int BYTES = 8 * B;
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

    // Chunk c (codes 8c..8c+7 of the group) as the fp16 pairs
    // (1024 + m c0, 1024 + m c4) (.. c1, c5) (.. c2, c6) (.. c3, c7), exact.
    __device__ static __forceinline__ Pairs chunk(const uint32_t *w, int c, uint32_t mv)
    {
        Pairs r;
        if constexpr (B == 4) {
            // code i at bits 4i: pair i sits at bits (4i, 16 + 4i); move it to bits 4..7
            const uint32_t x = w[c];
            r.p[0] = as_h2(and_or(x << 4, 0x00F000F0u, mv));
            r.p[1] = as_h2(and_or(x, 0x00F000F0u, mv));
            r.p[2] = as_h2(and_or(x >> 4, 0x00F000F0u, mv));
            r.p[3] = as_h2(and_or(x >> 8, 0x00F000F0u, mv));
        } else if constexpr (B == 2) {
            const uint32_t d = w[c >> 1];
            const uint32_t v = (c & 1) ? (d >> 16) : (d & 0xffffu);   // code i at bits 2i
            const uint32_t y = v | (v << 8);                  // pair i at bits (2i, 16 + 2i)
            r.p[0] = as_h2(and_or(y << 6, 0x00C000C0u, mv));
            r.p[1] = as_h2(and_or(y << 4, 0x00C000C0u, mv));
            r.p[2] = as_h2(and_or(y << 2, 0x00C000C0u, mv));
            r.p[3] = as_h2(and_or(y, 0x00C000C0u, mv));
        } else if constexpr (B == 8) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + i) << 16) | (uint32_t)i;
                r.p[i] = as_h2(perm(w[2 * c + 1], w[2 * c], sel) | mv);
            }
        } else {
            // 3 bytes at byte 3c of the group: code i at bits 3i of those 24
            const int o = 3 * c, i0 = o >> 2, sh = o & 3;     // compile-time after unrolling
            const uint32_t lo = w[i0], hi = w[(i0 + 1 < NDW) ? i0 + 1 : i0];
            const uint32_t u = perm(hi, lo, 0x0C000000u | ((uint32_t)(sh + 2) << 16) |
                                                ((uint32_t)(sh + 1) << 8) | (uint32_t)sh);
            // codes 0..3 stay at bits 0..11, codes 4..7 move to bits 16..27:
            // pair i at bits (3i, 16 + 3i); move it to bits 6..8
            const uint32_t z = (u & 0x00000FFFu) | ((u << 4) & 0x0FFF0000u);
            r.p[0] = as_h2(and_or(z << 6, 0x01C001C0u, mv));
            r.p[1] = as_h2(and_or(z << 3, 0x01C001C0u, mv));
            r.p[2] = as_h2(and_or(z, 0x01C001C0u, mv));
            r.p[3] = as_h2(and_or(z >> 3, 0x01C001C0u, mv));
        }
        return r;
    }
};

template <int GW>
struct State {
    f4 o[GW];                                 // lane (b, j): sum p''(1024+m c) for head i, position 4b+j of group u
    float m_run;                              // running max (log2 domain) of head j
    float l_lane;                             // this lane's share of head j's running sum
    float ps_lane[GW];                        // this lane's share of head j's sum of p'' (coded tokens), per group
    float pb_lane[GW];                        // this lane's share of head j's sum of p*bias, per group
};

// Token 4b+r's 32-bit value broadcast to the four lanes of quad b.
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int r)
{
    switch (r) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, true);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, true);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, true);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, true);
    }
}

// Sum over the lane's group row of q (fp16, from LDS) times the row's chunk
// pairs: T for tokens 4b..4b+3 of head j.
template <typename KF>
__device__ __forceinline__ f4 group_dot(const h4 (*qs)[4], KF kx)
{
    const int j = threadIdx.x & 3;
    f4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; c++) {
        const Pairs pr = kx(c);
        const h4 a0 = {pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1]};
        const h4 a1 = {pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
        s0 = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, qs[2 * c][j], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, qs[2 * c + 1][j], s1, 0, 0, 0);
    }
    return s0 + s1;
}

// Online softmax on the scores of one 64-token round (lane (b, j): tokens
// 4b..4b+3 of head j).  Rescales the state and returns the probabilities in
// fp32 (p <= 1).
template <int GW>
__device__ __forceinline__ f4 softmax_round(State<GW> &st, f4 s, int n_valid, float c)
{
    const int lane = threadIdx.x & 63, b = lane >> 2;
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) sc[i] = (4 * b + i < n_valid) ? s[i] * c : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.m_run = m_new;
    st.l_lane *= alpha;
#pragma unroll
    for (int u = 0; u < GW; u++) {
        st.ps_lane[u] *= alpha;
        st.pb_lane[u] *= alpha;
    }
    // alpha of each head, for the output rows this lane holds
    if (__any(alpha != 1.0f)) {
        const int base = lane & ~3;
        const float a0 = __shfl(alpha, base), a1 = __shfl(alpha, base + 1);
        const float a2 = __shfl(alpha, base + 2), a3 = __shfl(alpha, base + 3);
#pragma unroll
        for (int u = 0; u < GW; u++) {
            st.o[u][0] *= a0; st.o[u][1] *= a1; st.o[u][2] *= a2; st.o[u][3] *= a3;
        }
    }
    return f4{__builtin_amdgcn_exp2f(sc[0] - m_new), __builtin_amdgcn_exp2f(sc[1] - m_new),
              __builtin_amdgcn_exp2f(sc[2] - m_new), __builtin_amdgcn_exp2f(sc[3] - m_new)};
}

__device__ __forceinline__ void wave_sync()
{
    // One wave owns its LDS V tile: its LDS instructions execute in order,
    // so only the compiler needs a barrier between writes and reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// O += P.X for one 64-dim group: each lane writes its token's values to LDS
// (chunk order: position k of a chunk holds dim (k>>1) + 4(k&1)), then 16
// slices of 4 tokens whose B operand comes from ds_read_b64_tr_b16 (lane l
// gets position l of four consecutive tokens); lane l accumulates group
// position l.  vx(c) yields chunk c of the lane's row.
template <typename VF>
__device__ __forceinline__ f4 pv_round(f4 o, h4 a, _Float16 *vr, VF vx)
{
    const int lane = threadIdx.x & 63;
    // lane i of each 16-lane group addresses token 4S + i/4, positions
    // 16(l/16) + 4(i%4)..+3; bit 2 of the row is S&1, so even and odd S use
    // two bases.
    const int r0 = (lane & 15) >> 2, col = 16 * (lane >> 4) + 4 * (lane & 3);
    const _Float16 *vb0 = vr + r0 * VS + (col ^ vswz(r0));
    const _Float16 *vb1 = vr + r0 * VS + (col ^ vswz(r0 + 4));
#pragma unroll
    for (int cc = 0; cc < 8; cc++) {
        const Pairs pr = vx(cc);
        *reinterpret_cast<h8 *>(vr + lane * VS + ((8 * cc) ^ vswz(lane))) =
            h8{pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1], pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
    }
    wave_sync();
    f4 acc0 = o, acc1 = {0.f, 0.f, 0.f, 0.f};
#define KVQ_PV(ACC, S)                                                                                \
    ACC = __builtin_amdgcn_mfma_f32_4x4x4f16(                                                         \
        a,                                                                                            \
        __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(                               \
                                   (__attribute__((address_space(3))) s4 *)(((S) & 1 ? vb1 : vb0) + 4 * (S) * VS))), \
        ACC, 4, S, 0)
    KVQ_PV(acc0, 0); KVQ_PV(acc1, 1); KVQ_PV(acc0, 2); KVQ_PV(acc1, 3);
    KVQ_PV(acc0, 4); KVQ_PV(acc1, 5); KVQ_PV(acc0, 6); KVQ_PV(acc1, 7);
    KVQ_PV(acc0, 8); KVQ_PV(acc1, 9); KVQ_PV(acc0, 10); KVQ_PV(acc1, 11);
    KVQ_PV(acc0, 12); KVQ_PV(acc1, 13); KVQ_PV(acc0, 14); KVQ_PV(acc1, 15);
#undef KVQ_PV
    wave_sync();
    return acc0 + acc1;
}

// Widths and pool offsets of up to 64 consecutive blocks, one per lane, so
// a block's loads never wait on a dependent scalar load.
struct SplitMeta {
    int base, bits;
    uint32_t klo, khi, vlo, vhi;
};

__device__ __forceinline__ void split_meta(SplitMeta &sm, const DecodeArgs &p, int a, int j0, int j1, bool with_v)
{
    const int jb = j0 + (int)(threadIdx.x & 63);
    sm.base = j0;
    sm.bits = 0;
    sm.klo = sm.khi = sm.vlo = sm.vhi = 0;
    if (jb < j1) {
        const size_t e = (size_t)a * p.t.max_blocks + jb;
        sm.bits = p.t.bits[e];
        const uint64_t ko = p.k.offset[e];
        sm.klo = (uint32_t)ko; sm.khi = (uint32_t)(ko >> 32);
        if (with_v) {
            const uint64_t vo = p.v.offset[e];
            sm.vlo = (uint32_t)vo; sm.vhi = (uint32_t)(vo >> 32);
        }
    }
}

// fp32 (scale, bias) from a packed fp16 pair.
__device__ __forceinline__ f2 meta_of(uint32_t packed)
{
    const h2 sb = as_h2(packed);
    return f2{(float)sb[0], (float)sb[1]};
}

// Partial scores of one group for tokens 4b..4b+3 of head j:
// (s/m)(T - 1024 Q) + b Q with token 4b+r's (s, b) from km.
template <int B>
__device__ __forceinline__ f4 group_scores(const h4 (*qs)[4], float qg, const uint32_t *kw, uint32_t km)
{
    const uint32_t mv = opaque_magic();
    const f4 T = group_dot(qs, [&](int c) { return GroupRow<B>::chunk(kw, c, mv); });
    const float q1024 = 1024.0f * qg;
    f4 s;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const f2 ksb = meta_of(quad_bcast(km, r));
        s[r] = __builtin_fmaf(ksb[0] * (1.0f / CodeMul<B>::M), T[r] - q1024, ksb[1] * qg);
    }
    return s;
}

// Full scores from the waves' partials: each wave stores its partial in
// LDS, the workgroup meets at a barrier, and every wave adds the NW
// partials in the same order (so all waves hold identical scores).
template <int NW>
__device__ __forceinline__ f4 exchange(f4 part, f4 (*xs)[64], int w)
{
    if constexpr (NW == 1) {
        return part;
    } else {
        const int lane = threadIdx.x & 63;
        xs[w][lane] = part;
        __syncthreads();
        f4 s = xs[0][lane];
#pragma unroll
        for (int u = 1; u < NW; u++) s += xs[u][lane];
        return s;
    }
}

// One 64-token block: the K rows of the wave's GW groups for every token,
// the Q.K products and the exchange, then the V rows, the softmax and P.V
// per group.
template <int B, int NG, int GW>
__device__ __forceinline__ void round_block(State<GW> &st, const h4 (*qs)[4], const float *qg, const uint8_t *kblk,
                                            const uint8_t *vblk, int H, int g, int w, float c, _Float16 *vr,
                                            f4 (*xs)[64])
{
    constexpr int NW = NG / GW, ND = GroupRow<B>::NDW;
    constexpr uint32_t ROW = 8 * NG * B;                  // bytes of a full token row
    const uint32_t tok = (uint32_t)g * 64 + (threadIdx.x & 63);
    const uint32_t roff = tok * ROW + 8 * B * GW * w;
    const uint32_t moff = (uint32_t)H * 64 * ROW + 4 * (NG * tok + GW * w);
    uint32_t kw[GW * ND], vw[GW * ND], km[GW], vm[GW];
#pragma unroll
    for (int u = 0; u < GW; u++) GroupRow<B>::load(kw + ND * u, kblk + roff + 8 * B * u);
#pragma unroll
    for (int u = 0; u < GW; u++) km[u] = reinterpret_cast<const uint32_t *>(kblk + moff)[u];

    f4 part = group_scores<B>(qs, qg[0], kw, km[0]);
#pragma unroll
    for (int u = 1; u < GW; u++) part += group_scores<B>(qs + 16 * u, qg[u], kw + ND * u, km[u]);
    // the V rows are fetched once the K rows' registers are free (measured
    // faster than issuing them with the K rows: fewer live registers)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < GW; u++) GroupRow<B>::load(vw + ND * u, vblk + roff + 8 * B * u);
#pragma unroll
    for (int u = 0; u < GW; u++) vm[u] = reinterpret_cast<const uint32_t *>(vblk + moff)[u];
    const f4 s = exchange<NW>(part, xs, w);
    const f4 p = softmax_round<GW>(st, s, 64, c);
    st.l_lane += (p[0] + p[1]) + (p[2] + p[3]);
    const uint32_t mv = opaque_magic();
#pragma unroll
    for (int u = 0; u < GW; u++) {
        // p'' = fp16(p s 64/m) per token (the V scale of token 4b+r from its quad)
        f4 pv, pbv;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const f2 vsb = meta_of(quad_bcast(vm[u], r));
            pv[r] = p[r] * (vsb[0] * (FV / CodeMul<B>::M));
            pbv[r] = p[r] * vsb[1];
        }
        const h4 pa = __builtin_convertvector(pv, h4);
        st.ps_lane[u] += ((float)pa[0] + (float)pa[1]) + ((float)pa[2] + (float)pa[3]);
        st.pb_lane[u] += (pbv[0] + pbv[1]) + (pbv[2] + pbv[3]);
        st.o[u] = pv_round(st.o[u], pa, vr, [&](int cidx) { return GroupRow<B>::chunk(vw + ND * u, cidx, mv); });
    }
}

// 64 window tokens w0 .. w0+63 (rows past nw read row nw-1 and are masked):
// bf16 values straight into the products, probabilities rounded to fp16.
template <int NG, int GW>
__device__ __forceinline__ void round_window(State<GW> &st, const h4 (*qs)[4], const uint16_t *kwin,
                                             const uint16_t *vwin, int H, int g, int w, int w0, int nw, float c,
                                             _Float16 *vr, f4 (*xs)[64])
{
    constexpr int D = 64 * NG, NW = NG / GW;
    const int t = min(w0 + (int)(threadIdx.x & 63), nw - 1);
    const uint4 *kr = reinterpret_cast<const uint4 *>(kwin + ((size_t)t * H + g) * D + 64 * GW * w);
    const uint4 *vrow = reinterpret_cast<const uint4 *>(vwin + ((size_t)t * H + g) * D + 64 * GW * w);
    f4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < GW; u++)
        part += group_dot(qs + 16 * u, [&](int cidx) { return bf16_pairs(kr[8 * u + cidx]); });
    const f4 s = exchange<NW>(part, xs, w);
    const f4 p = softmax_round<GW>(st, s, nw - w0, c);
    const h4 pa = __builtin_convertvector(p, h4);
    // the running sum adds the rounded probabilities the products use
    st.l_lane += ((float)pa[0] + (float)pa[1]) + ((float)pa[2] + (float)pa[3]);
#pragma unroll
    for (int u = 0; u < GW; u++)
        st.o[u] = pv_round(st.o[u], pa, vr, [&](int cidx) { return bf16_pairs(vrow[8 * u + cidx]); });
}

// Query rows of KV head g's G heads for the 64 dims [64gr, 64gr+64), fp16,
// in the unpack order of the key chunks, into qs; returns Q of head j: the
// sum of its fp16 query over the group (lane (b, j) adds slice b, then the 16
// lanes of head j combine).
__device__ __forceinline__ float stage_query(const DecodeArgs &p, int a, int g, int gr, h4 (*qs)[4])
{
    const int lane = threadIdx.x & 63, b = lane >> 2, j = lane & 3;
    const int D = p.t.D;
    {
        const int h = lane >> 3, cc = lane & 7;                 // 4 heads x 8 chunks = 32 lanes
        if (lane < 32) {
            Pairs pr;
            if (h < p.G) {
                const uint4 v = *reinterpret_cast<const uint4 *>(p.q + ((size_t)a * p.Hq + g * p.G + h) * D +
                                                                 64 * gr + 8 * cc);
                pr = bf16_pairs(v);
            } else {
                pr.p[0] = pr.p[1] = pr.p[2] = pr.p[3] = h2{(_Float16)0.0f, (_Float16)0.0f};
            }
            qs[2 * cc][h] = h4{pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1]};
            qs[2 * cc + 1][h] = h4{pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
        }
    }
    wave_sync();
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    const h4 v = qs[b][j];
    float acc = __builtin_amdgcn_fdot2(h2{v[2], v[3]}, ones, __builtin_amdgcn_fdot2(h2{v[0], v[1]}, ones, 0.0f, false),
                                       false);
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) acc += __shfl_xor(acc, o);
    return acc;
}

// NG groups of head_dim, GW of them per wave.
template <int NG, int GW>
__global__ __launch_bounds__(64 * (NG / GW)) void decode_g4_split(DecodeArgs p)
{
    constexpr int D = 64 * NG, NW = NG / GW;
    __shared__ __attribute__((aligned(16))) h4 qs[NW][16 * GW][4];        // [wave][slice][head]
    __shared__ __attribute__((aligned(16))) _Float16 vt[NW][64 * VS];      // V tile per wave
    __shared__ __attribute__((aligned(16))) f4 xs[NW > 1 ? 2 : 1][NW][64]; // partial scores
    const int s = blockIdx.x, g = blockIdx.y, a = blockIdx.z;
    const int lane = threadIdx.x & 63, b = lane >> 2, j = lane & 3;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int nsb = (nb + p.SB - 1) / p.SB;
    const bool win = (s == nsb) && nw > 0;
    if (s > nsb || (s == nsb && !win)) return;

    // The split's block table first, so its loads overlap the query loads.
    SplitMeta sm;
    sm.base = -(1 << 20);
    const int j0 = s * p.SB, j1 = min(j0 + p.SB, nb);
    if (!win) split_meta(sm, p, a, j0, j1, true);

    float qg[GW];
#pragma unroll
    for (int u = 0; u < GW; u++) qg[u] = stage_query(p, a, g, GW * w + u, qs[w] + 16 * u);

    State<GW> st;
#pragma unroll
    for (int u = 0; u < GW; u++) {
        st.o[u] = f4{0.f, 0.f, 0.f, 0.f};
        st.ps_lane[u] = st.pb_lane[u] = 0.0f;
    }
    st.m_run = -INFINITY;
    st.l_lane = 0.0f;

    int buf = 0;
    if (!win) {
        for (int jb = j0; jb < j1; jb++, buf ^= (NW > 1)) {
            if (jb - sm.base >= 64) split_meta(sm, p, a, jb, j1, true);   // blocks are visited in order
            const int i = jb - sm.base;
            const int bw = __builtin_amdgcn_readlane(sm.bits, i);
            const uint8_t *kb = p.k.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sm.khi, i) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane(sm.klo, i));
            const uint8_t *vb = p.v.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sm.vhi, i) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane(sm.vlo, i));
            switch (bw) {
            case 2: round_block<2, NG, GW>(st, qs[w], qg, kb, vb, p.t.H, g, w, p.c, vt[w], xs[buf]); break;
            case 3: round_block<3, NG, GW>(st, qs[w], qg, kb, vb, p.t.H, g, w, p.c, vt[w], xs[buf]); break;
            case 4: round_block<4, NG, GW>(st, qs[w], qg, kb, vb, p.t.H, g, w, p.c, vt[w], xs[buf]); break;
            default: round_block<8, NG, GW>(st, qs[w], qg, kb, vb, p.t.H, g, w, p.c, vt[w], xs[buf]); break;
            }
        }
    } else {
        const uint16_t *kwin = p.k.window + (size_t)a * p.t.window_cap * p.t.H * D;
        const uint16_t *vwin = p.v.window + (size_t)a * p.t.window_cap * p.t.H * D;
        for (int w0 = 0; w0 < nw; w0 += 64, buf ^= (NW > 1))
            round_window<NG, GW>(st, qs[w], kwin, vwin, p.t.H, g, w, w0, nw, p.c, vt[w], xs[buf]);
    }

    // Head j's sums over the 16 lanes that hold it.
    float l = st.l_lane, ps[GW], pb[GW];
#pragma unroll
    for (int u = 0; u < GW; u++) {
        ps[u] = st.ps_lane[u];
        pb[u] = st.pb_lane[u];
    }
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) {
        l += __shfl_xor(l, o);
#pragma unroll
        for (int u = 0; u < GW; u++) {
            ps[u] += __shfl_xor(ps[u], o);
            pb[u] += __shfl_xor(pb[u], o);
        }
    }
    const size_t stride = (size_t)(D + 2);
    const size_t rbase = (size_t)a * p.Hq + (size_t)g * p.G;
    if (w == 0 && b == 0 && j < p.G) {
        float *pr = p.part + ((rbase + j) * p.n_splits + s) * stride;
        pr[0] = st.m_run;
        pr[1] = l;
    }
    // lane l holds position l (dim 64(GW w + u) + d) of head i in o[u][i]:
    // output = (sum p''(1024+m c) - 1024 sum p'')/64 + sum p b for coded
    // tokens, sum p v for the window (lane i holds head i's sums)
    const int d = (lane & ~7) | ((lane & 7) >> 1) | ((lane & 1) << 2);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float psi[GW], pbi[GW];
#pragma unroll
        for (int u = 0; u < GW; u++) {
            psi[u] = __shfl(ps[u], i);
            pbi[u] = __shfl(pb[u], i);
        }
        if (i < p.G) {
            float *pr = p.part + ((rbase + i) * p.n_splits + s) * stride + 2 + 64 * GW * w + d;
#pragma unroll
            for (int u = 0; u < GW; u++)
                pr[64 * u] = win ? st.o[u][i] : __builtin_fmaf(st.o[u][i] - 1024.0f * psi[u], 1.0f / FV, pbi[u]);
        }
    }
}

// Block scores for top-K selection: the Q.K products and scale/bias
// corrections of the decode above, over every group of the head, then the
// largest score of the block over its 64 tokens and the KV head's G query
// heads, times the softmax scale.  One wave per (split, KV head, sequence);
// scores_h [A][max_blocks][H].
template <int B, int NG>
__device__ __forceinline__ float block_max(const h4 (*qs)[16][4], const float *qg, const uint8_t *kblk, int H,
                                           int g, int G)
{
    constexpr uint32_t ROW = 8 * NG * B;
    const uint32_t tok = (uint32_t)g * 64 + threadIdx.x;
    uint32_t kw[NG][GroupRow<B>::NDW], km[NG];
#pragma unroll
    for (int w = 0; w < NG; w++) {
        GroupRow<B>::load(kw[w], kblk + tok * ROW + 8 * B * w);
        km[w] = *reinterpret_cast<const uint32_t *>(kblk + (uint32_t)H * 64 * ROW + 4 * (NG * tok + w));
    }
    f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NG; w++) s += group_scores<B>(qs[w], qg[w], kw[w], km[w]);
    float m = ((int)(threadIdx.x & 3) < G) ? fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) : -INFINITY;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    return m;
}

template <int NG>
__global__ __launch_bounds__(64) void decode_g4_scores(DecodeArgs p, float scale, float *scores_h)
{
    __shared__ __attribute__((aligned(16))) h4 qs[NG][16][4];
    const int s = blockIdx.x, g = blockIdx.y, a = blockIdx.z;
    const int nb = seq_blocks(p.t, a);
    const int j0 = s * p.SB, j1 = min(j0 + p.SB, nb);
    if (j0 >= j1) return;
    SplitMeta sm;
    split_meta(sm, p, a, j0, j1, false);
    float qg[NG];
#pragma unroll
    for (int w = 0; w < NG; w++) qg[w] = stage_query(p, a, g, w, qs[w]);
    for (int jb = j0; jb < j1; jb++) {
        if (jb - sm.base >= 64) split_meta(sm, p, a, jb, j1, false);   // blocks are visited in order
        const int i = jb - sm.base;
        const int bw = __builtin_amdgcn_readlane(sm.bits, i);
        const uint8_t *kb = p.k.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sm.khi, i) << 32) |
                                        (uint32_t)__builtin_amdgcn_readlane(sm.klo, i));
        float m;
        switch (bw) {
        case 2: m = block_max<2, NG>(qs, qg, kb, p.t.H, g, p.G); break;
        case 3: m = block_max<3, NG>(qs, qg, kb, p.t.H, g, p.G); break;
        case 4: m = block_max<4, NG>(qs, qg, kb, p.t.H, g, p.G); break;
        default: m = block_max<8, NG>(qs, qg, kb, p.t.H, g, p.G); break;
        }
        if (threadIdx.x == 0) scores_h[((size_t)a * p.t.max_blocks + jb) * p.t.H + g] = scale * m;
    }
}

}  // namespace

bool decode_g4_supported(int D, int G) { return G <= 4 && (D == 64 || D == 128 || D == 256); }

// 64-dim groups per wave: head_dim 64 and 128 run one wave per workgroup,
// head_dim 256 two waves of 128 dims (measured against one wave of 256 dims
// and four of 64: fewer registers per wave than the first, less repeated
// softmax work and LDS than the second).
constexpr int GW256 = 2;

static int g4_waves(int D) { return D == 256 ? 4 / GW256 : 1; }

void decode_g4_plan(int A, int H, int D, int max_blocks, int window_cap, int *SB, int *n_splits)
{
    // Longest splits that still give about 2048 workgroups (more, shorter
    // splits and fewer, longer ones both measured slower on the Llama and
    // Gemma decode shapes); the merge reads at most 512 splits.
    (void)D;
    int sb = 64;
    while (sb > 1 && (long)A * H * ((max_blocks + sb - 1) / sb) < 2048) sb >>= 1;
    while ((max_blocks + sb - 1) / sb + 1 > 512) sb <<= 1;
    *SB = sb;
    *n_splits = (max_blocks + sb - 1) / sb + (window_cap > 0 ? 1 : 0);
    if (*n_splits < 1) *n_splits = 1;
}

hipError_t launch_g4_scores(const DecodeArgs &p, float scale, float *scores_h, hipStream_t s)
{
    const int nsb = (p.t.max_blocks + p.SB - 1) / p.SB;
    if (nsb == 0) return hipSuccess;
    dim3 grid(nsb, p.t.H, p.t.A);
    switch (p.t.D) {
    case 64: decode_g4_scores<1><<<grid, 64, 0, s>>>(p, scale, scores_h); break;
    case 128: decode_g4_scores<2><<<grid, 64, 0, s>>>(p, scale, scores_h); break;
    case 256: decode_g4_scores<4><<<grid, 64, 0, s>>>(p, scale, scores_h); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_g4(const DecodeArgs &p, hipStream_t s)
{
    dim3 grid(p.n_splits, p.t.H, p.t.A);
    switch (p.t.D) {
    case 64: decode_g4_split<1, 1><<<grid, 64, 0, s>>>(p); break;
    case 128: decode_g4_split<2, 2><<<grid, 64, 0, s>>>(p); break;
    case 256: decode_g4_split<4, GW256><<<grid, 64 * g4_waves(256), 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_merge(p, s);
}

}  // namespace kvq
