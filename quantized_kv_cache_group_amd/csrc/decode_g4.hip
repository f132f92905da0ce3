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
// leave 12 of its 16 head rows empty.  v_mfma_f32_4x4x4_16b_f16 runs 16
// independent 4x4x4 products, so a wave of 64 lanes maps lane l to token l
// of a 64-token block:
//   Q.K^T  block b = tokens 4b..4b+3; A = K rows (lane = token, 4 dims per
//          instruction), B = the G query rows (read from LDS), so lane (b, j)
//          ends with the scores of tokens 4b..4b+3 for head j;
//   P.V    for each 4-token slice s, A = P[heads][tokens 4s..4s+3], which is
//          exactly what the lanes of block s hold after the softmax, broadcast
//          to all 16 blocks by the instruction's CBSZ/ABID fields; B = V rows
//          of those 4 tokens for 4 output dims per block: each lane writes its
//          V row to LDS and ds_read_b64_tr_b16 hands lane l dim l of four
//          consecutive tokens.  No lane shuffles move probabilities.
//
// Codes are never dequantized element by element.  An and_or with a magic
// exponent turns two codes into the exact fp16 values 1024 + code, and the
// matrix instructions consume those.  Per 64-dim group g of token t (scale
// s, bias b; the restored value is s*code + b):
//   q . K_t  = sum_g s_tg (T_tg - 1024 Q_g) + b_tg Q_g,  T_tg = sum_{d in g} q_d (1024 + code)
//   sum_t p_t V_t[d] = sum_t p'_tg (1024 + code) - 1024 sum_t p'_tg + sum_t p_t b_tg,
//                      p'_tg = fp16(p_t s_tg),
// with Q_g the sum of the (fp16) query over the group, all in fp32.  That
// halves the vector work per code against dequantize-then-multiply, and the
// restored values enter the products unrounded (a token's s and b reach the
// lanes holding its scores through a quad broadcast).  The softmax runs in
// fp32 (exp2); probabilities rounded to fp16 feed the running sum.
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

constexpr int VS = 64;                        // LDS row stride of one 64-dim V set (halves)

// 16-byte chunk c of V row r sits at chunk c ^ vswz(r).  gfx950's LDS serves
// a 16-byte write for 8 lanes per cycle over 32 banks and an 8-byte read for
// 32 lanes over 64 banks; with this swap the row stores (8 consecutive rows,
// one chunk) and the transposed reads (4 consecutive rows x 8 chunks per 32
// lanes) both spread over distinct banks.  A 72-half pitch without the swap
// left every transposed read two-way conflicted.
__device__ __forceinline__ int vswz(int r) { return ((r & 1) ^ ((r & 2) << 1) ^ ((r >> 1) & 2)) << 3; }

// (x & mask) | magic.  Written in plain C so the compiler sees every VALU
// write that feeds a matrix instruction (it inserts the wait states such a
// read needs); magic_v comes from opaque_magic(), a vector register the
// compiler cannot fold back into a literal, so the pair selects to one
// v_and_or_b32 (a VALU instruction here reads at most one scalar register).
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

// A lane's full token row of codes: D*B/8 bytes as dwords.
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

    // Chunk c (8 codes) as the fp16 pairs (1024+c0, 1024+c4) (1024+c1, 1024+c5)
    // (1024+c2, 1024+c6) (1024+c3, 1024+c7), exact.  mv holds MAGIC.
    __device__ static __forceinline__ Pairs chunk(const uint32_t *w, int c, uint32_t mv)
    {
        Pairs r;
        if constexpr (B == 4) {
            const uint32_t x = w[c];                          // code i at bits 4i
#pragma unroll
            for (int i = 0; i < 4; i++) r.p[i] = as_h2(and_or(x >> (4 * i), 0x000F000Fu, mv));
        } else if constexpr (B == 2) {
            const uint32_t d = w[c >> 1];
            const uint32_t v = (c & 1) ? (d >> 16) : (d & 0xffffu);   // code i at bits 2i
            const uint32_t y = v | (v << 8);                  // codes 4..7 at bits 16..23
#pragma unroll
            for (int i = 0; i < 4; i++) r.p[i] = as_h2(and_or(y >> (2 * i), 0x00030003u, mv));
        } else if constexpr (B == 8) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + i) << 16) | (uint32_t)i;
                r.p[i] = as_h2(perm(w[2 * c + 1], w[2 * c], sel) | mv);
            }
        } else {
            // 3 bytes at byte o of the row: code i at bits 3i of those 24
            const int o = 3 * c, i0 = o >> 2, sh = o & 3;     // compile-time after unrolling
            const uint32_t lo = w[i0], hi = w[(i0 + 1 < NDW) ? i0 + 1 : i0];
            const uint32_t u = perm(hi, lo, 0x0C000000u | ((uint32_t)(sh + 2) << 16) |
                                                ((uint32_t)(sh + 1) << 8) | (uint32_t)sh);
            // codes 0..3 stay at bits 0..11, codes 4..7 move to bits 16..27
            const uint32_t z = (u & 0x00000FFFu) | ((u << 4) & 0x0FFF0000u);
#pragma unroll
            for (int i = 0; i < 4; i++) r.p[i] = as_h2(and_or(z >> (3 * i), 0x00070007u, mv));
        }
        return r;
    }
};

template <int NG>
struct State {
    f4 o[NG];                                 // lane (b, j): sum p'(1024+code) for head i, dim 64hh + pos 4b+j
    float m_run;                              // running max (log2 domain) of head j
    float l_lane;                             // this lane's share of head j's running sum
    float ps_lane[NG];                        // this lane's share of head j's sum of p' (coded tokens), per group
    float pb_lane[NG];                        // this lane's share of head j's sum of p*bias, per group
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

// Per-group sums over the lane's key row of q (fp16, from LDS) times the
// row's chunk pairs: T[g] for tokens 4b..4b+3 of head j.
template <int NG, typename KF>
__device__ __forceinline__ void group_dots(f4 (&T)[NG], const h4 (*qs)[4], KF kx)
{
    const int j = threadIdx.x & 3;
#pragma unroll
    for (int g = 0; g < NG; g++) {
        f4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 8 * g; c < 8 * g + 8; c++) {
            const Pairs pr = kx(c);
            const h4 a0 = {pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1]};
            const h4 a1 = {pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
            s0 = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, qs[2 * c][j], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, qs[2 * c + 1][j], s1, 0, 0, 0);
        }
        T[g] = s0 + s1;
    }
}

// Online softmax on the scores of one 64-token round (lane (b, j): tokens
// 4b..4b+3 of head j).  Rescales the state and returns the probabilities
// rounded to fp16 (the running sum adds exactly these).
template <int NG>
__device__ __forceinline__ h4 softmax_round(State<NG> &st, f4 s, int n_valid, float c)
{
    const int lane = threadIdx.x, b = lane >> 2;
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
#pragma unroll
    for (int g = 0; g < NG; g++) {
        st.ps_lane[g] *= alpha;
        st.pb_lane[g] *= alpha;
    }
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
    return h4{p01[0], p01[1], p23[0], p23[1]};
}

__device__ __forceinline__ void wave_sync()
{
    // One wave owns the LDS buffers: its LDS instructions execute in order,
    // so only the compiler needs a barrier between writes and reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// O += P'.X for every 64-dim set hh: each lane writes its token's row of set
// hh to LDS (chunk order: position k of a chunk holds dim (k>>1) + 4(k&1)),
// then 16 slices of 4 tokens whose B operand comes from
// ds_read_b64_tr_b16 (lane l gets position l of four consecutive tokens);
// lane l accumulates output position 64hh + l.  pa(hh) is the A operand of
// set hh; vx(c) yields chunk c of the lane's row.
template <int NG, typename PF, typename VF>
__device__ __forceinline__ void pv_round(State<NG> &st, PF pa, _Float16 *vr, VF vx)
{
    const int lane = threadIdx.x;
    // lane i of each 16-lane group addresses token 4S + i/4, positions
    // 16(l/16) + 4(i%4)..+3 of the set
    // Rows 4S + (lane&15)/4: bit 2 of the row is S&1, so even and odd S use
    // two bases.
    const int r0 = (lane & 15) >> 2, col = 16 * (lane >> 4) + 4 * (lane & 3);
    const _Float16 *vb0 = vr + r0 * VS + (col ^ vswz(r0));
    const _Float16 *vb1 = vr + r0 * VS + (col ^ vswz(r0 + 4));
#pragma unroll
    for (int hh = 0; hh < NG; hh++) {
#pragma unroll
        for (int cc = 0; cc < 8; cc++) {
            const Pairs pr = vx(8 * hh + cc);
            *reinterpret_cast<h8 *>(vr + lane * VS + ((8 * cc) ^ vswz(lane))) =
                h8{pr.p[0][0], pr.p[0][1], pr.p[1][0], pr.p[1][1], pr.p[2][0], pr.p[2][1], pr.p[3][0], pr.p[3][1]};
        }
        wave_sync();
        const h4 a = pa(hh);
        f4 acc0 = st.o[hh], acc1 = {0.f, 0.f, 0.f, 0.f};
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
        st.o[hh] = acc0 + acc1;
        wave_sync();
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

// fp32 (scale, bias) from a packed fp16 pair.
__device__ __forceinline__ f2 meta_of(uint32_t packed)
{
    const h2 sb = as_h2(packed);
    return f2{(float)sb[0], (float)sb[1]};
}

// A 64-token block in three phases: the Q.K products (width-specific
// unpack of the lane's K row), the scores and the online softmax, then P.V
// (width-specific unpack of the V row).
template <int B, int NG>
__device__ __forceinline__ void dots_phase(f4 (&T)[NG], const h4 (*qs)[4], const uint32_t *kw)
{
    const uint32_t mv = opaque_magic();
    group_dots<NG>(T, qs, [&](int cidx) { return FullRow<B, NG>::chunk(kw, cidx, mv); });
}

// scores: sum_g s (T - 1024 Q_g) + b Q_g, with token 4b+r's (s, b) from km;
// returns P' = fp16(p s_v) per group and adds the bias and P' sums.
template <int NG>
__device__ __forceinline__ f4 scores_of(const f4 (&T)[NG], const uint32_t *km, const float (&qg)[NG])
{
    f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < NG; gg++) {
        const float q1024 = 1024.0f * qg[gg];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const f2 ksb = meta_of(quad_bcast(km[gg], r));
            s[r] = __builtin_fmaf(ksb[0], T[gg][r] - q1024, __builtin_fmaf(ksb[1], qg[gg], s[r]));
        }
    }
    return s;
}

template <int NG>
__device__ __forceinline__ void score_phase(State<NG> &st, h4 (&pg)[NG], const f4 (&T)[NG], const uint32_t *km,
                                            const uint32_t *vm, const float (&qg)[NG], float c)
{
    const f4 s = scores_of<NG>(T, km, qg);
    f2 vsb[NG][4];
#pragma unroll
    for (int gg = 0; gg < NG; gg++)
#pragma unroll
        for (int r = 0; r < 4; r++) vsb[gg][r] = meta_of(quad_bcast(vm[gg], r));
    const h4 p = softmax_round<NG>(st, s, 64, c);
    const f4 pf = {(float)p[0], (float)p[1], (float)p[2], (float)p[3]};
#pragma unroll
    for (int gg = 0; gg < NG; gg++) {
        const f4 pv = {pf[0] * vsb[gg][0][0], pf[1] * vsb[gg][1][0], pf[2] * vsb[gg][2][0], pf[3] * vsb[gg][3][0]};
        pg[gg] = __builtin_convertvector(pv, h4);
        st.ps_lane[gg] += ((float)pg[gg][0] + (float)pg[gg][1]) + ((float)pg[gg][2] + (float)pg[gg][3]);
        st.pb_lane[gg] += __builtin_fmaf(pf[0], vsb[gg][0][1], pf[1] * vsb[gg][1][1]) +
                          __builtin_fmaf(pf[2], vsb[gg][2][1], pf[3] * vsb[gg][3][1]);
    }
}

template <int B, int NG>
__device__ __forceinline__ void pv_phase(State<NG> &st, const h4 (&pg)[NG], const uint32_t *vw, _Float16 *vr)
{
    const uint32_t mv = opaque_magic();
    pv_round<NG>(st, [&](int hh) { return pg[hh]; }, vr,
                 [&](int cidx) { return FullRow<B, NG>::chunk(vw, cidx, mv); });
}

// The V row is fetched once the K row's registers are free (a scheduling
// barrier keeps its loads after the K row's last use), so a row's two
// halves are never live together.
template <int B, int NG>
__device__ __forceinline__ void round_block(State<NG> &st, const h4 (*qs)[4], const float (&qg)[NG],
                                            const uint8_t *kblk, const uint8_t *vblk, int H, int g, float c,
                                            _Float16 *vr)
{
    constexpr uint32_t CODE_ROW = 8 * NG * B;
    const uint32_t row = (uint32_t)g * 64 + threadIdx.x;
    const uint32_t moff = (uint32_t)H * 64 * CODE_ROW + 4 * NG * row;
    uint32_t kw[FullRow<B, NG>::NDW], km[NG], vm[NG];
    FullRow<B, NG>::load(kw, kblk + row * CODE_ROW);
#pragma unroll
    for (int i = 0; i < NG; i++) km[i] = reinterpret_cast<const uint32_t *>(kblk + moff)[i];
    f4 T[NG];
    dots_phase<B, NG>(T, qs, kw);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t vw[FullRow<B, NG>::NDW];
    FullRow<B, NG>::load(vw, vblk + row * CODE_ROW);
#pragma unroll
    for (int i = 0; i < NG; i++) vm[i] = reinterpret_cast<const uint32_t *>(vblk + moff)[i];
    h4 pg[NG];
    score_phase<NG>(st, pg, T, km, vm, qg, c);
    pv_phase<B, NG>(st, pg, vw, vr);
}

// 64 window tokens w0 .. w0+63 (rows past nw read row nw-1 and are masked):
// bf16 values straight into the products.
template <int NG>
__device__ __forceinline__ void round_window(State<NG> &st, const h4 (*qs)[4], const uint16_t *kw,
                                             const uint16_t *vw, int H, int g, int w0, int nw,
                                             float c, _Float16 *vr)
{
    constexpr int D = 64 * NG;
    const int t = min(w0 + (int)threadIdx.x, nw - 1);
    const uint4 *kr = reinterpret_cast<const uint4 *>(kw + ((size_t)t * H + g) * D);
    const uint4 *vrow = reinterpret_cast<const uint4 *>(vw + ((size_t)t * H + g) * D);
    f4 T[NG];
    group_dots<NG>(T, qs, [&](int cidx) { return bf16_pairs(kr[cidx]); });
    f4 s = T[0];
#pragma unroll
    for (int gg = 1; gg < NG; gg++) s += T[gg];
    const h4 p = softmax_round<NG>(st, s, nw - w0, c);
    pv_round<NG>(st, [&](int) { return p; }, vr, [&](int cidx) { return bf16_pairs(vrow[cidx]); });
}

// Query rows of KV head g's G heads, fp16, in the unpack order of the key
// chunks, into qs; and Q_g of head j: the sum of its fp16 query over each
// 64-dim group (lane (b, j) adds slice 16g + b, then the 16 lanes of head j
// combine).
template <int NG>
__device__ __forceinline__ void stage_query(const DecodeArgs &p, int a, int g, h4 (*qs)[4], float (&qg)[NG])
{
    constexpr int D = 64 * NG, NCH = 8 * NG;
    const int lane = threadIdx.x, b = lane >> 2, j = lane & 3;
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
    wave_sync();
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int gg = 0; gg < NG; gg++) {
        const h4 v = qs[16 * gg + b][j];
        float acc = __builtin_amdgcn_fdot2(h2{v[2], v[3]}, ones, __builtin_amdgcn_fdot2(h2{v[0], v[1]}, ones, 0.0f, false),
                                           false);
#pragma unroll
        for (int o = 4; o < 64; o <<= 1) acc += __shfl_xor(acc, o);
        qg[gg] = acc;
    }
}

template <int NG>
__global__ __launch_bounds__(64, (NG <= 2 ? 3 : 2)) void decode_g4_split(DecodeArgs p)
{
    constexpr int D = 64 * NG, NCH = 8 * NG;
    __shared__ __attribute__((aligned(16))) h4 qs[2 * NCH][4];      // [slice][head], permuted dims
    __shared__ __attribute__((aligned(16))) _Float16 vt[64 * VS];  // V rows, one 64-dim set
    const int s = blockIdx.x, g = blockIdx.y, a = blockIdx.z;
    const int lane = threadIdx.x, b = lane >> 2, j = lane & 3;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int nsb = (nb + p.SB - 1) / p.SB;
    const bool win = (s == nsb) && nw > 0;
    if (s > nsb || (s == nsb && !win)) return;

    // The split's block table first, so its loads overlap the query loads.
    SplitMeta sm;
    sm.base = -(1 << 20);
    const int j0 = s * p.SB, j1 = min(j0 + p.SB, nb);
    if (!win) split_meta(sm, p, a, j0, j1);

    float qg[NG];
    stage_query<NG>(p, a, g, qs, qg);

    State<NG> st;
#pragma unroll
    for (int hh = 0; hh < NG; hh++) {
        st.o[hh] = f4{0.f, 0.f, 0.f, 0.f};
        st.ps_lane[hh] = 0.0f;
        st.pb_lane[hh] = 0.0f;
    }
    st.m_run = -INFINITY;
    st.l_lane = 0.0f;

    if (!win) {
        for (int jb = j0; jb < j1; jb++) {
            if (jb - sm.base >= 64) split_meta(sm, p, a, jb, j1);   // blocks are visited in order
            const int i = jb - sm.base;
            const int bw = __builtin_amdgcn_readlane(sm.bits, i);
            const uint8_t *kb = p.k.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sm.khi, i) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane(sm.klo, i));
            const uint8_t *vb = p.v.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sm.vhi, i) << 32) |
                                            (uint32_t)__builtin_amdgcn_readlane(sm.vlo, i));
            switch (bw) {
            case 2: round_block<2, NG>(st, qs, qg, kb, vb, p.t.H, g, p.c, vt); break;
            case 3: round_block<3, NG>(st, qs, qg, kb, vb, p.t.H, g, p.c, vt); break;
            case 4: round_block<4, NG>(st, qs, qg, kb, vb, p.t.H, g, p.c, vt); break;
            default: round_block<8, NG>(st, qs, qg, kb, vb, p.t.H, g, p.c, vt); break;
            }
        }
    } else {
        const uint16_t *kw = p.k.window + (size_t)a * p.t.window_cap * p.t.H * D;
        const uint16_t *vw = p.v.window + (size_t)a * p.t.window_cap * p.t.H * D;
        for (int w0 = 0; w0 < nw; w0 += 64) round_window<NG>(st, qs, kw, vw, p.t.H, g, w0, nw, p.c, vt);
    }

    // Head j's sums over the 16 lanes that hold it.
    float l = st.l_lane, ps[NG], pb[NG];
#pragma unroll
    for (int gg = 0; gg < NG; gg++) {
        ps[gg] = st.ps_lane[gg];
        pb[gg] = st.pb_lane[gg];
    }
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) {
        l += __shfl_xor(l, o);
#pragma unroll
        for (int gg = 0; gg < NG; gg++) {
            ps[gg] += __shfl_xor(ps[gg], o);
            pb[gg] += __shfl_xor(pb[gg], o);
        }
    }
    const size_t stride = (size_t)(D + 2);
    const size_t rbase = (size_t)a * p.Hq + (size_t)g * p.G;
    if (b == 0 && j < p.G) {
        float *pr = p.part + ((rbase + j) * p.n_splits + s) * stride;
        pr[0] = st.m_run;
        pr[1] = l;
    }
    // lane l holds dim 64hh + (chunk-order position l) of head i in o[hh][i]:
    // output = sum p'(1024+code) - 1024 sum p' + sum p b (lane i holds head i's sums)
    const int d = ((4 * b + j) & ~7) | (((4 * b + j) & 7) >> 1) | (((4 * b + j) & 1) << 2);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float corr[NG];
#pragma unroll
        for (int gg = 0; gg < NG; gg++) corr[gg] = __shfl(pb[gg], i) - 1024.0f * __shfl(ps[gg], i);
        if (i < p.G) {
            float *pr = p.part + ((rbase + i) * p.n_splits + s) * stride + 2;
#pragma unroll
            for (int hh = 0; hh < NG; hh++) pr[64 * hh + d] = st.o[hh][i] + corr[hh];
        }
    }
}

// Block scores for top-K selection: the Q.K products and scale/bias
// corrections of the decode above, then the largest score of the block over
// its 64 tokens and the KV head's G query heads, times the softmax scale.
// One wave per (split, KV head, sequence); scores_h [A][max_blocks][H].
template <int B, int NG>
__device__ __forceinline__ float block_max(const h4 (*qs)[4], const float (&qg)[NG], const uint8_t *kblk, int H,
                                           int g, int G)
{
    constexpr uint32_t CODE_ROW = 8 * NG * B;
    const uint32_t row = (uint32_t)g * 64 + threadIdx.x;
    const uint32_t moff = (uint32_t)H * 64 * CODE_ROW + 4 * NG * row;
    uint32_t kw[FullRow<B, NG>::NDW], km[NG];
    FullRow<B, NG>::load(kw, kblk + row * CODE_ROW);
#pragma unroll
    for (int i = 0; i < NG; i++) km[i] = reinterpret_cast<const uint32_t *>(kblk + moff)[i];
    f4 T[NG];
    dots_phase<B, NG>(T, qs, kw);
    const f4 s = scores_of<NG>(T, km, qg);
    float m = ((int)(threadIdx.x & 3) < G) ? fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) : -INFINITY;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    return m;
}

template <int NG>
__global__ __launch_bounds__(64, (NG <= 2 ? 3 : 2)) void decode_g4_scores(DecodeArgs p, float scale, float *scores_h)
{
    constexpr int NCH = 8 * NG;
    __shared__ __attribute__((aligned(16))) h4 qs[2 * NCH][4];
    const int s = blockIdx.x, g = blockIdx.y, a = blockIdx.z;
    const int nb = seq_blocks(p.t, a);
    const int j0 = s * p.SB, j1 = min(j0 + p.SB, nb);
    if (j0 >= j1) return;
    SplitMeta sm;
    split_meta(sm, p, a, j0, j1);
    float qg[NG];
    stage_query<NG>(p, a, g, qs, qg);
    for (int jb = j0; jb < j1; jb++) {
        if (jb - sm.base >= 64) split_meta(sm, p, a, jb, j1);   // blocks are visited in order
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
    case 64: decode_g4_split<1><<<grid, 64, 0, s>>>(p); break;
    case 128: decode_g4_split<2><<<grid, 64, 0, s>>>(p); break;
    case 256: decode_g4_split<4><<<grid, 64, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
