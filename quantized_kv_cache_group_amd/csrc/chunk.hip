// Chunk attention for new-phase tokens over a restored quantized cache
// (gfx950, matrix cores).
//
// What it computes (Agent Memory Below the Prompt, arXiv 2603.04428,
// Abstract: cross-phase context injection, new tokens attending to a cache
// restored in 4-bit form without recomputing the earlier phase): for new
// token i of sequence a and query head h, softmax attention over the
// 64*n_blocks[a] quantized tokens, the n_window[a] bf16 window tokens and the
// new tokens 0..i, all of KV head h / G.
//
// Work decomposition: a workgroup is WV waves x 32 query rows of one KV
// head; a query row is a (new token, query head) pair, token-major.  Keys
// are walked in tiles of 64 (one quantized block), split across SPLITS
// workgroups whose partials the merge kernel combines.  Per tile:
//   1. all lanes dequantize the tile into LDS: K as fp16 rows (dims in
//      the chunk order the unpack produces), V transposed (V^T[d][key]) with
//      keys permuted so a lane's 8 probabilities line up with 8 consecutive
//      LDS halves; the raw codes of the next tile are already in registers;
//   2. each wave computes S^T = K.Q^T with v_mfma_f32_32x32x16_f16 (A = 32
//      keys x 16 dims from LDS, B = the wave's 32 query rows from registers),
//      so lane l owns query row l%32 and 16 of every 32 keys;
//   3. online softmax per row in fp32 (exp2), probabilities rounded to fp16
//      (the running sum adds the rounded values);
//   4. O^T += V^T.P^T (A = 32 dims x 16 keys from LDS, B = P^T from the
//      lane's own registers).
// The 32x32x16 shape sustains about 1.5x the rate of 16x16x32 here.
// The causal mask only applies to tiles that reach the new tokens.
#include "kvq_internal.h"
#include "unpack.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int TILE = 64;          // keys per tile
constexpr float LAZY = 8.0f;      // running-max slack, log2 units
template <int NG>
struct Cfg {
    static constexpr int D = 64 * NG;
    // 8 waves (2 per SIMD) up to head_dim 128; at 256 the O^T and Q operands
    // need the whole 512-register file of a wave, so 4 waves.
    static constexpr int WV = NG == 4 ? 4 : 8;
    static constexpr int NR = 32;                         // query rows per wave (one 32-row tile)
    static constexpr int ROWS = WV * NR;                  // rows per workgroup
    static constexpr int KS = D / 16;                     // K-steps of S^T = K.Q^T
    static constexpr int DT = D / 32;                     // 32-dim output tiles
    static constexpr int KROW = D + 8;                    // LDS K row stride (halves)
    static constexpr int VROW = TILE + 8;                 // LDS V^T row stride (halves)
    static constexpr int CPT = D / (8 * WV);              // chunks of 8 dims per dequant lane
};

// Position of key k (0..63) of a tile in the V^T rows.  In the S^T tile of
// v_mfma_f32_32x32x16_f16 lane half h holds, for the 16 keys of P.V K-step u,
// keys 16u + 8a + 4h + b (a, b in 0..1, 0..3) in register order; placing
// them at 16u + 8h + 4a + b makes them 8 consecutive halves of a V^T row.
__device__ __forceinline__ int vpos(int k)
{
    const int u = k >> 4, kk = k & 15;
    return 16 * u + 8 * ((kk & 7) >> 2) + 4 * (kk >> 3) + (kk & 3);
}

// Raw registers of one dequant lane's share of a tile: key = lane (0..63),
// dims [w*D/WV, (w+1)*D/WV) for wave w of WV, so one LDS write instruction of
// a wave covers 64 keys of one V^T row (no bank conflicts).  Sized for bf16
// rows, which also covers every code width.
template <int NG>
struct TileRaw {
    static constexpr int W = 4 * Cfg<NG>::CPT;            // dwords
    uint32_t k[W], v[W];
    uint32_t km, vm;
    int bits;                                             // 0: bf16 rows, else code width
    int r0;                                               // byte offset of chunk 0 in k/v
};

// Load CPT*B code bytes of a row share: dwords covering [off, off+CPT*B);
// r0 is the byte offset of the first code byte in the first dword.
template <int NG, int B>
__device__ __forceinline__ void load_codes(uint32_t (&k)[TileRaw<NG>::W], uint32_t (&v)[TileRaw<NG>::W], int &r0,
                                           const uint8_t *krow, const uint8_t *vrow, int off)
{
    constexpr int NB = Cfg<NG>::CPT * B;                 // bytes
    if constexpr (NB % 4 == 0) {                          // offset is a multiple of NB: aligned
        constexpr int NDW = NB / 4;
        if constexpr (NB % 16 == 0) {
#pragma unroll
            for (int i = 0; i < NDW / 4; i++) {
                const uint4 x = reinterpret_cast<const uint4 *>(krow + off)[i];
                const uint4 y = reinterpret_cast<const uint4 *>(vrow + off)[i];
                k[4 * i] = x.x; k[4 * i + 1] = x.y; k[4 * i + 2] = x.z; k[4 * i + 3] = x.w;
                v[4 * i] = y.x; v[4 * i + 1] = y.y; v[4 * i + 2] = y.z; v[4 * i + 3] = y.w;
            }
        } else if constexpr (NB % 8 == 0) {
#pragma unroll
            for (int i = 0; i < NDW / 2; i++) {
                const uint2 x = reinterpret_cast<const uint2 *>(krow + off)[i];
                const uint2 y = reinterpret_cast<const uint2 *>(vrow + off)[i];
                k[2 * i] = x.x; k[2 * i + 1] = x.y;
                v[2 * i] = y.x; v[2 * i + 1] = y.y;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NDW; i++) {
                k[i] = reinterpret_cast<const uint32_t *>(krow + off)[i];
                v[i] = reinterpret_cast<const uint32_t *>(vrow + off)[i];
            }
        }
    } else {
        // 2 or 3 bytes (head_dim 64) or 6 bytes (head_dim 128 at 3 bits) at an
        // unaligned offset: the two dwords around them.  The second one stays
        // inside the block (code rows are followed by the metadata).
        const int base = off & ~3;
        const uint2 x = {reinterpret_cast<const uint32_t *>(krow + base)[0],
                         reinterpret_cast<const uint32_t *>(krow + base)[1]};
        const uint2 y = {reinterpret_cast<const uint32_t *>(vrow + base)[0],
                         reinterpret_cast<const uint32_t *>(vrow + base)[1]};
        k[0] = x.x; k[1] = x.y;
        v[0] = y.x; v[1] = y.y;
        r0 = off & 3;
    }
}

// Block-table entries of 64 consecutive key tiles, one per lane: the loop
// takes a tile's code width and pool offsets with v_readlane instead of a
// scalar load whose latency would stall every tile.
struct MetaWin {
    int base;                              // first tile of the window
    int bits;                              // lane i: width of tile base+i (0: bf16 rows)
    uint32_t klo, khi, vlo, vhi;           // lane i: K / V pool offsets of that tile
};

__device__ __forceinline__ void meta_fetch(MetaWin &mw, const ChunkArgs &p, int a, int base, int nb)
{
    const int kt = base + (threadIdx.x & 63);
    mw.base = base;
    mw.bits = 0;
    mw.klo = mw.khi = mw.vlo = mw.vhi = 0;
    if (kt < nb) {
        const size_t e = (size_t)a * p.t.max_blocks + kt;
        mw.bits = p.t.bits[e];
        const uint64_t ko = p.k.offset[e], vo = p.v.offset[e];
        mw.klo = (uint32_t)ko;
        mw.khi = (uint32_t)(ko >> 32);
        mw.vlo = (uint32_t)vo;
        mw.vhi = (uint32_t)(vo >> 32);
    }
}

// Raw registers of key tile kt: codes and metadata of a quantized block, or
// bf16 rows of window / new tokens.  All fields are assigned once after the
// branches, so the record stays in registers.
template <int NG>
__device__ __forceinline__ void load_raw(TileRaw<NG> &r, MetaWin &mw, const ChunkArgs &p, int a, int g, int kt,
                                         int nb, int nw, int T)
{
    using C = Cfg<NG>;
    constexpr int W = TileRaw<NG>::W;
    const int tid = threadIdx.x, key = tid & 63, qq = tid >> 6;
    const int t = kt * TILE + key;
    uint32_t k[W], v[W], km = 0, vm = 0;
#pragma unroll
    for (int i = 0; i < W; i++) k[i] = v[i] = 0;
    int bits = 0, r0 = 0;
    if (kt < nb) {
        if (kt - mw.base >= 64) meta_fetch(mw, p, a, kt, nb);   // tiles are visited in order
        const int i = kt - mw.base;
        bits = __builtin_amdgcn_readlane(mw.bits, i);
        const uint64_t ko = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(mw.khi, i) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane(mw.klo, i);
        const uint64_t vo = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(mw.vhi, i) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane(mw.vlo, i);
        // byte offsets inside a block fit 32 bits: uniform base + lane offset
        const uint32_t code_row = (uint32_t)(C::D / 8) * bits;
        const uint32_t row = (uint32_t)g * 64 + key;
        const uint8_t *kb = p.k.pool + ko;
        const uint8_t *vb = p.v.pool + vo;
        const uint32_t moff = (uint32_t)p.t.H * 64 * code_row + 4 * (row * NG + (qq * C::D / C::WV) / 64);
        km = *reinterpret_cast<const uint32_t *>(kb + moff);
        vm = *reinterpret_cast<const uint32_t *>(vb + moff);
        const uint8_t *kr = kb + row * code_row, *vr = vb + row * code_row;
        const int off = qq * C::CPT * bits;
        switch (bits) {
        case 2: load_codes<NG, 2>(k, v, r0, kr, vr, off); break;
        case 3: load_codes<NG, 3>(k, v, r0, kr, vr, off); break;
        case 4: load_codes<NG, 4>(k, v, r0, kr, vr, off); break;
        default: load_codes<NG, 8>(k, v, r0, kr, vr, off); break;
        }
    } else {
        // bf16 rows: window tokens, then new tokens; rows past the end read
        // the last row (they are masked).
        const int tt = min(t, T + p.n_new - 1) - 64 * nb;
        const uint16_t *ks, *vs;
        if (tt < nw) {
            ks = p.k.window + (((size_t)a * p.t.window_cap + tt) * p.t.H + g) * C::D;
            vs = p.v.window + (((size_t)a * p.t.window_cap + tt) * p.t.H + g) * C::D;
        } else {
            ks = p.k_new + (((size_t)a * p.n_new + (tt - nw)) * p.t.H + g) * C::D;
            vs = p.v_new + (((size_t)a * p.n_new + (tt - nw)) * p.t.H + g) * C::D;
        }
        const uint4 *k4 = reinterpret_cast<const uint4 *>(ks + qq * C::D / C::WV);
        const uint4 *v4 = reinterpret_cast<const uint4 *>(vs + qq * C::D / C::WV);
#pragma unroll
        for (int i = 0; i < W / 4; i++) {
            const uint4 x = k4[i], y = v4[i];
            k[4 * i] = x.x; k[4 * i + 1] = x.y; k[4 * i + 2] = x.z; k[4 * i + 3] = x.w;
            v[4 * i] = y.x; v[4 * i + 1] = y.y; v[4 * i + 2] = y.z; v[4 * i + 3] = y.w;
        }
    }
#pragma unroll
    for (int i = 0; i < W; i++) {
        r.k[i] = k[i];
        r.v[i] = v[i];
    }
    r.km = km;
    r.vm = vm;
    r.bits = bits;
    r.r0 = r0;
}

// Chunk c (8 dims) of this lane's share as dequantized fp16 pairs.
template <int NG, int B>
__device__ __forceinline__ Pairs raw_chunk(const uint32_t *w, uint32_t meta, int c, int r0)
{
    constexpr int NB = Cfg<NG>::CPT * B;
    Pairs pr;
    if constexpr (B == 4 && NB % 4 == 0) {
        pr = Unpack<4>::run(w[c]);
    } else if constexpr (B == 2) {
        if constexpr (NB % 4 == 0) {
            const uint32_t d = w[c >> 1];
            pr = Unpack<2>::run((c & 1) ? (d >> 16) : (d & 0xffffu));
        } else {                                          // one 16-bit chunk at byte r0 (0 or 2)
            pr = Unpack<2>::run((w[0] >> (8 * r0)) & 0xffffu);
        }
    } else if constexpr (B == 8) {
        pr = Unpack<8>::run2(w[2 * c], w[2 * c + 1]);
    } else if constexpr (B == 3) {
        if constexpr (NB % 4 == 0) {                      // dword-aligned share
            constexpr int NDW = NB / 4;
            const int o = 3 * c, i = o >> 2;              // compile-time after unrolling
            pr = Unpack<3>::run3(w[i], w[(i + 1 < NDW) ? i + 1 : i], o & 3);
        } else {                                          // 3 or 6 bytes at byte r0 of w[0..1]
            const int o = r0 + 3 * c;                     // <= 6, and o + 2 <= 7
            // shift instead of selecting between two array elements, which
            // would index the array at run time and move it to scratch
            const uint64_t d = ((uint64_t)w[1] << 32) | w[0];
            pr = Unpack<3>::run3((uint32_t)(d >> (8 * (o & 4))), w[1], o & 3);
        }
    } else {
        const uint4 v = {w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
        return bf16_pairs(v);
    }
    dequant(pr, meta);
    return pr;
}

template <int NG, int B>
__device__ __forceinline__ void store_tile_w(const TileRaw<NG> &r, _Float16 *ks, _Float16 *vs)
{
    using C = Cfg<NG>;
    const int tid = threadIdx.x, key = tid & 63, qq = tid >> 6;
    const int vp = vpos(key);
#pragma unroll
    for (int c = 0; c < C::CPT; c++) {
        const int d0 = (qq * C::CPT + c) * 8;
        const Pairs pk = raw_chunk<NG, B>(r.k, r.km, c, r.r0);
        h8 o;
        o[0] = pk.p[0][0]; o[1] = pk.p[0][1]; o[2] = pk.p[1][0]; o[3] = pk.p[1][1];
        o[4] = pk.p[2][0]; o[5] = pk.p[2][1]; o[6] = pk.p[3][0]; o[7] = pk.p[3][1];
        *reinterpret_cast<h8 *>(ks + key * C::KROW + d0) = o;
        const Pairs pv = raw_chunk<NG, B>(r.v, r.vm, c, r.r0);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            vs[(d0 + i) * C::VROW + vp] = pv.p[i][0];
            vs[(d0 + i + 4) * C::VROW + vp] = pv.p[i][1];
        }
    }
}

template <int NG>
__device__ __forceinline__ void store_tile(const TileRaw<NG> &r, _Float16 *ks, _Float16 *vs)
{
    switch (r.bits) {
    case 2: store_tile_w<NG, 2>(r, ks, vs); break;
    case 3: store_tile_w<NG, 3>(r, ks, vs); break;
    case 4: store_tile_w<NG, 4>(r, ks, vs); break;
    case 8: store_tile_w<NG, 8>(r, ks, vs); break;
    default: store_tile_w<NG, 0>(r, ks, vs); break;
    }
}

typedef float f16x __attribute__((ext_vector_type(16)));

// Per-wave state of the key loop: lane l owns query row l%32; lane half
// hh = l/32 selects which 8 of every 16 K positions it supplies.
template <int NG>
struct Rows {
    using C = Cfg<NG>;
    h8 qop[C::KS];                         // B operand of S^T = K.Q^T: chunk 2ks+hh of the row
    f16x acc[C::DT];                       // O^T tiles: dims 32dt + 8(r/4) + 4hh + r%4
    float m_run, l_run;
    int lim;                               // keys this row attends to
    int lim_min;                           // smallest limit over the wave
};

// One 64-key tile: S^T from the current LDS buffers, the next tile's
// dequantize into the other buffers (same basic block, so the scheduler can
// interleave its vector work with the matrix instructions), then softmax and
// O^T += V^T.P^T.
template <int NG>
__device__ __forceinline__ void tile_step(Rows<NG> &w, const _Float16 *kc, const _Float16 *vc,
                                          _Float16 *kn, _Float16 *vn, TileRaw<NG> &raw, MetaWin &mw, bool store_next,
                                          bool load_next, const ChunkArgs &p, int a, int g, int kt,
                                          int nb, int nw, int T)
{
    using C = Cfg<NG>;
    const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
    const int t0 = kt * TILE;
    f16x st[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
#pragma unroll
        for (int e = 0; e < 16; e++) st[mt][e] = 0.0f;
#pragma unroll
        for (int k = 0; k < C::KS; k++) {
            const h8 av = *reinterpret_cast<const h8 *>(kc + (32 * mt + m) * C::KROW + 16 * k + 8 * hh);
            st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, w.qop[k], st[mt], 0, 0, 0);
        }
    }
    if (store_next) {
        store_tile<NG>(raw, kn, vn);
        if (load_next) load_raw<NG>(raw, mw, p, a, g, kt + 2, nb, nw, T);
    }

    // Online softmax of the lane's row: keys 32mt + 8(r/4) + 4hh + r%4.
    // Scores are scaled inside the exp2 argument: c > 0, so the row max of
    // c*s is c times the max of s.
    if (t0 + TILE > w.lim_min) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (t0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3) >= w.lim) st[mt][r] = -INFINITY;
    }
    float mx = st[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int r = (mt == 0 ? 1 : 0); r < 16; r++) mx = fmaxf(mx, st[mt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy running max: keep the current reference unless the tile's max
    // exceeds it by more than LAZY (log2 units); probabilities then stay
    // below 2^LAZY (fine for fp16) and most tiles skip the O rescale.
    const float tmax = mx * p.c;
    const float m_new = (tmax > w.m_run + LAZY) ? tmax : w.m_run;
    // rows with no valid key yet keep m = -inf; use 0 to avoid inf-inf
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_use);
    w.m_run = m_new;
    float lsum = 0.0f;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    h8 pb[4];                                  // B operand of K-step u: regs 8(u%2)..+7 of tile u/2
#pragma unroll
    for (int u = 0; u < 4; u++) {
        h8 o;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int r = 8 * (u & 1) + e;
            const h2 pa = __builtin_convertvector(
                f2{__builtin_amdgcn_exp2f(__builtin_fmaf(st[u >> 1][r], p.c, -m_use)),
                   __builtin_amdgcn_exp2f(__builtin_fmaf(st[u >> 1][r + 1], p.c, -m_use))}, h2);
            o[e] = pa[0];
            o[e + 1] = pa[1];
            lsum = __builtin_amdgcn_fdot2(pa, ones, lsum, false);
        }
        pb[u] = o;
    }
    w.l_run = w.l_run * alpha + lsum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++) w.acc[dt] *= alpha;
    }
    // O^T += V^T . P^T over the 64 keys (4 K-steps of 16).
#pragma unroll
    for (int u = 0; u < 4; u++) {
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++) {
            const h8 av = *reinterpret_cast<const h8 *>(vc + (32 * dt + m) * C::VROW + 16 * u + 8 * hh);
            w.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[u], w.acc[dt], 0, 0, 0);
        }
    }
    __syncthreads();                     // next buffers written, current ones no longer read
}

template <int NG>
__global__ __launch_bounds__(64 * Cfg<NG>::WV, 1) void chunk_split(ChunkArgs p)
{
    using C = Cfg<NG>;
    __shared__ __attribute__((aligned(16))) _Float16 ks0[TILE * C::KROW];
    __shared__ __attribute__((aligned(16))) _Float16 vs0[C::D * C::VROW];
    __shared__ __attribute__((aligned(16))) _Float16 ks1[TILE * C::KROW];
    __shared__ __attribute__((aligned(16))) _Float16 vs1[C::D * C::VROW];

    const int s = blockIdx.x, a = blockIdx.z;
    const int g = blockIdx.y / p.n_row_tiles, rt = blockIdx.y % p.n_row_tiles;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int T = 64 * nb + nw;                          // restored tokens

    // Rows of the workgroup: R = rt*ROWS + r, token R / G, head g*G + R % G.
    const int row0 = rt * C::ROWS;
    const int i_last = min(p.n_new - 1, (row0 + C::ROWS - 1) / p.G);
    const int lim_wg = T + i_last + 1;                   // keys any row of the workgroup sees
    const int n_tiles = (lim_wg + TILE - 1) / TILE;
    const int kt0 = s * p.split_tiles;
    const int kt1 = min(kt0 + p.split_tiles, n_tiles);
    if (kt0 >= kt1) return;

    // The wave's query row (lane l: row l%32) and its key limit.
    const int m = lane & 31, hh = lane >> 5;
    Rows<NG> w;
    const int R = row0 + wave * C::NR + m;
    const int ti = R / p.G, head = g * p.G + R % p.G;
    const bool rv = ti < p.n_new;
    w.lim = rv ? T + ti + 1 : 0;
    {
        const uint16_t *qr = p.q_new + (((size_t)a * p.n_new + (rv ? ti : 0)) * p.Hq + head) * C::D;
#pragma unroll
        for (int k = 0; k < C::KS; k++) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qr + 8 * (2 * k + hh));
            const Pairs pr = bf16_pairs(v);
            h8 o;
            o[0] = pr.p[0][0]; o[1] = pr.p[0][1]; o[2] = pr.p[1][0]; o[3] = pr.p[1][1];
            o[4] = pr.p[2][0]; o[5] = pr.p[2][1]; o[6] = pr.p[3][0]; o[7] = pr.p[3][1];
            if (!rv) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
            w.qop[k] = o;
        }
    }
    int lim_min = rv ? w.lim : (1 << 30);
    for (int o = 1; o < 64; o <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, o));
    w.lim_min = lim_min;
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++)
#pragma unroll
        for (int e = 0; e < 16; e++) w.acc[dt][e] = 0.0f;
    w.m_run = -INFINITY;
    w.l_run = 0.0f;

    TileRaw<NG> raw;
    MetaWin mw;
    mw.base = -(1 << 20);
    load_raw<NG>(raw, mw, p, a, g, kt0, nb, nw, T);
    store_tile<NG>(raw, ks0, vs0);
    if (kt0 + 1 < kt1) load_raw<NG>(raw, mw, p, a, g, kt0 + 1, nb, nw, T);
    __syncthreads();
    for (int kt = kt0; kt < kt1; kt += 2) {
        tile_step<NG>(w, ks0, vs0, ks1, vs1, raw, mw, kt + 1 < kt1, kt + 2 < kt1, p, a, g, kt, nb, nw, T);
        if (kt + 1 < kt1)
            tile_step<NG>(w, ks1, vs1, ks0, vs0, raw, mw, kt + 2 < kt1, kt + 3 < kt1, p, a, g, kt + 1, nb, nw, T);
    }

    // Partial of the lane's row if it has a key in this split.
    const size_t stride = (size_t)(C::D + 2);
    float l = w.l_run + __shfl_xor(w.l_run, 32);
    if (rv && kt0 * TILE < w.lim) {
        const size_t orow = ((size_t)a * p.n_new + ti) * p.Hq + head;
        float *pr = p.part + (orow * p.n_splits + s) * stride;
        if (hh == 0) { pr[0] = w.m_run; pr[1] = l; }
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++)
#pragma unroll
            for (int r = 0; r < 16; r++) pr[2 + 32 * dt + 8 * (r >> 2) + 4 * hh + (r & 3)] = w.acc[dt][r];
    }
}

// ---- staggered key loop (head_dim 64 and 128) -------------------------------
//
// Eight waves, two per SIMD (waves w and w+4 share one).  Per tile each wave
// runs S^T (matrix), softmax (vector), P.V (matrix) and the dequantize of
// tile t+2 (vector); group A (waves 0-3) in that order, group B (waves 4-7)
// with the dequantize first, so each SIMD mostly pairs one wave's matrix
// work with the other's vector work.  Three LDS tile buffers and one barrier
// per tile: between barriers t-1 and t, tile t is read from buffer t%3 and
// tile t+2 written into buffer (t+2)%3, whose tile t-1 was last read before
// barrier t-1.

__device__ __forceinline__ float xhalf_max(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Instruction order for a block of N operand reads from LDS each feeding one
// matrix instruction: PF reads ahead, so LDS latency hides behind the
// matrix instructions instead of stalling each of them.
template <int N>
__device__ __forceinline__ void mfma_prefetch_order()
{
    constexpr int PF = N < 6 ? N : 6;
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int i = 0; i < N; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + PF < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}

// v_max3_f32 without the operand canonicalization fmaxf carries (scores are
// never NaN): two independent chains over the 32 scores of a lane.
__device__ __forceinline__ float max3(float a, float b, float c)
{
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

__device__ __forceinline__ float tile_max(const f16x (&st)[2])
{
    float m0 = max3(st[0][0], st[0][1], st[0][2]);
    float m1 = max3(st[1][0], st[1][1], st[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
        m0 = max3(m0, st[0][r], st[0][r + 1]);
        m1 = max3(m1, st[1][r], st[1][r + 1]);
    }
    return max3(m0, m1, max3(st[0][15], st[1][15], m0));
}

// S^T of one tile (K-step outer: consecutive instructions are independent).
template <int NG>
__device__ __forceinline__ void s_phase(const Rows<NG> &w, const _Float16 *kc, f16x (&st)[2])
{
    using C = Cfg<NG>;
    const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int e = 0; e < 16; e++) st[mt][e] = 0.0f;
#pragma unroll
    for (int k = 0; k < C::KS; k++)
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            const h8 av = *reinterpret_cast<const h8 *>(kc + (32 * mt + m) * C::KROW + 16 * k + 8 * hh);
            st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, w.qop[k], st[mt], 0, 0, 0);
        }
    mfma_prefetch_order<2 * C::KS>();
}

// Online softmax of the lane's row over one tile's scores (keys
// 32mt + 8(r/4) + 4hh + r%4), O^T rescale included.  Scores are scaled
// inside the exp2 argument (c > 0).
template <int NG, bool MASK>
__device__ __forceinline__ void softmax_phase(Rows<NG> &w, f16x (&st)[2], h8 (&pb)[4], int t0, float c)
{
    using C = Cfg<NG>;
    const int hh = (threadIdx.x & 63) >> 5;
    if (MASK) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (t0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3) >= w.lim) st[mt][r] = -INFINITY;
    }
    float mx = tile_max(st);
    mx = xhalf_max(mx);
    // Lazy running max: the reference moves only when the tile's max exceeds
    // it by more than LAZY (log2 units), so probabilities stay below 2^LAZY
    // (safe in fp16) and most tiles need no O^T rescale.
    const float m_old = w.m_run;
    const float tmax = mx * c;
    const float m_new = (tmax > m_old + LAZY) ? tmax : m_old;
    // no valid key yet: m stays -inf, probabilities are exp2(-inf) = 0
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_old - m_new);
    w.m_run = m_new;
    float lsum = 0.0f;
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int u = 0; u < 4; u++) {
        h8 o;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int r = 8 * (u & 1) + e;
            const h2 pa = __builtin_convertvector(
                f2{__builtin_amdgcn_exp2f(__builtin_fmaf(st[u >> 1][r], c, -m_use)),
                   __builtin_amdgcn_exp2f(__builtin_fmaf(st[u >> 1][r + 1], c, -m_use))}, h2);
            o[e] = pa[0];
            o[e + 1] = pa[1];
            lsum = __builtin_amdgcn_fdot2(pa, ones, lsum, false);
        }
        pb[u] = o;
    }
    w.l_run = w.l_run * alpha + lsum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++) w.acc[dt] *= alpha;
    }
}

template <int NG>
__device__ __forceinline__ void pv_phase(Rows<NG> &w, const _Float16 *vc, const h8 (&pb)[4])
{
    using C = Cfg<NG>;
    const int lane = threadIdx.x & 63, m = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++) {
            const h8 av = *reinterpret_cast<const h8 *>(vc + (32 * dt + m) * C::VROW + 16 * u + 8 * hh);
            w.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[u], w.acc[dt], 0, 0, 0);
        }
    mfma_prefetch_order<4 * C::DT>();
}

template <int NG>
__global__ __launch_bounds__(512, 1) void chunk_split_pp(ChunkArgs p)
{
    using C = Cfg<NG>;
    static_assert(C::WV == 8, "ping-pong needs two waves per SIMD");
    constexpr int KT = TILE * C::KROW, BUF = KT + C::D * C::VROW;
    __shared__ __attribute__((aligned(16))) _Float16 lds[3 * BUF];

    const int s = blockIdx.x, a = blockIdx.z;
    const int g = blockIdx.y / p.n_row_tiles, rt = blockIdx.y % p.n_row_tiles;
    // the wave index is uniform per wave; readfirstlane lets the compiler know
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int T = 64 * nb + nw;

    const int row0 = rt * C::ROWS;
    const int i_last = min(p.n_new - 1, (row0 + C::ROWS - 1) / p.G);
    const int lim_wg = T + i_last + 1;
    const int n_tiles = (lim_wg + TILE - 1) / TILE;
    const int kt0 = s * p.split_tiles;
    const int kt1 = min(kt0 + p.split_tiles, n_tiles);
    if (kt0 >= kt1) return;
    const int n = kt1 - kt0;

    const int m = lane & 31, hh = lane >> 5;
    Rows<NG> w;
    const int R = row0 + wave * C::NR + m;
    const int ti = R / p.G, head = g * p.G + R % p.G;
    const bool rv = ti < p.n_new;
    w.lim = rv ? T + ti + 1 : 0;
    {
        const uint16_t *qr = p.q_new + (((size_t)a * p.n_new + (rv ? ti : 0)) * p.Hq + head) * C::D;
#pragma unroll
        for (int k = 0; k < C::KS; k++) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qr + 8 * (2 * k + hh));
            const Pairs pr = bf16_pairs(v);
            h8 o;
            o[0] = pr.p[0][0]; o[1] = pr.p[0][1]; o[2] = pr.p[1][0]; o[3] = pr.p[1][1];
            o[4] = pr.p[2][0]; o[5] = pr.p[2][1]; o[6] = pr.p[3][0]; o[7] = pr.p[3][1];
            if (!rv) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
            w.qop[k] = o;
        }
    }
    int lim_min = rv ? w.lim : (1 << 30);
    for (int o = 1; o < 64; o <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, o));
    w.lim_min = lim_min;
#pragma unroll
    for (int dt = 0; dt < C::DT; dt++)
#pragma unroll
        for (int e = 0; e < 16; e++) w.acc[dt][e] = 0.0f;
    w.m_run = -INFINITY;
    w.l_run = 0.0f;

    // Prologue: tiles 0 and 1 in buffers 0 and 1, codes of tile 2 in registers.
    TileRaw<NG> raw;
    MetaWin mw;
    mw.base = -(1 << 20);
    load_raw<NG>(raw, mw, p, a, g, kt0, nb, nw, T);
    store_tile<NG>(raw, lds, lds + KT);
    if (n > 1) {
        load_raw<NG>(raw, mw, p, a, g, kt0 + 1, nb, nw, T);
        store_tile<NG>(raw, lds + BUF, lds + BUF + KT);
        if (n > 2) load_raw<NG>(raw, mw, p, a, g, kt0 + 2, nb, nw, T);
    }
    __syncthreads();
    // Group B dequantizes first, so that on each SIMD one wave's matrix
    // phase meets the other wave's vector phase.
    const bool late = wave >= 4;
    int cb = 0;
    for (int j = 0; j < n; j++) {
        _Float16 *bc = lds + cb * BUF;
        _Float16 *bf = lds + (cb == 0 ? 2 : cb - 1) * BUF;   // buffer of tile j + 2
        const int t0 = (kt0 + j) * TILE;
        if (late && j + 2 < n) {
            store_tile<NG>(raw, bf, bf + KT);
            if (j + 3 < n) load_raw<NG>(raw, mw, p, a, g, kt0 + j + 3, nb, nw, T);
        }
        f16x st[2];
        h8 pb[4];
        s_phase<NG>(w, bc, st);
        if (t0 + TILE > w.lim_min) softmax_phase<NG, true>(w, st, pb, t0, p.c);
        else softmax_phase<NG, false>(w, st, pb, t0, p.c);
        pv_phase<NG>(w, bc + KT, pb);
        if (!late && j + 2 < n) {
            store_tile<NG>(raw, bf, bf + KT);
            if (j + 3 < n) load_raw<NG>(raw, mw, p, a, g, kt0 + j + 3, nb, nw, T);
        }
        __syncthreads();
        cb = cb == 2 ? 0 : cb + 1;
    }

    const size_t stride = (size_t)(C::D + 2);
    const float l = xhalf_sum(w.l_run);
    if (rv && kt0 * TILE < w.lim) {
        const size_t orow = ((size_t)a * p.n_new + ti) * p.Hq + head;
        float *pr = p.part + (orow * p.n_splits + s) * stride;
        if (hh == 0) { pr[0] = w.m_run; pr[1] = l; }
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++)
#pragma unroll
            for (int r = 0; r < 16; r++) pr[2 + 32 * dt + 8 * (r >> 2) + 4 * hh + (r & 3)] = w.acc[dt][r];
    }
}

// One wave per output row: combine the splits that saw its keys.
__global__ __launch_bounds__(256) void chunk_merge(ChunkArgs p)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t row = (size_t)blockIdx.x * 4 + wave;
    const size_t rows = (size_t)p.t.A * p.n_new * p.Hq;
    if (row >= rows) return;
    const int i = (int)((row / p.Hq) % p.n_new);
    const int a = (int)(row / ((size_t)p.Hq * p.n_new));
    const int D = p.t.D;
    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int lim = 64 * nb + nw + i + 1;
    const int ns = (lim + TILE * p.split_tiles - 1) / (TILE * p.split_tiles);
    const size_t stride = (size_t)(D + 2);
    const float *pr = p.part + row * p.n_splits * stride;
    if (ns <= 8) {
        // Up to 8 splits: every split's (max, sum) (lane s) and the lane's
        // dims of every split are loaded before the first use, so the row
        // costs one memory round trip.
        float mv = -INFINITY, lv = 0.0f;
        if (lane < ns) {
            mv = pr[lane * stride];
            lv = pr[lane * stride + 1];
        }
        float v[8][4];
#pragma unroll
        for (int s = 0; s < 8; s++)
#pragma unroll
            for (int k = 0; k < 4; k++)
                v[s][k] = (s < ns && 64 * k + lane < D) ? pr[s * stride + 2 + 64 * k + lane] : 0.0f;
        float M = mv;
#pragma unroll
        for (int x = 32; x > 0; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
        const float wgt = (lane < ns && M > -INFINITY) ? __builtin_amdgcn_exp2f(mv - M) : 0.0f;
        float L = wgt * lv;
#pragma unroll
        for (int x = 32; x > 0; x >>= 1) L += __shfl_xor(L, x);
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 8; s++) {
            if (s < ns) {
                const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wgt), s));
#pragma unroll
                for (int k = 0; k < 4; k++) acc[k] = __builtin_fmaf(ws, v[s][k], acc[k]);
            }
        }
        float *o = p.out + row * D;
#pragma unroll
        for (int k = 0; k < 4; k++)
            if (64 * k + lane < D) o[64 * k + lane] = acc[k] * inv;
        return;
    }
    float M = -INFINITY;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, pr[s * stride]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.0f;
    for (int s = lane; s < ns; s += 64) L += __builtin_amdgcn_exp2f(pr[s * stride] - M) * pr[s * stride + 1];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float *o = p.out + row * D;
    for (int d = lane; d < D; d += 64) {
        float acc = 0.0f;
        for (int s = 0; s < ns; s++) acc += __builtin_amdgcn_exp2f(pr[s * stride] - M) * pr[s * stride + 2 + d];
        o[d] = acc * inv;
    }
}

}  // namespace

bool chunk_supported(int D) { return D == 64 || D == 128 || D == 256; }

int chunk_rows_per_wg(int D) { return D == 256 ? Cfg<4>::ROWS : Cfg<2>::ROWS; }

hipError_t launch_chunk(const ChunkArgs &p, hipStream_t s)
{
    dim3 grid(p.n_splits, p.t.H * p.n_row_tiles, p.t.A);
    switch (p.t.D) {
    case 64: chunk_split_pp<1><<<grid, 64 * Cfg<1>::WV, 0, s>>>(p); break;
    case 128: chunk_split_pp<2><<<grid, 64 * Cfg<2>::WV, 0, s>>>(p); break;
    case 256: chunk_split<4><<<grid, 64 * Cfg<4>::WV, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t rows = (size_t)p.t.A * p.n_new * p.Hq;
    chunk_merge<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace kvq
