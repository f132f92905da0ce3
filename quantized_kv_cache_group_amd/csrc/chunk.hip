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
// Work decomposition: a workgroup is 4 waves x ROWS query rows of one KV
// head; a query row is a (new token, query head) pair, token-major.  Keys
// are walked in tiles of 64 (one quantized block), split across SPLITS
// workgroups whose partials the merge kernel combines.  Per tile:
//   1. all 256 lanes dequantize the tile into LDS: K as fp16 rows (dims in
//      the chunk order the unpack produces), V transposed (V^T[d][key]) with
//      keys permuted so a lane's 8 probabilities line up with 8 consecutive
//      LDS halves; the raw codes of the next tile are already in registers;
//   2. each wave computes S^T = K.Q^T with v_mfma_f32_16x16x32_f16 (A = 16
//      keys x 32 dims from LDS, B = the wave's query rows from registers),
//      so a lane owns one query row and 4 keys per 16-key tile;
//   3. online softmax per row in fp32 (exp2), probabilities rounded to fp16
//      (the running sum adds the rounded values);
//   4. O^T += V^T.P^T (A = 16 dims x 32 keys from LDS, B = P^T from the
//      lane's own registers).
// The causal mask only applies to tiles that reach the new tokens.
#include "kvq_internal.h"
#include "unpack.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int TILE = 64;          // keys per tile
constexpr int WAVES = 4;

template <int NG>
struct Cfg {
    static constexpr int D = 64 * NG;
    static constexpr int NR = (NG >= 4) ? 16 : 32;       // query rows per wave
    static constexpr int NTN = NR / 16;                   // 16-row column tiles per wave
    static constexpr int ROWS = WAVES * NR;               // rows per workgroup
    static constexpr int KS = D / 32;                     // K-steps of Q.K^T
    static constexpr int DT = D / 16;                     // 16-dim output tiles
    static constexpr int KROW = D + 8;                    // LDS K row stride (halves)
    static constexpr int VROW = TILE + 8;                 // LDS V^T row stride (halves)
    static constexpr int CPT = D / 32;                    // chunks of 8 dims per dequant lane
};

// Position of key k (0..63) of a tile in the V^T rows: within each 32-key
// half, lane quarter q of the P^T operand holds keys 4q..4q+3 (first
// 16-key tile) and 16+4q..16+4q+3 (second), as 8 consecutive positions.
__device__ __forceinline__ int vpos(int k)
{
    const int h32 = k & ~31, kk = k & 31;
    return h32 + 8 * ((kk & 15) >> 2) + 4 * (kk >> 4) + (kk & 3);
}

// Raw registers of one dequant lane's share of a tile: key = lane (0..63),
// dims [w*D/4, (w+1)*D/4) for wave w, so one LDS write instruction of a wave
// covers 64 keys of one V^T row (no bank conflicts).  Sized for bf16 rows (D/2 bytes), which
// also covers every code width.
template <int NG>
struct TileRaw {
    static constexpr int W = 8 * NG;                      // dwords
    uint32_t k[W], v[W];
    uint32_t km, vm;
    int bits;                                             // 0: bf16 rows, else code width
    int r0;                                               // byte offset of chunk 0 in k/v
};

// Load CPT*B code bytes of a row share: dwords covering [off, off+CPT*B).
template <int NG, int B>
__device__ __forceinline__ void load_codes(TileRaw<NG> &r, const uint8_t *krow, const uint8_t *vrow, int off)
{
    constexpr int NB = Cfg<NG>::CPT * B;                 // bytes
    if constexpr (NB % 4 == 0) {
        constexpr int NDW = NB / 4;
        if constexpr (NB % 16 == 0) {
#pragma unroll
            for (int i = 0; i < NDW / 4; i++) {
                const uint4 x = reinterpret_cast<const uint4 *>(krow + off)[i];
                const uint4 y = reinterpret_cast<const uint4 *>(vrow + off)[i];
                r.k[4 * i] = x.x; r.k[4 * i + 1] = x.y; r.k[4 * i + 2] = x.z; r.k[4 * i + 3] = x.w;
                r.v[4 * i] = y.x; r.v[4 * i + 1] = y.y; r.v[4 * i + 2] = y.z; r.v[4 * i + 3] = y.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NDW; i++) {
                r.k[i] = reinterpret_cast<const uint32_t *>(krow + off)[i];
                r.v[i] = reinterpret_cast<const uint32_t *>(vrow + off)[i];
            }
        }
        r.r0 = 0;
    } else {
        // 3-bit codes at head_dim 64: 6 bytes at a 2-byte aligned offset
        const int base = off & ~3;
        r.k[0] = reinterpret_cast<const uint32_t *>(krow + base)[0];
        r.k[1] = reinterpret_cast<const uint32_t *>(krow + base)[1];
        r.v[0] = reinterpret_cast<const uint32_t *>(vrow + base)[0];
        r.v[1] = reinterpret_cast<const uint32_t *>(vrow + base)[1];
        r.r0 = off & 3;
    }
}

template <int NG>
__device__ __forceinline__ void load_raw(TileRaw<NG> &r, const ChunkArgs &p, int a, int g, int kt,
                                         int nb, int nw, int T)
{
    using C = Cfg<NG>;
    const int tid = threadIdx.x, key = tid & 63, qq = tid >> 6;
    const int t = kt * TILE + key;
    if (kt < nb) {
        const size_t e = (size_t)a * p.t.max_blocks + kt;
        const int b = p.t.bits[e];
        r.bits = b;
        const size_t code_row = (size_t)C::D * b / 8;
        const size_t row = (size_t)g * 64 + key;
        const uint8_t *kb = p.k.pool + p.k.offset[e];
        const uint8_t *vb = p.v.pool + p.v.offset[e];
        const size_t meta0 = (size_t)p.t.H * 64 * code_row;
        const int grp = (qq * C::D / 4) / 64;
        r.km = reinterpret_cast<const uint32_t *>(kb + meta0)[row * NG + grp];
        r.vm = reinterpret_cast<const uint32_t *>(vb + meta0)[row * NG + grp];
        const uint8_t *kr = kb + row * code_row, *vr = vb + row * code_row;
        const int off = qq * C::CPT * b;
        switch (b) {
        case 2: load_codes<NG, 2>(r, kr, vr, off); break;
        case 3: load_codes<NG, 3>(r, kr, vr, off); break;
        case 4: load_codes<NG, 4>(r, kr, vr, off); break;
        default: load_codes<NG, 8>(r, kr, vr, off); break;
        }
    } else {
        // bf16 rows: window tokens, then new tokens; rows past the end read
        // the last row (they are masked).
        r.bits = 0;
        r.r0 = 0;
        const int tt = min(t, T + p.n_new - 1) - 64 * nb;
        const uint16_t *ks, *vs;
        if (tt < nw) {
            ks = p.k.window + (((size_t)a * p.t.window_cap + tt) * p.t.H + g) * C::D;
            vs = p.v.window + (((size_t)a * p.t.window_cap + tt) * p.t.H + g) * C::D;
        } else {
            ks = p.k_new + (((size_t)a * p.n_new + (tt - nw)) * p.t.H + g) * C::D;
            vs = p.v_new + (((size_t)a * p.n_new + (tt - nw)) * p.t.H + g) * C::D;
        }
        const uint4 *k4 = reinterpret_cast<const uint4 *>(ks + qq * C::D / 4);
        const uint4 *v4 = reinterpret_cast<const uint4 *>(vs + qq * C::D / 4);
#pragma unroll
        for (int i = 0; i < TileRaw<NG>::W / 4; i++) {
            const uint4 x = k4[i], y = v4[i];
            r.k[4 * i] = x.x; r.k[4 * i + 1] = x.y; r.k[4 * i + 2] = x.z; r.k[4 * i + 3] = x.w;
            r.v[4 * i] = y.x; r.v[4 * i + 1] = y.y; r.v[4 * i + 2] = y.z; r.v[4 * i + 3] = y.w;
        }
        r.km = r.vm = 0;
    }
}

// Chunk c (8 dims) of this lane's share as dequantized fp16 pairs.
template <int NG, int B>
__device__ __forceinline__ Pairs raw_chunk(const uint32_t *w, uint32_t meta, int c, int r0)
{
    Pairs pr;
    if constexpr (B == 4) {
        pr = Unpack<4>::run(w[c]);
    } else if constexpr (B == 2) {
        const uint32_t d = w[c >> 1];
        pr = Unpack<2>::run((c & 1) ? (d >> 16) : (d & 0xffffu));
    } else if constexpr (B == 8) {
        pr = Unpack<8>::run2(w[2 * c], w[2 * c + 1]);
    } else if constexpr (B == 3) {
        constexpr int NB = Cfg<NG>::CPT * 3;
        if constexpr (NB % 4 == 0) {                      // dword-aligned share
            constexpr int NDW = NB / 4;
            const int o = 3 * c, i = o >> 2;              // compile-time after unrolling
            pr = Unpack<3>::run3(w[i], w[(i + 1 < NDW) ? i + 1 : i], o & 3);
        } else {                                          // 6 bytes at byte r0 of w[0..1]
            const int o = r0 + 3 * c;                     // <= 5
            pr = Unpack<3>::run3(o >= 4 ? w[1] : w[0], w[1], o & 3);
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

template <int NG>
__global__ __launch_bounds__(256, 2) void chunk_split(ChunkArgs p)
{
    using C = Cfg<NG>;
    __shared__ __attribute__((aligned(16))) _Float16 ks[TILE * C::KROW];
    __shared__ __attribute__((aligned(16))) _Float16 vs[C::D * C::VROW];
    __shared__ int lim_max_s;

    const int s = blockIdx.x, a = blockIdx.z;
    const int g = blockIdx.y / p.n_row_tiles, rt = blockIdx.y % p.n_row_tiles;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, q = lane >> 4;
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

    // The wave's query rows and their key limits.
    int lim[C::NTN];
    bool rv[C::NTN];
    h8 qop[C::NTN][C::KS];
#pragma unroll
    for (int nt = 0; nt < C::NTN; nt++) {
        const int R = row0 + wave * C::NR + nt * 16 + n;
        const int i = R / p.G, h = g * p.G + R % p.G;
        rv[nt] = i < p.n_new;
        lim[nt] = rv[nt] ? T + i + 1 : 0;
        const uint16_t *qr = p.q_new + (((size_t)a * p.n_new + (rv[nt] ? i : 0)) * p.Hq + h) * C::D;
#pragma unroll
        for (int k = 0; k < C::KS; k++) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qr + 8 * (4 * k + q));
            const Pairs pr = bf16_pairs(v);
            h8 o;
            o[0] = pr.p[0][0]; o[1] = pr.p[0][1]; o[2] = pr.p[1][0]; o[3] = pr.p[1][1];
            o[4] = pr.p[2][0]; o[5] = pr.p[2][1]; o[6] = pr.p[3][0]; o[7] = pr.p[3][1];
            if (!rv[nt]) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
            qop[nt][k] = o;
        }
    }
    int lim_min = 1 << 30;
#pragma unroll
    for (int nt = 0; nt < C::NTN; nt++) if (rv[nt]) lim_min = min(lim_min, lim[nt]);
    // smallest limit over the wave (for the per-tile mask test)
    for (int o = 1; o < 64; o <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, o));

    f4 acc[C::NTN][C::DT];
#pragma unroll
    for (int nt = 0; nt < C::NTN; nt++)
#pragma unroll
        for (int dt = 0; dt < C::DT; dt++) acc[nt][dt] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run[C::NTN], l_run[C::NTN];
#pragma unroll
    for (int nt = 0; nt < C::NTN; nt++) { m_run[nt] = -INFINITY; l_run[nt] = 0.0f; }

    TileRaw<NG> raw;
    load_raw<NG>(raw, p, a, g, kt0, nb, nw, T);
    for (int kt = kt0; kt < kt1; kt++) {
        __syncthreads();                                 // previous tile's LDS reads are done
        store_tile<NG>(raw, ks, vs);
        if (kt + 1 < kt1) load_raw<NG>(raw, p, a, g, kt + 1, nb, nw, T);
        __syncthreads();

        const int t0 = kt * TILE;
        const bool masked = t0 + TILE > lim_min;
        // S^T tiles: [16 keys][16 rows] for 4 key tiles x NTN row tiles.
        f4 st[4][C::NTN];
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
#pragma unroll
            for (int nt = 0; nt < C::NTN; nt++) st[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < C::KS; k++) {
                const h8 av = *reinterpret_cast<const h8 *>(ks + (16 * mt + n) * C::KROW + 32 * k + 8 * q);
#pragma unroll
                for (int nt = 0; nt < C::NTN; nt++)
                    st[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qop[nt][k], st[mt][nt], 0, 0, 0);
            }
        }
        // Online softmax per row (lane's row n of tile nt; keys 16mt + 4q + j).
        // Scores are scaled inside the exp2 argument: c > 0, so the row max
        // of c*s is c times the max of s.
        h8 pb[C::NTN][2];
#pragma unroll
        for (int nt = 0; nt < C::NTN; nt++) {
            if (masked) {
#pragma unroll
                for (int mt = 0; mt < 4; mt++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        if (t0 + 16 * mt + 4 * q + j >= lim[nt]) st[mt][nt][j] = -INFINITY;
            }
            float mx = fmaxf(fmaxf(st[0][nt][0], st[0][nt][1]), fmaxf(st[0][nt][2], st[0][nt][3]));
#pragma unroll
            for (int mt = 1; mt < 4; mt++)
                mx = fmaxf(mx, fmaxf(fmaxf(st[mt][nt][0], st[mt][nt][1]), fmaxf(st[mt][nt][2], st[mt][nt][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[nt], mx * p.c);
            // rows with no valid key yet keep m = -inf; use 0 to avoid inf-inf
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
            m_run[nt] = m_new;
            float lsum = 0.0f;
            const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int ksx = 0; ksx < 2; ksx++) {
                // K-step ksx: key tiles 2ksx (positions 0..3) and 2ksx+1 (4..7)
                h8 o;
#pragma unroll
                for (int hm = 0; hm < 2; hm++) {
                    const f4 v = st[2 * ksx + hm][nt];
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const h2 pa = __builtin_convertvector(
                            f2{__builtin_amdgcn_exp2f(__builtin_fmaf(v[e], p.c, -m_use)),
                               __builtin_amdgcn_exp2f(__builtin_fmaf(v[e + 1], p.c, -m_use))}, h2);
                        o[4 * hm + e] = pa[0];
                        o[4 * hm + e + 1] = pa[1];
                        lsum = __builtin_amdgcn_fdot2(pa, ones, lsum, false);
                    }
                }
                pb[nt][ksx] = o;
            }
            l_run[nt] = l_run[nt] * alpha + lsum;
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < C::DT; dt++) acc[nt][dt] *= alpha;
            }
        }
        // O^T += V^T . P^T over the 64 keys (2 K-steps of 32).
#pragma unroll
        for (int ksx = 0; ksx < 2; ksx++) {
#pragma unroll
            for (int dt = 0; dt < C::DT; dt++) {
                const h8 av = *reinterpret_cast<const h8 *>(vs + (16 * dt + n) * C::VROW + 32 * ksx + 8 * q);
#pragma unroll
                for (int nt = 0; nt < C::NTN; nt++)
                    acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[nt][ksx], acc[nt][dt], 0, 0, 0);
            }
        }
    }

    // Partials of rows that have a key in this split.
    const size_t stride = (size_t)(C::D + 2);
#pragma unroll
    for (int nt = 0; nt < C::NTN; nt++) {
        float l = l_run[nt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int R = row0 + wave * C::NR + nt * 16 + n;
        const int i = R / p.G, h = g * p.G + R % p.G;
        if (rv[nt] && kt0 * TILE < lim[nt]) {
            const size_t orow = ((size_t)a * p.n_new + i) * p.Hq + h;
            float *pr = p.part + (orow * p.n_splits + s) * stride;
            if (q == 0) { pr[0] = m_run[nt]; pr[1] = l; }
#pragma unroll
            for (int dt = 0; dt < C::DT; dt++)
#pragma unroll
                for (int j = 0; j < 4; j++) pr[2 + 16 * dt + 4 * q + j] = acc[nt][dt][j];
        }
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

int chunk_rows_per_wg(int D) { return D >= 256 ? WAVES * 16 : WAVES * 32; }

hipError_t launch_chunk(const ChunkArgs &p, hipStream_t s)
{
    dim3 grid(p.n_splits, p.t.H * p.n_row_tiles, p.t.A);
    switch (p.t.D) {
    case 64: chunk_split<1><<<grid, 256, 0, s>>>(p); break;
    case 128: chunk_split<2><<<grid, 256, 0, s>>>(p); break;
    case 256: chunk_split<4><<<grid, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t rows = (size_t)p.t.A * p.n_new * p.Hq;
    chunk_merge<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace kvq
