// Latent (MLA) decode over a quantized latent cache (gfx950, matrix cores).
//
// What it computes (DeepSeek-V2-Lite absorbed attention as the pages use
// it for their MLA model; softmax attention of one query token per head):
// one latent KV head of 512 dims, quantized in 64-token blocks, with an
// optional bf16 rope part of 64 dims per token kept beside it.  Query head h
// (of up to 16) scores key t as q_h . [latent_t ; rope_t] (576 dims) and
// averages the dequantized latents (512 dims) as values.
//
// Work decomposition: a workgroup of eight waves takes one sequence and SB
// consecutive blocks (or the sequence's bf16 window).  Per 64-key tile all
// 512 lanes dequantize once into LDS as K rows [key][576] (double-buffered,
// while the codes of the tile after next load into registers).  Wave w owns
// keys 16(w%4)..+15 of every tile and latent dims 256(w/4)..+255 of the
// output, with its own online softmax:
//   S^T[key][head] = K.Q^T    v_mfma_f32_16x16x32_f16, 18 K-steps over 576 dims
//   O^T[dim][head] += V^T.P^T v_mfma_f32_16x16x16_f16, 16 tiles of 16 dims
// The V^T operand is read from the same K rows with ds_read_b64_tr_b16 (each
// lane gets one dim of four consecutive keys), and the S^T result layout
// (lane: head l%16, keys 4(l/16)..+3) is exactly the B operand of the P.V
// product, so probabilities never leave registers.  Waves 4-7 dequantize
// before their matrix work, waves 0-3 after, so the two waves of a SIMD
// overlap.  At the end the key groups combine through LDS into one partial
// (m, l, acc[512]) per head; the decode merge kernel combines the splits.
#include "kvq_internal.h"
#include "unpack.h"

namespace kvq {
namespace {

using namespace dev;

constexpr int DL = 512;                 // latent dims
constexpr int TILE = 64;                // keys per tile (one block)
constexpr int OT = 256 / 16;            // 16-dim output tiles per wave
constexpr float LAZY = 8.0f;            // running-max slack, log2 units

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

template <int R>
struct MCfg {
    static constexpr int DK = DL + R;   // score dims
    static constexpr int KR = DK + 16;  // LDS K row stride (halves)
    static constexpr int KS = DK / 32;  // K-steps of S^T
    static constexpr int BUF = TILE * KR;
};

// LDS rows are 8 dwords (mod 32) apart, and row r keeps its 16-byte chunks
// pairwise swapped (position ^ 8) when bit 2 of r is set.  gfx950's LDS reads
// through 64 banks, serving a 16-byte read for 16 lanes per cycle (lanes 0-3,
// 12-15, 20-27 together, then 4-11, 16-19, 28-31; the same for 32-63) and an
// 8-byte read for 32 consecutive lanes; writes go through 32 banks, eight
// lanes per cycle for 16 bytes.  With this layout the K-operand reads, the
// transposed V reads and the dequantized row stores all run without bank
// conflicts (the 4-dword row step without a swap cost 4 extra cycles per
// K read and 2 per transposed read).
__device__ __forceinline__ int swz(int row) { return ((row >> 2) & 1) << 3; }

// One lane's share of a quantized tile: key = tid & 63, latent group
// e = tid >> 6 (dims 64e..64e+63, 8 chunks of 8 codes), its metadata, and
// rope dims 8e..8e+7.
struct MlaRaw {
    uint32_t c[16];                     // 8 chunks x B bytes, unused dwords zero
    uint32_t m;                         // (scale, bias) of the group
    uint32_t r[4];                      // 8 bf16 rope values
    int bits;
};

template <int B>
__device__ __forceinline__ void load_share(uint32_t (&c)[16], const uint8_t *p)
{
#pragma unroll
    for (int i = 0; i < B; i++) {
        const uint2 x = reinterpret_cast<const uint2 *>(p)[i];
        c[2 * i] = x.x;
        c[2 * i + 1] = x.y;
    }
}

// Widths and pool offsets of up to 64 consecutive blocks, one per lane, so
// a tile's loads never wait on a dependent scalar load.
struct MlaMeta {
    int base, bits;
    uint32_t lo, hi;
    int rope_blk;                       // block of the rope rows (DecodeArgs::rope_map)
};

__device__ __forceinline__ void mla_meta(MlaMeta &mm, const DecodeArgs &p, int a, int j0, int j1)
{
    const int jb = j0 + (int)(threadIdx.x & 63);
    mm.base = j0;
    mm.bits = 0;
    mm.lo = mm.hi = 0;
    mm.rope_blk = jb;
    if (jb < j1) {
        const size_t e = (size_t)a * p.t.max_blocks + jb;
        if (p.rope_map) mm.rope_blk = p.rope_map[e];
        mm.bits = p.t.bits[e];
        const uint64_t o = p.k.offset[e];
        mm.lo = (uint32_t)o;
        mm.hi = (uint32_t)(o >> 32);
    }
}

// Codes, metadata and rope of block kt (all fields assigned once, so the
// record stays in registers across the width branches).
template <int R>
__device__ __forceinline__ void load_block(MlaRaw &raw, MlaMeta &mm, const DecodeArgs &p, const uint16_t *rope,
                                           int64_t rope_tokens, int a, int kt, int j1)
{
    const int tid = threadIdx.x, key = tid & 63, e8 = tid >> 6;
    if (kt - mm.base >= 64) mla_meta(mm, p, a, kt, j1);   // blocks are visited in order
    const int i = kt - mm.base;
    const int b = __builtin_amdgcn_readlane(mm.bits, i);
    const uint8_t *blk = p.k.pool + (((uint64_t)(uint32_t)__builtin_amdgcn_readlane(mm.hi, i) << 32) |
                                     (uint32_t)__builtin_amdgcn_readlane(mm.lo, i));
    const uint32_t row_bytes = (uint32_t)(DL / 8) * b;
    uint32_t c[16];
#pragma unroll
    for (int x = 0; x < 16; x++) c[x] = 0;
    const uint8_t *share = blk + (key * row_bytes + e8 * (row_bytes / 8));
    switch (b) {
    case 2: load_share<2>(c, share); break;
    case 3: load_share<3>(c, share); break;
    case 4: load_share<4>(c, share); break;
    default: load_share<8>(c, share); break;
    }
    const uint32_t mw = *reinterpret_cast<const uint32_t *>(blk + (64 * row_bytes + 4 * (key * (DL / 64) + e8)));
    uint4 rr = {0, 0, 0, 0};
    if (R) {
        const int rb = __builtin_amdgcn_readlane(mm.rope_blk, i);
        rr = *reinterpret_cast<const uint4 *>(rope + ((size_t)a * rope_tokens + (size_t)rb * TILE + key) * R + 8 * e8);
    }
#pragma unroll
    for (int x = 0; x < 16; x++) raw.c[x] = c[x];
    raw.r[0] = rr.x; raw.r[1] = rr.y; raw.r[2] = rr.z; raw.r[3] = rr.w;
    raw.m = mw;
    raw.bits = b;
}

// Chunk ch (8 latent dims) of the share, dequantized.
template <int B>
__device__ __forceinline__ Pairs share_chunk(const MlaRaw &raw, int ch)
{
    Pairs pr;
    if constexpr (B == 4) {
        pr = Unpack<4>::run(raw.c[ch]);
    } else if constexpr (B == 2) {
        const uint32_t d = raw.c[ch >> 1];
        pr = Unpack<2>::run((ch & 1) ? (d >> 16) : (d & 0xffffu));
    } else if constexpr (B == 8) {
        pr = Unpack<8>::run2(raw.c[2 * ch], raw.c[2 * ch + 1]);
    } else {
        const int o = 3 * ch, i = o >> 2;                 // compile-time after unrolling
        pr = Unpack<3>::run3(raw.c[i], raw.c[i + 1 < 6 ? i + 1 : i], o & 3);
    }
    dequant(pr, raw.m);
    return pr;
}

// The fp16 pairs (c0,c4) (c1,c5) (c2,c6) (c3,c7) of a chunk as 8 halves in
// that order: K rows keep each chunk in this order (the query operand is
// built the same way); stored position k holds dim (k>>1) + 4(k&1).
__device__ __forceinline__ h8 row_order(const Pairs &p)
{
    h8 o;
    o[0] = p.p[0][0]; o[1] = p.p[0][1]; o[2] = p.p[1][0]; o[3] = p.p[1][1];
    o[4] = p.p[2][0]; o[5] = p.p[2][1]; o[6] = p.p[3][0]; o[7] = p.p[3][1];
    return o;
}

template <int R, int B>
__device__ __forceinline__ void store_block(const MlaRaw &raw, _Float16 *kh)
{
    constexpr int KR = MCfg<R>::KR;
    const int tid = threadIdx.x, key = tid & 63, e8 = tid >> 6;
    _Float16 *row = kh + key * KR;
    const int sw = swz(key);
#pragma unroll
    for (int ch = 0; ch < 8; ch++)
        *reinterpret_cast<h8 *>(row + ((64 * e8 + 8 * ch) ^ sw)) = row_order(share_chunk<B>(raw, ch));
    if (R) {
        const uint4 x = {raw.r[0], raw.r[1], raw.r[2], raw.r[3]};
        *reinterpret_cast<h8 *>(row + ((DL + 8 * e8) ^ sw)) = row_order(bf16_pairs(x));
    }
}

template <int R>
__device__ __forceinline__ void store_raw(const MlaRaw &raw, _Float16 *kh)
{
    switch (raw.bits) {
    case 2: store_block<R, 2>(raw, kh); break;
    case 3: store_block<R, 3>(raw, kh); break;
    case 4: store_block<R, 4>(raw, kh); break;
    default: store_block<R, 8>(raw, kh); break;
    }
}

// bf16 window rows w0.. of sequence a straight into LDS (rows past the
// window repeat its last row; they are masked).
template <int R>
__device__ __forceinline__ void store_window(const DecodeArgs &p, const uint16_t *rope, int64_t rope_tokens, int a,
                                             int nb, int nw, int w0, _Float16 *kh)
{
    constexpr int KR = MCfg<R>::KR;
    const int tid = threadIdx.x, key = tid & 63, e8 = tid >> 6;
    const int w = min(w0 + key, nw - 1);
    const uint4 *src = reinterpret_cast<const uint4 *>(p.k.window + ((size_t)a * p.t.window_cap + w) * DL + 64 * e8);
    _Float16 *row = kh + key * KR;
    const int sw = swz(key);
#pragma unroll
    for (int ch = 0; ch < 8; ch++)
        *reinterpret_cast<h8 *>(row + ((64 * e8 + 8 * ch) ^ sw)) = row_order(bf16_pairs(src[ch]));
    if (R) {
        int rnb = nb;
        if (p.rope_map) rnb = min(max(p.rope_nb[a], 0), p.rope_max_blocks);
        const uint4 *rp = reinterpret_cast<const uint4 *>(
            rope + ((size_t)a * rope_tokens + (size_t)rnb * TILE + w) * R + 8 * e8);
        *reinterpret_cast<h8 *>(row + ((DL + 8 * e8) ^ sw)) = row_order(bf16_pairs(rp[0]));
    }
}

// Per-wave state: lane l is head l%16; of each tile it scores keys
// 16(w%4) + 4(l/16) + r and holds O^T rows (stored positions)
// 256(w/4) + 16t + 4(l/16) + r.
template <int R>
struct MlaState {
    h8 qop[MCfg<R>::KS];
    f4 acc[OT];
    float m_run, l_run;
};

template <int R>
__device__ __forceinline__ void tile_compute(MlaState<R> &w, const _Float16 *kh, int valid, float c, int kg, int dh)
{
    constexpr int KR = MCfg<R>::KR, KS = MCfg<R>::KS;
    const int lane = threadIdx.x & 63, m = lane & 15, kq = lane >> 4;
    const int k0 = 16 * kg;
    // two independent accumulator chains over the K-steps
    f4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    const _Float16 *ka = kh + (k0 + m) * KR + ((8 * kq) ^ swz(m));   // k0 is a multiple of 16
#pragma unroll
    for (int s = 0; s < KS; s += 2) {
        const h8 a0 = *reinterpret_cast<const h8 *>(ka + 32 * s);
        const h8 a1 = *reinterpret_cast<const h8 *>(ka + 32 * (s + 1));
        sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, w.qop[s], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, w.qop[s + 1], sb, 0, 0, 0);
    }
    f4 st = sa + sb;
    if (valid < TILE) {
#pragma unroll
        for (int r = 0; r < 4; r++)
            if (k0 + 4 * kq + r >= valid) st[r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_old = w.m_run;
    const float tmax = mx * c;
    const float m_new = (tmax > m_old + LAZY) ? tmax : m_old;
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_old - m_new);
    w.m_run = m_new;
    const h2 p01 = __builtin_convertvector(f2{__builtin_amdgcn_exp2f(__builtin_fmaf(st[0], c, -m_use)),
                                               __builtin_amdgcn_exp2f(__builtin_fmaf(st[1], c, -m_use))}, h2);
    const h2 p23 = __builtin_convertvector(f2{__builtin_amdgcn_exp2f(__builtin_fmaf(st[2], c, -m_use)),
                                               __builtin_amdgcn_exp2f(__builtin_fmaf(st[3], c, -m_use))}, h2);
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    w.l_run = w.l_run * alpha + __builtin_amdgcn_fdot2(p23, ones, __builtin_amdgcn_fdot2(p01, ones, 0.0f, false), false);
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < OT; t++) w.acc[t] *= alpha;
    }
    const h4 pb = {p01[0], p01[1], p23[0], p23[1]};
    // V^T operand: lane j of each 16-lane group addresses key k0 + 4(l/16) + j/4,
    // positions n0 + 4(j%4)..+3; the transposed read hands lane l position
    // n0 + l%16 of those four keys.
    const _Float16 *vb = kh + (k0 + 4 * kq + (m >> 2)) * KR + ((256 * dh + 4 * (m & 3)) ^ swz(4 * kq));
#pragma unroll
    for (int t = 0; t < OT; t++) {
        const s4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4 *)(vb + 16 * t));
        w.acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, raw), pb, w.acc[t], 0, 0, 0);
    }
}

// Query chunks loaded by stage's lanes (chunk tid + 512 i = head, K-step,
// quarter) into LDS in operand form, and each lane's operands back.  A head's
// 4 KS chunks sit 4 KS + 1 chunks apart, so the 16 heads a read serves start
// on 16 different 4-bank groups (no bank conflicts).
template <int R>
__device__ __forceinline__ void stage_query(_Float16 *qs, const uint4 (&qv)[(16 * MCfg<R>::KS * 4 + 511) / 512])
{
    constexpr int HC = MCfg<R>::KS * 4, QCH = 16 * HC, QPL = (QCH + 511) / 512;
#pragma unroll
    for (int i = 0; i < QPL; i++) {
        const int ch = threadIdx.x + 512 * i;
        if (ch < QCH) *reinterpret_cast<h8 *>(qs + 8 * (ch + ch / HC)) = row_order(bf16_pairs(qv[i]));
    }
}

template <int R>
__device__ __forceinline__ void load_query(MlaState<R> &w, const _Float16 *qs, bool hv)
{
    constexpr int KS = MCfg<R>::KS;
    const int lane = threadIdx.x & 63, m = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int k = 0; k < KS; k++) {
        h8 o = *reinterpret_cast<const h8 *>(qs + 8 * (m * (4 * KS + 1) + 4 * k + kq));
        if (!hv) o = h8{0, 0, 0, 0, 0, 0, 0, 0};
        w.qop[k] = o;
    }
}

template <int R>
__global__ __launch_bounds__(512, 1) void mla_split(DecodeArgs p, const uint16_t *rope, int64_t rope_tokens)
{
    using C = MCfg<R>;
    __shared__ __attribute__((aligned(16))) _Float16 lds[2 * C::BUF];

    const int s = blockIdx.x, a = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, kq = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3, dh = wave >> 2;
    // The split's block table and the query rows do not depend on the
    // sequence's counts: their loads go out with the count loads (table
    // entries up to the split's end within max_blocks are valid memory;
    // those past n_blocks are never used).  Block data waits for the counts.
    MlaMeta mm;
    mm.base = -(1 << 20);
    mm.rope_blk = 0;
    if (s * p.SB < p.t.max_blocks) mla_meta(mm, p, a, s * p.SB, min(s * p.SB + p.SB, p.t.max_blocks));

    MlaState<R> w;
    const bool hv = m < p.Hq;
    // The query rows once per workgroup: 16 heads x KS K-steps x 4 lane
    // quarters of 8 dims, as fp16 operand chunks, into the second tile buffer
    // (unused until tile 1 is stored); each wave then reads its operands from
    // LDS instead of every wave fetching all rows.  The loads go out before the
    // first tiles' loads, the LDS stores after them.
    constexpr int QCH = 16 * C::KS * 4, QPL = (QCH + 511) / 512;
    _Float16 *qs = lds + C::BUF;
    uint4 qv[QPL];
#pragma unroll
    for (int i = 0; i < QPL; i++) {
        const int ch = tid + 512 * i, h = ch / (4 * C::KS), k = (ch >> 2) % C::KS, q4 = ch & 3;
        qv[i] = uint4{0, 0, 0, 0};
        if (ch < QCH && h < p.Hq)
            qv[i] = *reinterpret_cast<const uint4 *>(p.q + ((size_t)a * p.Hq + h) * C::DK + 32 * k + 8 * q4);
    }
#pragma unroll
    for (int t = 0; t < OT; t++) w.acc[t] = f4{0.f, 0.f, 0.f, 0.f};
    w.m_run = -INFINITY;
    w.l_run = 0.0f;

    const int nb = seq_blocks(p.t, a), nw = seq_window(p.t, a);
    const int nsb = (nb + p.SB - 1) / p.SB;
    const bool win = (s == nsb) && nw > 0;
    if (s > nsb || (s == nsb && !win)) return;

    if (!win) {
        // Tile j in buffer j&1; between barriers the tile j+1 is stored into
        // the other buffer (last read before the previous barrier).
        const int j0 = s * p.SB, j1 = min(j0 + p.SB, nb), n = j1 - j0;
        MlaRaw raw, raw1;
        load_block<R>(raw, mm, p, rope, rope_tokens, a, j0, j1);
        if (n > 1) load_block<R>(raw1, mm, p, rope, rope_tokens, a, j0 + 1, j1);
        stage_query<R>(qs, qv);
        __syncthreads();
        load_query<R>(w, qs, hv);
        __syncthreads();
        store_raw<R>(raw, lds);
        if (n > 1) raw = raw1;
        __syncthreads();
        for (int j = 0; j < n; j++) {
            _Float16 *cur = lds + (j & 1) * C::BUF, *nxt = lds + ((j + 1) & 1) * C::BUF;
            if (dh && j + 1 < n) {
                store_raw<R>(raw, nxt);
                if (j + 2 < n) load_block<R>(raw, mm, p, rope, rope_tokens, a, j0 + j + 2, j1);
            }
            tile_compute<R>(w, cur, TILE, p.c, kg, dh);
            if (!dh && j + 1 < n) {
                store_raw<R>(raw, nxt);
                if (j + 2 < n) load_block<R>(raw, mm, p, rope, rope_tokens, a, j0 + j + 2, j1);
            }
            __syncthreads();
        }
    } else {
        stage_query<R>(qs, qv);
        __syncthreads();
        load_query<R>(w, qs, hv);
        __syncthreads();
        for (int w0 = 0; w0 < nw; w0 += TILE) {
            store_window<R>(p, rope, rope_tokens, a, nb, nw, w0, lds);
            __syncthreads();
            tile_compute<R>(w, lds, nw - w0, p.c, kg, dh);
            __syncthreads();
        }
    }

    // Combine the four key groups: wave (kg, dh) writes its 16 O^T tiles as
    // they sit in its registers ([tile][lane] 16-byte units), the dh = 0
    // waves their (m, l); after one barrier wave (kg, dh) sums tiles
    // 4kg..+3 of its dim half over the four key groups, rescaled to the
    // common max per head, and writes them to the partial rows (lane (h, kq)
    // holds stored positions 256dh + 16t + 4kq..+3 of head h).
    constexpr int TB = OT * 64 * 16;                       // one wave's tiles (bytes)
    static_assert(8 * TB + 128 * 4 <= 2 * C::BUF * 2, "combine buffer exceeds the tile buffers");
    float l = w.l_run + __shfl_xor(w.l_run, 16);
    l += __shfl_xor(l, 32);
    uint8_t *cbuf = reinterpret_cast<uint8_t *>(lds);
    float *ml = reinterpret_cast<float *>(cbuf + 8 * TB);   // m [4][16], l [4][16]
#pragma unroll
    for (int t = 0; t < OT; t++) *reinterpret_cast<f4 *>(cbuf + wave * TB + (t * 64 + lane) * 16) = w.acc[t];
    if (kq == 0 && dh == 0) {
        ml[kg * 16 + m] = w.m_run;
        ml[64 + kg * 16 + m] = l;
    }
    __syncthreads();
    float fu[4];
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; u++) M = fmaxf(M, ml[u * 16 + m]);
    float L = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const float mu = ml[u * 16 + m];
        fu[u] = (mu == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mu - M);
        L += fu[u] * ml[64 + u * 16 + m];
    }
    const int stride = DL + 2;
    float *prow = p.part + ((size_t)(a * p.Hq + m) * p.n_splits + s) * stride;
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
        const int t = 4 * kg + tt;
        f4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; u++) v += fu[u] * *reinterpret_cast<const f4 *>(cbuf + (4 * dh + u) * TB + (t * 64 + lane) * 16);
        // stored positions 8c..8c+7 hold dims 8c + (0 4 1 5 2 6 3 7): lanes kq
        // and kq ^ 1 (16 lanes apart) trade two values so that the even one
        // holds dims 8c..8c+3 and the odd one 8c+4..8c+7, written as two
        // 8-byte stores (a partial row starts 8-byte aligned)
        const bool odd = kq & 1;
        const float y0 = __shfl_xor(odd ? v[0] : v[1], 16), y1 = __shfl_xor(odd ? v[2] : v[3], 16);
        if (hv) {
            const int d0 = 256 * dh + 16 * t + 8 * (kq >> 1) + 4 * odd;
            float2 *dst = reinterpret_cast<float2 *>(prow + 2 + d0);
            dst[0] = odd ? float2{y0, y1} : float2{v[0], v[2]};
            dst[1] = odd ? float2{v[1], v[3]} : float2{y0, y1};
        }
    }
    if (wave == 0 && kq == 0 && hv) {
        prow[0] = M;
        prow[1] = L;
    }
}

}  // namespace

bool mla_supported(int D, int H, int G, int rope_dim)
{
    return D == DL && H == 1 && G <= 16 && (rope_dim == 0 || rope_dim == 64);
}

void mla_plan(int A, int max_blocks, int window_cap, int *SB, int *n_splits)
{
    // about one workgroup per compute unit (the kernel holds 148 KB of LDS)
    int sb = 1;
    while ((long)A * ((max_blocks + sb - 1) / sb) > 256) sb <<= 1;
    *SB = sb;
    *n_splits = (max_blocks + sb - 1) / sb + (window_cap > 0 ? 1 : 0);
    if (*n_splits < 1) *n_splits = 1;
}

hipError_t launch_mla(const DecodeArgs &p, const uint16_t *rope, int rope_dim, int64_t rope_tokens, hipStream_t s)
{
    dim3 grid(p.n_splits, 1, p.t.A);
    if (rope_dim == 64) mla_split<64><<<grid, 512, 0, s>>>(p, rope, rope_tokens);
    else mla_split<0><<<grid, 512, 0, s>>>(p, rope, rope_tokens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_merge(p, s);
}

}  // namespace kvq
