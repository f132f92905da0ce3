// Device helpers shared by the attention kernels: packed-code unpacking to
// fp16 and small vector types.  A chunk is 8 consecutive codes of one
// (token, head) row; it unpacks to the four fp16 pairs (c0,c4) (c1,c5) (c2,c6)
// (c3,c7), so every width yields the same element order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace dev {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr uint32_t MAGIC = 0x64006400u;   // fp16 1024.0 in both halves

// MAGIC in a vector register the compiler cannot fold back into a literal:
// (x & mask) | magic then selects to one v_and_or_b32 with the mask in a
// scalar register (a VALU instruction here reads at most one scalar
// operand, so with two literals it would take two instructions).  The empty
// asm emits nothing.
__device__ __forceinline__ uint32_t magic_v()
{
    uint32_t m = MAGIC;
    asm("" : "+v"(m));
    return m;
}

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
        const uint32_t w8 = w >> 8, mv = magic_v();
        const h2 x0 = as_h2((w & 0x000F000Fu) | mv);
        const h2 x1 = as_h2((w & 0x00F000F0u) | mv);
        const h2 x2 = as_h2((w8 & 0x000F000Fu) | mv);
        const h2 x3 = as_h2((w8 & 0x00F000F0u) | mv);
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
        const uint32_t mv = magic_v();
        Pairs r;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const h2 x = as_h2((y & (0x00030003u << (2 * i))) | mv);
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
        const uint32_t mv = magic_v();
        Pairs r;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + i) << 16) | (uint32_t)i;
            r.p[i] = __builtin_elementwise_fma(as_h2(perm(w1, w0, sel) | mv), one, m1024);
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
        const uint32_t mv = magic_v();
        const h2 x0 = as_h2((z & 0x00700007u) | mv);                    // c0 x1,  c4 x16
        const h2 x1 = as_h2((z & 0x03800038u) | mv);                    // c1 x8,  c5 x128
        const h2 x2 = as_h2((z & 0x000001C0u) | ((z2 & 0x001C0000u) | mv));  // c2 x64, c6 x4
        const h2 x3 = as_h2((z2 & 0x00E0000Eu) | mv);                   // c3 x2,  c7 x32
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


// Lane q (0..3) of a 16x16x32 operand, for one 64-dim group of a token
// row: chunks 2q and 2q+1 of 8 codes (2B bytes at byte 2Bq of the group),
// held as NDW dwords, so each 32-dim K-step lies in one group.
template <int B>
struct GRow {
    static constexpr bool ODD = (B == 3);                    // 6 bytes at offset 6q
    static constexpr int NDW = ODD ? 2 : (2 * B) / 4;

    __device__ static __forceinline__ void load(uint32_t *w, const uint8_t *grp, int q)
    {
        if constexpr (ODD) {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(grp + ((6 * q) & ~3));
            w[0] = p[0];
            w[1] = p[1];
        } else if constexpr (B == 2) {
            w[0] = reinterpret_cast<const uint32_t *>(grp)[q];
        } else if constexpr (B == 4) {
            const uint2 v = reinterpret_cast<const uint2 *>(grp)[q];
            w[0] = v.x; w[1] = v.y;
        } else {
            const uint4 v = reinterpret_cast<const uint4 *>(grp)[q];
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        }
    }

    // Exact codes of the lane's chunk u (0 or 1) as fp16 pairs.
    __device__ static __forceinline__ Pairs chunk(const uint32_t *w, int q, int u)
    {
        if constexpr (B == 4) {
            return Unpack<4>::run(w[u]);
        } else if constexpr (B == 2) {
            return Unpack<2>::run(u ? (w[0] >> 16) : (w[0] & 0xffffu));
        } else if constexpr (B == 8) {
            return Unpack<8>::run2(w[2 * u], w[2 * u + 1]);
        } else {
            const int o = ((6 * q) & 3) + 3 * u;               // o <= 5
            return Unpack<3>::run3(o >= 4 ? w[1] : w[0], w[1], o & 3);
        }
    }
};

__device__ __forceinline__ h8 operand(const Pairs &pr)
{
    h8 v;
    v[0] = pr.p[0][0]; v[1] = pr.p[0][1];
    v[2] = pr.p[1][0]; v[3] = pr.p[1][1];
    v[4] = pr.p[2][0]; v[5] = pr.p[2][1];
    v[6] = pr.p[3][0]; v[7] = pr.p[3][1];
    return v;
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

// Dequantized fp16 values of a chunk: fma(code, scale, bias) per element,
// with meta = {fp16 scale, fp16 bias}.
__device__ __forceinline__ void dequant(Pairs &pr, uint32_t meta)
{
    const h2 sb = as_h2(meta);
    const h2 s = {sb[0], sb[0]}, b = {sb[1], sb[1]};
#pragma unroll
    for (int i = 0; i < 4; i++) pr.p[i] = __builtin_elementwise_fma(pr.p[i], s, b);
}

__device__ __forceinline__ int seq_blocks(const Tables &t, int a) { return clampi(t.n_blocks[a], 0, t.max_blocks); }
__device__ __forceinline__ int seq_window(const Tables &t, int a)
{
    return t.n_window ? clampi(t.n_window[a], 0, t.window_cap) : 0;
}

}  // namespace dev
}  // namespace kvq
