// CacheCard image of one sequence: gather from / scatter to the cache.
//
// A CacheCard carries one agent's quantized KV groups, their widths and the
// recent native-precision rows, so the cache can be persisted and handed to
// another process (QKVShare, Metodologia: the CacheCard; Agent Memory Below
// the Prompt, arXiv 2603.04428, Abstract: per-agent caches persisted in 4-bit
// form and reloaded).  The image concatenates, in this order:
//   K block payloads   block j: kvq_block_bytes(bits[j], H, D) bytes, j < nb
//   V block payloads   (absent for a latent cache)
//   K window rows      bf16 [W][H][D]
//   V window rows      (absent for a latent cache)
//   rope rows          bf16 [64*nb + W][H][R]   (absent when R == 0)
//   widths             uint8 [nb]
// Every segment but the last is a multiple of 128 bytes, so all start
// 16-byte aligned.  The kernel is a set of contiguous copies: grid.x
// enumerates quarters of the block slots of K and V, then 16 KiB chunks of
// the windows and the rope rows; slots past the sequence's counts exit.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int CHUNK = 16384;                   // bytes per workgroup for rows
constexpr int PARTS = 4;                       // workgroups per block payload

struct CardArgs {
    Tables t;
    const uint64_t *k_offset, *v_offset;       // v_offset null: latent
    uint8_t *k_pool, *v_pool;
    uint16_t *k_window, *v_window;
    uint16_t *rope;
    int rope_dim;
    int seq;
    uint8_t *image;
    uint64_t image_bytes;
    int to_image;                              // 1 gather, 0 scatter
    int w_chunks, r_chunks;                    // 16 KiB chunks of one window, of the rope rows
};

__device__ __forceinline__ uint64_t bb(int bits, int H, int D) { return (uint64_t)H * D * (8 * bits + 4); }

// Sums of the block sizes of blocks [0, j) and [0, nb) of the sequence, in
// one pass over the widths (every thread gets both; 256 threads).
__device__ void blocks_prefix(const CardArgs &p, int j, int nb, uint64_t &before, uint64_t &all)
{
    __shared__ unsigned long long part[2][4];
    const uint8_t *bits = p.t.bits + (size_t)p.seq * p.t.max_blocks;
    unsigned long long sa = 0, sb = 0;
    for (int i = threadIdx.x; i < nb; i += blockDim.x) {
        const uint64_t b = bb(bits[i], p.t.H, p.t.D);
        sa += b;
        if (i < j) sb += b;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        sa += __shfl_xor(sa, o);
        sb += __shfl_xor(sb, o);
    }
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = sa;
        part[1][threadIdx.x >> 6] = sb;
    }
    __syncthreads();
    all = part[0][0] + part[0][1] + part[0][2] + part[0][3];
    before = part[1][0] + part[1][1] + part[1][2] + part[1][3];
}

// Copy n bytes (a multiple of 16) between device memory and the image.
__device__ __forceinline__ void copy16(const CardArgs &p, uint8_t *mem, uint64_t img_off, uint64_t n)
{
    if (img_off >= p.image_bytes) return;
    if (n > p.image_bytes - img_off) n = p.image_bytes - img_off;   // never past the image
    uint4 *dst = reinterpret_cast<uint4 *>(p.to_image ? p.image + img_off : mem);
    const uint4 *src = reinterpret_cast<const uint4 *>(p.to_image ? mem : p.image + img_off);
    const uint64_t m = n / 16;
    uint64_t i = threadIdx.x;
    for (; i + 3 * blockDim.x < m; i += 4 * blockDim.x) {     // four loads in flight per lane
        const uint4 a = src[i], b = src[i + blockDim.x], c = src[i + 2 * blockDim.x], d = src[i + 3 * blockDim.x];
        dst[i] = a;
        dst[i + blockDim.x] = b;
        dst[i + 2 * blockDim.x] = c;
        dst[i + 3 * blockDim.x] = d;
    }
    for (; i < m; i += blockDim.x) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void card_copy(CardArgs p)
{
    const int H = p.t.H, D = p.t.D, R = p.rope_dim;
    const int a = p.seq;
    int nb = p.t.n_blocks[a];
    nb = nb < 0 ? 0 : (nb > p.t.max_blocks ? p.t.max_blocks : nb);
    int W = p.t.n_window ? p.t.n_window[a] : 0;
    W = W < 0 ? 0 : (W > p.t.window_cap ? p.t.window_cap : W);
    const int n_kv = p.v_pool ? 2 : 1;
    const int mb = p.t.max_blocks;
    int x = blockIdx.x;
    const bool is_block = x < n_kv * mb * PARTS;
    const int jx = is_block ? (x % (mb * PARTS)) / PARTS : 0;
    uint64_t before, kv_bytes;
    blocks_prefix(p, jx, nb, before, kv_bytes);
    const uint64_t row = (uint64_t)H * D * 2;
    const uint64_t win_off = kv_bytes * n_kv;
    if (is_block) {                                           // one part of a block payload
        const int kv = x / (mb * PARTS), part = x % PARTS;
        if (jx >= nb) return;
        const size_t e = (size_t)a * mb + jx;
        const uint64_t n = bb(p.t.bits[e], H, D), pn = (n / 16 + PARTS - 1) / PARTS * 16;
        const uint64_t beg = (uint64_t)part * pn;
        if (beg >= n) return;
        uint8_t *blk = (kv ? p.v_pool : p.k_pool) + (kv ? p.v_offset : p.k_offset)[e];
        copy16(p, blk + beg, kv * kv_bytes + before + beg, n - beg < pn ? n - beg : pn);
        return;
    }
    x -= n_kv * mb * PARTS;
    if (x < n_kv * p.w_chunks) {                              // window rows
        const int kv = x / p.w_chunks, c = x % p.w_chunks;
        const uint64_t total = (uint64_t)W * row, beg = (uint64_t)c * CHUNK;
        if (beg >= total) return;
        const uint64_t n = total - beg < (uint64_t)CHUNK ? total - beg : (uint64_t)CHUNK;
        uint8_t *win = reinterpret_cast<uint8_t *>((kv ? p.v_window : p.k_window) +
                                                   (size_t)a * p.t.window_cap * H * D);
        copy16(p, win + beg, win_off + kv * total + beg, n);
        return;
    }
    x -= n_kv * p.w_chunks;
    if (R && x < p.r_chunks) {                                // rope rows, by token position
        const uint64_t total = (uint64_t)(64 * (uint64_t)nb + W) * H * R * 2, beg = (uint64_t)x * CHUNK;
        if (beg >= total) return;
        const uint64_t n = total - beg < (uint64_t)CHUNK ? total - beg : (uint64_t)CHUNK;
        const size_t rope_tokens = (size_t)64 * mb + p.t.window_cap;
        uint8_t *rp = reinterpret_cast<uint8_t *>(p.rope + (size_t)a * rope_tokens * H * R);
        copy16(p, rp + beg, win_off + n_kv * (uint64_t)W * row + beg, n);
        return;
    }
    if (R) x -= p.r_chunks;
    if (x == 0 && p.to_image) {                               // widths (gather only)
        const uint64_t off = win_off + n_kv * (uint64_t)W * row + (R ? (uint64_t)(64 * (uint64_t)nb + W) * H * R * 2 : 0);
        const uint8_t *bits = p.t.bits + (size_t)a * mb;
        for (int i = threadIdx.x; i < nb; i += blockDim.x)
            if (off + i < p.image_bytes) p.image[off + i] = bits[i];
    }
}

}  // namespace

hipError_t launch_card(const Tables &t, const uint64_t *k_offset, const uint64_t *v_offset, uint8_t *k_pool,
                       uint8_t *v_pool, uint16_t *k_window, uint16_t *v_window, uint16_t *rope, int rope_dim,
                       int seq, uint8_t *image, uint64_t image_bytes, int to_image, hipStream_t s)
{
    CardArgs p;
    p.t = t;
    p.k_offset = k_offset;
    p.v_offset = v_offset;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.k_window = k_window;
    p.v_window = v_window;
    p.rope = rope;
    p.rope_dim = rope_dim;
    p.seq = seq;
    p.image = image;
    p.image_bytes = image_bytes;
    p.to_image = to_image;
    const uint64_t row = (uint64_t)t.H * t.D * 2;
    p.w_chunks = t.window_cap > 0 ? (int)((t.window_cap * row + CHUNK - 1) / CHUNK) : 0;
    p.r_chunks = rope_dim ? (int)((((uint64_t)64 * t.max_blocks + t.window_cap) * t.H * rope_dim * 2 + CHUNK - 1) /
                                  CHUNK)
                          : 0;
    const int n_kv = v_pool ? 2 : 1;
    const int64_t gx = (int64_t)n_kv * t.max_blocks * PARTS + (int64_t)n_kv * p.w_chunks + p.r_chunks + 1;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    card_copy<<<(unsigned)gx, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace kvq
