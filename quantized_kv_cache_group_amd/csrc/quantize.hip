// Quantize and restore kernels (gfx950).
//
// Format and arithmetic: affine min/max groups of 64 elements along head_dim,
// fp16 scale and bias, codes against the stored fp16 values, little-endian
// bitstream packing (the reading of the "quantized KV groups" of QKVShare,
// Metodologia, and of the 4-bit format of Agent Memory Below the Prompt,
// Abstract; one width per block as in CoMixKV, Abstract).
//
// This translation unit is compiled with -ffp-contract=off: the codes,
// scales and biases it writes are bit-for-bit the documented sequence of IEEE
// binary32 operations (its two divisions are computed by sequences proven
// equal to the correctly rounded quotient on every input they can receive).
// It is also compiled with the IEEE mode bit off (-mno-amdgpu-ieee,
// -fno-honor-nans): NaN and Inf inputs are a precondition violation, and for
// finite operands min/max then need no canonicalising instruction.
//
// Layout of the work: one workgroup (256 lanes, 4 wave64s) per (head,
// block, sequence), heads fastest in the grid, so workgroups running side by
// side read neighbouring slices of the same token rows.  A group of 64 bf16
// values (128 contiguous bytes) belongs to 8 lanes, 8 values (16 bytes) each,
// so a wave covers 8 groups per step and its global loads are full 128-byte
// segments.  min/max use 3 DPP exchanges
// inside each 8-lane slice.  Every lane loads all of its data before the
// arithmetic, to keep several 16-byte loads in flight per lane.
#include "kvq_internal.h"

namespace kvq {
namespace {

// Ids straight from the compiler builtins: with the IEEE mode bit off, the
// device library's id functions (behind threadIdx, blockIdx, gridDim) do
// not inline into these kernels and would be real calls, whose results the
// compiler can no longer see as wave-uniform.
__device__ __forceinline__ int tid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int wg_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int wg_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int wg_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }
// Largest grid y of the quantize and restore launches; the launchers split
// larger block counts into several launches.
constexpr int kGridY = 65535;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // plain vector: no struct copies

// Streaming accesses: the bf16 source rows, the code words and the restored
// rows are each touched once, so their loads and stores carry the
// non-temporal hint (measured: restore 22% faster, quantize up to 3%).  The
// 4-byte scale/bias words stay plain stores: one lane in eight writes one,
// and they reach full cache lines only by merging in the cache.  The
// attention kernels, whose lanes share cache lines, are slower with the hint
// and do not use it.
template <typename T>
__device__ __forceinline__ void stream_store(T *p, T v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ uint4 stream_load16(const void *p)
{
    const u32x4 t = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f)
{
    _Float16 h = (_Float16)f;                      // v_cvt_f16_f32, round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

// Lane exchanges inside 8-lane slices through DPP, which the compiler fuses
// into the consuming min/max: xor 1 and xor 2 are quad permutations; once a
// quad holds one value, the half-row mirror (lane i <- lane 7-i) brings the
// other quad's.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;                  // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;                  // quad_perm [2,3,0,1]
constexpr int DPP_NEXT = 0xF9;                  // quad_perm [1,2,3,3]: lane j <- j+1 (j < 3)
constexpr int DPP_HALF_MIRROR = 0x141;          // row_half_mirror

// bf16 round to nearest even of a finite fp32 value.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int seq_blocks(const Tables &t, int a)
{
    int nb = t.n_blocks[a];
    return nb < 0 ? 0 : (nb > t.max_blocks ? t.max_blocks : nb);
}
__device__ __forceinline__ int seq_window(const Tables &t, int a)
{
    if (!t.n_window) return 0;
    int nw = t.n_window[a];
    return nw < 0 ? 0 : (nw > t.window_cap ? t.window_cap : nw);
}

// One lane's share of a group: 8 bf16 values (raw) at positions 8*sub ..
// 8*sub+7, sub = lane & 7; the 8 lanes of an aligned 8-lane slice hold one
// group and must all be active.  Writes the lane's codes into the group's
// 2B code words at gc and, from sub 0, the packed {fp16 scale, fp16 bias}.
template <int B>
__device__ __forceinline__ void quant_lane(const uint4 raw, int lane, uint8_t *gc, uint32_t *meta_word)
{
    constexpr int N = (1 << B) - 1;
    const int sub = lane & 7;
    float x[8];
    x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x);
    x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
    x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z);
    x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; i++) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
    mn = fminf(mn, dpp_f<DPP_XOR1>(mn));
    mx = fmaxf(mx, dpp_f<DPP_XOR1>(mx));
    mn = fminf(mn, dpp_f<DPP_XOR2>(mn));
    mx = fmaxf(mx, dpp_f<DPP_XOR2>(mx));
    mn = fminf(mn, dpp_f<DPP_HALF_MIRROR>(mn));
    mx = fmaxf(mx, dpp_f<DPP_HALF_MIRROR>(mx));
    mn = mn + 0.0f;                             // a zero extreme is +0
    mx = mx + 0.0f;
    // s = (mx - mn) / N, correctly rounded: reciprocal multiply plus one
    // fma correction.  For N = 3, 7, 15, 255 this equals the IEEE
    // quotient for every non-negative finite dividend (an exhaustive
    // check over all 2^31 such floats is in the test suite).
    const float range = mx - mn;
    constexpr float RN = 1.0f / (float)N;
    const float q0 = range * RN;
    float s = __builtin_fmaf(__builtin_fmaf(-q0, (float)N, range), RN, q0);
    // keep the binary32 rounding of s: without this barrier the compiler
    // may fuse the fma with the fp16 conversion (one rounding, not two)
    asm volatile("" : "+v"(s));
    const uint16_t sh = f32_to_f16_bits(s);
    const uint16_t bh = f32_to_f16_bits(mn);
    const float sf = f16_bits_to_f32(sh);
    const float bf = f16_bits_to_f32(bh);
    // 1/sf, correctly rounded: hardware reciprocal (within 1 ulp) and one
    // Newton step; exact for every positive finite fp16 sf from any start
    // within 2 ulp (checked exhaustively in the test suite).
    const float y0 = __builtin_amdgcn_rcpf(sf);
    const float inv = (sf == 0.0f) ? 0.0f : __builtin_fmaf(__builtin_fmaf(-sf, y0, 1.0f), y0, y0);

    // This lane's 8 codes, b bits each: codes 0..3 in lo, 4..7 in hi
    // (for b <= 4 the caller only uses lo | hi << 4b, formed below).
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float t = (x[i] - bf) * inv;
        // round half to even, then clamp to [0, N] (one med3; the clamp
        // equals max(0, min(N, r)) for every non-NaN r)
        const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(t), 0.0f, (float)N);
        const uint32_t cq = (uint32_t)r;
        if (i < 4) lo |= cq << (B * i);
        else hi |= cq << (B * (i - 4));
    }
    const uint64_t v = (B == 8) ? ((uint64_t)lo | ((uint64_t)hi << 32))
                                : (uint64_t)(lo | (hi << (4 * B)));

    if constexpr (B == 4) {
        stream_store(reinterpret_cast<uint32_t *>(gc) + sub, (uint32_t)v);
    } else if constexpr (B == 8) {
        stream_store(reinterpret_cast<uint64_t *>(gc) + sub, v);
    } else if constexpr (B == 2) {
        uint32_t mine = (uint32_t)v;                // 16 bits
        uint32_t other = dpp_u<DPP_XOR1>(mine);
        if ((sub & 1) == 0) stream_store(reinterpret_cast<uint32_t *>(gc) + (sub >> 1), mine | (other << 16));
    } else {                                        // B == 3: 24 bits, 4 lanes -> 3 words
        uint32_t mine = (uint32_t)v;
        uint32_t next = dpp_u<DPP_NEXT>(mine);      // lane j+1 of the same quad
        int j = sub & 3;
        if (j < 3) {
            uint32_t w = (mine >> (8 * j)) | (next << (24 - 8 * j));
            stream_store(reinterpret_cast<uint32_t *>(gc) + 3 * (sub >> 2) + j, w);
        }
    }
    if (sub == 0) *meta_word = (uint32_t)sh | ((uint32_t)bh << 16);
}

// Group index of this lane's k-th 16-byte piece inside a (block, head): a
// group of 64 bf16 values (128 contiguous bytes) belongs to 8 lanes, so a
// wave covers 8 groups per step and the 4 waves 32.
__device__ __forceinline__ int piece_group(int k)
{
    return (int)(tid_x() >> 6) * 8 + (int)((tid_x() & 63) >> 3) + 32 * k;
}

// Codes and scale/bias of the 64 tokens x D dims of head h of a block of
// width B, from this lane's pieces raw[k] (group piece_group(k)).
template <int B, int NG>
__device__ __forceinline__ void quant_rows(const uint4 (&raw)[2 * NG], uint8_t *__restrict__ blk, int H, int h)
{
    constexpr int D = NG * 64;
    constexpr int CODE_ROW = D * B / 8;             // bytes per (head, token)
    const int lane = tid_x() & 63;
    uint8_t *codes = blk + (size_t)h * 64 * CODE_ROW;
    uint32_t *meta = reinterpret_cast<uint32_t *>(blk + (size_t)H * 64 * CODE_ROW + (size_t)h * 64 * NG * 4);
#pragma unroll
    for (int k = 0; k < 2 * NG; k++) {
        const int gi = piece_group(k);
        quant_lane<B>(raw[k], lane, codes + (size_t)gi * (8 * B), meta + gi);
    }
}

// This lane's 2*NG pieces of head h of a block's source rows.
template <int NG>
__device__ __forceinline__ void load_rows(uint4 (&raw)[2 * NG], const uint16_t *__restrict__ src_blk, int H, int h)
{
    constexpr int D = NG * 64;
    const int sub = tid_x() & 7;
#pragma unroll
    for (int k = 0; k < 2 * NG; k++) {
        const int gi = piece_group(k);
        const int r = gi / NG, g = gi % NG;
        raw[k] = stream_load16(src_blk + ((size_t)r * H + h) * D + g * 64 + sub * 8);
    }
}

// One workgroup per (head, block, tensor x sequence).  The kernel has no
// loop over blocks: a loop lets the compiler keep every lane's per-piece
// addresses live across it, which costs occupancy; launches with more
// blocks than one grid dimension holds are split by the launcher (j0).
template <int NG>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a)
{
    const int h = wg_x();
    const int j = a.j0 + wg_y();
    const int x = wg_z() >= a.t.A ? 1 : 0;          // tensor: K, then V
    const int s = wg_z() - x * a.t.A;
    if (j >= seq_blocks(a.t, s)) return;
    // the rows do not depend on the block's table entries: their loads are
    // in flight together with the entries'
    uint4 raw[2 * NG];
    load_rows<NG>(raw, a.src[x] + ((size_t)s * a.src_seq_tokens + (size_t)j * 64) * a.t.H * (NG * 64), a.t.H, h);
    const int b = a.t.bits[(size_t)s * a.t.max_blocks + j];
    uint8_t *blk = a.pool[x] + a.offset[x][(size_t)s * a.t.max_blocks + j];
    switch (b) {
    case 2: quant_rows<2, NG>(raw, blk, a.t.H, h); break;
    case 3: quant_rows<3, NG>(raw, blk, a.t.H, h); break;
    case 4: quant_rows<4, NG>(raw, blk, a.t.H, h); break;
    case 8: quant_rows<8, NG>(raw, blk, a.t.H, h); break;
    default: break;                                 // precondition violation: nothing written
    }
}

// ---- append (quantize on append / window roll) ------------------------------
// For sequence a with W window tokens, the stream T = window[0..W) ++
// new[0..n_new) ends as: k = (W + n_new - keep) / 64 new blocks (when W +
// n_new > keep) made of T[0 .. 64k), then the window T[64k ..).  Widths and
// pool offsets of the new blocks are the caller's table entries nb .. nb+k-1.
// Blocks past max_blocks and window tokens past window_cap are never written
// (either would be a precondition violation).
__device__ __forceinline__ void append_plan(const AppendArgs &p, int a, int &nb, int &W, int &k, int &W2)
{
    nb = seq_blocks(p.t, a);
    W = seq_window(p.t, a);
    append_counts(nb, W, p.n_new, p.keep, p.t.max_blocks, p.t.window_cap, &k, &W2);
}

// A 64-element slice (16-byte piece c of 8) of stream token t of head h:
// from the window (base win_a, token stride ts) or from the new rows.
__device__ __forceinline__ const uint16_t *stream_piece(const uint16_t *win_a, const uint16_t *new_a, size_t ts,
                                                         int W, int t, int h, int width, int col)
{
    return (t < W ? win_a + (size_t)t * ts : new_a + (size_t)(t - W) * ts) + (size_t)h * width + col;
}

// Blocks: one workgroup per (new block i, tensor, head h, sequence a), all
// groups of the head; x = 2i + tensor (K, V), or i for a latent cache.
// Blocks only read the stream, so they run side by side; the window moves in
// the next launch.
template <int NG>
__global__ __launch_bounds__(256) void append_blocks(AppendArgs p)
{
    constexpr int D = NG * 64;
    const int n_kv = p.v_pool ? 2 : 1;
    const int kv = wg_x() % n_kv, i = wg_x() / n_kv, h = wg_y(), a = wg_z();
    const int H = p.t.H;
    int nb, W, k, W2;
    append_plan(p, a, nb, W, k, W2);
    if (i >= k) return;
    const size_t e = (size_t)a * p.t.max_blocks + nb + i;
    const uint16_t *win_a = kv ? p.v_window : p.k_window;
    if (win_a) win_a += (size_t)a * p.t.window_cap * H * D;
    const uint16_t *new_a = (kv ? p.v_new : p.k_new) + (size_t)a * p.n_new * H * D;
    const int sub = tid_x() & 7;
    uint4 raw[2 * NG];
#pragma unroll
    for (int kk = 0; kk < 2 * NG; kk++) {
        const int gi = piece_group(kk);
        const int r = gi / NG, g = gi % NG;
        raw[kk] = stream_load16(stream_piece(win_a, new_a, (size_t)H * D, W, 64 * i + r, h, D, 64 * g + 8 * sub));
    }
    const int B = p.t.bits[e];
    uint8_t *blk = (kv ? p.v_pool : p.k_pool) + (kv ? p.v_offset : p.k_offset)[e];
    switch (B) {
    case 2: quant_rows<2, NG>(raw, blk, H, h); break;
    case 3: quant_rows<3, NG>(raw, blk, H, h); break;
    case 4: quant_rows<4, NG>(raw, blk, H, h); break;
    case 8: quant_rows<8, NG>(raw, blk, H, h); break;
    default: break;                                 // precondition violation: nothing written
    }
}

// Window: window[u] = T[64k + u] for u < W2.  Workgroups per (slice, row
// chunk, head, sequence), slice g < D/64 the 64-dim group g of K and V, the
// last slice (rope_dim 64) the new tokens' rope rows, which are indexed by
// token position and so never move.  The old window rows read are
// [64k, W) and the rows written [0, W2) (only [W, W2) when k == 0): when
// these overlap, one workgroup per slice moves the rows in ordered rounds of
// WR tokens (a round loads all of its source pieces into registers, waits at
// a barrier, then stores; a round writes [r0, r0+WR) and reads
// [64k + r0, 64k + r0 + WR), so it never writes what a later round reads);
// otherwise every chunk of CR rows is moved by its own workgroup.
constexpr int WR = 192;                              // window rows per round
constexpr int WR_PER = WR * 8 / 256;                 // 16-byte pieces per lane and round
constexpr int CR = 32;                               // rows per chunk: one 16-byte piece per lane
__host__ __device__ __forceinline__ int window_chunks(int window_cap) { return window_cap > CR ? (window_cap + CR - 1) / CR : 1; }

template <int NKV>
__device__ __forceinline__ void window_rounds(const AppendArgs &p, int a, int h, int g, int W, int k, int W2)
{
    const int H = p.t.H, D = p.t.D, tid = tid_x();
    const uint16_t *src_w[2] = {p.k_window + (size_t)a * p.t.window_cap * H * D,
                                NKV > 1 ? p.v_window + (size_t)a * p.t.window_cap * H * D : nullptr};
    const uint16_t *src_n[2] = {p.k_new + (size_t)a * p.n_new * H * D,
                                NKV > 1 ? p.v_new + (size_t)a * p.n_new * H * D : nullptr};
    uint16_t *dst_w[2] = {p.k_window + (size_t)a * p.t.window_cap * H * D,
                          NKV > 1 ? p.v_window + (size_t)a * p.t.window_cap * H * D : nullptr};
    for (int r0 = (k == 0 ? W : 0); r0 < W2; r0 += WR) {
        u32x4 v[WR_PER][NKV];
#pragma unroll
        for (int rep = 0; rep < WR_PER; rep++) {
            const int idx = tid + 256 * rep;
            const int u = min(r0 + (idx >> 3), W2 - 1), col = 8 * (idx & 7);   // clamped: in bounds
#pragma unroll
            for (int kv = 0; kv < NKV; kv++)
                v[rep][kv] = *reinterpret_cast<const u32x4 *>(
                    stream_piece(src_w[kv], src_n[kv], (size_t)H * D, W, 64 * k + u, h, D, 64 * g + col));
        }
        if (k > 0) __syncthreads();                 // every source piece is in registers
#pragma unroll
        for (int rep = 0; rep < WR_PER; rep++) {
            const int idx = tid + 256 * rep;
            const int u = r0 + (idx >> 3), col = 8 * (idx & 7);
            if (u < W2) {
#pragma unroll
                for (int kv = 0; kv < NKV; kv++)
                    *reinterpret_cast<u32x4 *>(dst_w[kv] + ((size_t)u * H + h) * D + 64 * g + col) = v[rep][kv];
            }
        }
    }
}

__global__ __launch_bounds__(256) void append_window(AppendArgs p)
{
    const int RC = window_chunks(p.t.window_cap);
    const int g = wg_x() / RC, c = wg_x() % RC, h = wg_y(), a = wg_z();
    const int H = p.t.H, D = p.t.D, NG = D / 64, R = p.rope_dim;
    const int tid = tid_x();
    int nb, W, k, W2;
    append_plan(p, a, nb, W, k, W2);
    if (p.counts_in_window && wg_x() == 0 && h == 0 && tid == 0) {
        p.n_blocks_out[a] = nb + k;
        if (p.n_window_out) p.n_window_out[a] = W2;
    }
    if (g >= NG) {
        // token W + i of the stream is sequence position 64*nb + W + i
        const size_t rope_tokens = (size_t)64 * p.t.max_blocks + p.t.window_cap;
        const int64_t room = (int64_t)rope_tokens - (64 * (int64_t)nb + W);
        const int n = (int)min((int64_t)p.n_new, room);
        uint16_t *dst = p.rope + ((size_t)a * rope_tokens + (size_t)64 * nb + W) * H * R;
        const uint16_t *src = p.rope_new + (size_t)a * p.n_new * H * R;
        for (int idx = c * 256 + tid; idx < n * 8; idx += RC * 256) {
            const int i = idx >> 3, col = 8 * (idx & 7);
            *reinterpret_cast<uint4 *>(dst + ((size_t)i * H + h) * R + col) =
                *reinterpret_cast<const uint4 *>(src + ((size_t)i * H + h) * R + col);
        }
        return;
    }
    const int nkv = p.v_pool ? 2 : 1;
    if (k > 0 && 64 * k < W && 64 * k < W2) {       // reads and writes overlap
        if (c == 0) {
            if (nkv == 2) window_rounds<2>(p, a, h, g, W, k, W2);
            else window_rounds<1>(p, a, h, g, W, k, W2);
        }
        return;
    }
    const int u = c * CR + (tid >> 3), col = 8 * (tid & 7);
    if (u < (k == 0 ? W : 0) || u >= W2) return;
    for (int kv = 0; kv < nkv; kv++) {
        uint16_t *win_a = (kv ? p.v_window : p.k_window) + (size_t)a * p.t.window_cap * H * D;
        const uint16_t *new_a = (kv ? p.v_new : p.k_new) + (size_t)a * p.n_new * H * D;
        const uint4 v = *reinterpret_cast<const uint4 *>(
            stream_piece(win_a, new_a, (size_t)H * D, W, 64 * k + u, h, D, 64 * g + col));
        *reinterpret_cast<uint4 *>(win_a + ((size_t)u * H + h) * D + 64 * g + col) = v;
    }
}

// New counts, after every slice has read the old ones (a launch of its own
// when the outputs are the counts the kernels read).
__global__ void append_counts(AppendArgs p)
{
    const int a = wg_x() * 256 + tid_x();
    if (a >= p.t.A) return;
    int nb, W, k, W2;
    append_plan(p, a, nb, W, k, W2);
    p.n_blocks_out[a] = nb + k;
    if (p.n_window_out) p.n_window_out[a] = W2;
}

// ---- restore ---------------------------------------------------------------
template <int B>
__device__ __forceinline__ void lane_codes(const uint8_t *gc, int sub, uint32_t c[8])
{
    // This lane's 8 codes occupy stream bits [8B*sub, 8B*sub + 8B) of the group.
    const uint32_t *w = reinterpret_cast<const uint32_t *>(gc);
    uint64_t bitsv;
    if constexpr (B == 8) {
        uint2 p = reinterpret_cast<const uint2 *>(gc)[sub];
        bitsv = (uint64_t)p.x | ((uint64_t)p.y << 32);
    } else if constexpr (B == 4) {
        bitsv = w[sub];
    } else if constexpr (B == 2) {
        bitsv = (w[sub >> 1] >> ((sub & 1) * 16)) & 0xffffu;
    } else {
        int pos = 24 * sub, wi = pos >> 5, o = pos & 31;
        uint64_t lo = w[wi];
        if (o + 24 > 32) lo |= (uint64_t)w[wi + 1] << 32;
        bitsv = (lo >> o) & 0xffffffu;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) c[i] = (uint32_t)(bitsv >> (B * i)) & ((1u << B) - 1u);
}

template <int B, int NG>
__device__ __forceinline__ void restore_block(const uint8_t *__restrict__ blk, int H, int h,
                                              void *dst_blk, int out_f32)
{
    constexpr int D = NG * 64;
    constexpr int CODE_ROW = D * B / 8;
    const int lane = tid_x() & 63, wave = tid_x() >> 6;
    const int sub = lane & 7, gl = lane >> 3;
    const uint8_t *codes = blk + (size_t)h * 64 * CODE_ROW;
    const uint32_t *meta = reinterpret_cast<const uint32_t *>(blk + (size_t)H * 64 * CODE_ROW +
                                                              (size_t)h * 64 * NG * 4);
#pragma unroll 2
    for (int k = 0; k < 2 * NG; k++) {
        const int gi = wave * 8 + gl + 32 * k;
        const int r = gi / NG, g = gi % NG;
        uint32_t c[8];
        lane_codes<B>(codes + (size_t)gi * 8 * B, sub, c);
        const uint32_t m = meta[gi];
        const float sf = f16_bits_to_f32((uint16_t)(m & 0xffffu));
        const float bf = f16_bits_to_f32((uint16_t)(m >> 16));
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; i++) y[i] = __builtin_fmaf((float)c[i], sf, bf);
        const size_t e = ((size_t)r * H + h) * D + g * 64 + sub * 8;
        if (out_f32) {
            u32x4 *o = reinterpret_cast<u32x4 *>(static_cast<float *>(dst_blk) + e);
            stream_store(o, u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                                  __float_as_uint(y[3])});
            stream_store(o + 1, u32x4{__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                                      __float_as_uint(y[7])});
        } else {
            u32x4 o;
            o.x = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
            o.y = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
            o.z = f32_to_bf16_bits(y[4]) | (f32_to_bf16_bits(y[5]) << 16);
            o.w = f32_to_bf16_bits(y[6]) | (f32_to_bf16_bits(y[7]) << 16);
            stream_store(reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(dst_blk) + e), o);
        }
    }
}

// Grid (heads, items, sequences), item j0 + y: the sequence's blocks, then
// its 64-token window tiles.  Heads are on the fastest grid dimension, so
// workgroups dispatched together fill whole token rows of the output.
template <int NG>
__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a)
{
    constexpr int D = NG * 64;
    const int h = wg_x(), s = wg_z();
    const int j = a.j0 + wg_y();
    const int nb = seq_blocks(a.t, s);
    const int H = a.t.H;
    const size_t esz = a.out_f32 ? 4 : 2;
    char *dst_seq = static_cast<char *>(a.dst) + (size_t)s * a.dst_seq_tokens * H * D * esz;
    if (j < nb) {
        const int b = a.t.bits[(size_t)s * a.t.max_blocks + j];
        const uint8_t *blk = a.s.pool + a.s.offset[(size_t)s * a.t.max_blocks + j];
        void *dst_blk = dst_seq + (size_t)j * 64 * H * D * esz;
        switch (b) {
        case 2: restore_block<2, NG>(blk, H, h, dst_blk, a.out_f32); break;
        case 3: restore_block<3, NG>(blk, H, h, dst_blk, a.out_f32); break;
        case 4: restore_block<4, NG>(blk, H, h, dst_blk, a.out_f32); break;
        case 8: restore_block<8, NG>(blk, H, h, dst_blk, a.out_f32); break;
        default: break;
        }
        return;
    }
    // Window tiles: 64 window tokens each, written after the blocks.
    const int wt = j - a.t.max_blocks;
    if (wt < 0) return;
    const int nw = seq_window(a.t, s);
    const int w0 = wt * 64;
    if (w0 >= nw) return;
    const int rows = min(64, nw - w0);
    const uint16_t *win = a.s.window + ((size_t)s * a.t.window_cap + w0) * H * D;
    const size_t tok0 = (size_t)nb * 64 + w0;
    for (int e = tid_x() * 8; e < rows * D; e += 256 * 8) {
        const int r = e / D, d = e % D;
        const uint4 v = *reinterpret_cast<const uint4 *>(win + ((size_t)r * H + h) * D + d);
        const size_t o = ((tok0 + r) * H + h) * D + d;
        if (a.out_f32) {
            u32x4 *p = reinterpret_cast<u32x4 *>(reinterpret_cast<float *>(dst_seq) + o);
            stream_store(p, u32x4{v.x << 16, v.x & 0xffff0000u, v.y << 16, v.y & 0xffff0000u});
            stream_store(p + 1, u32x4{v.z << 16, v.z & 0xffff0000u, v.w << 16, v.w & 0xffff0000u});
        } else {
            stream_store(reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(dst_seq) + o),
                         u32x4{v.x, v.y, v.z, v.w});
        }
    }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &args, hipStream_t s)
{
    if (args.t.max_blocks == 0) return hipSuccess;
    if (args.n_tensors < 1 || args.n_tensors > 2 || (int64_t)args.t.A * args.n_tensors > 65535)
        return hipErrorInvalidValue;
    if (args.t.D % 64 || args.t.D < 64 || args.t.D > 512) return hipErrorInvalidValue;
    QuantArgs a = args;
    for (int64_t j0 = 0; j0 < args.t.max_blocks; j0 += kGridY) {
        a.j0 = (int)j0;
        const int64_t left = args.t.max_blocks - j0;
        dim3 grid(a.t.H, (unsigned)(left < kGridY ? left : kGridY), a.t.A * a.n_tensors);
        switch (a.t.D / 64) {
        case 1: quantize_kernel<1><<<grid, 256, 0, s>>>(a); break;
        case 2: quantize_kernel<2><<<grid, 256, 0, s>>>(a); break;
        case 3: quantize_kernel<3><<<grid, 256, 0, s>>>(a); break;
        case 4: quantize_kernel<4><<<grid, 256, 0, s>>>(a); break;
        case 5: quantize_kernel<5><<<grid, 256, 0, s>>>(a); break;
        case 6: quantize_kernel<6><<<grid, 256, 0, s>>>(a); break;
        case 7: quantize_kernel<7><<<grid, 256, 0, s>>>(a); break;
        default: quantize_kernel<8><<<grid, 256, 0, s>>>(a); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s)
{
    // A call cuts at most (window_cap + n_new - keep) / 64 blocks per sequence.
    const int64_t kmax = a.t.window_cap + (int64_t)a.n_new > a.keep
                             ? (a.t.window_cap + (int64_t)a.n_new - a.keep) / 64 : 0;
    const int64_t kgrid = kmax < a.t.max_blocks ? kmax : a.t.max_blocks;
    const int n_kv = a.v_pool ? 2 : 1;
    if (kgrid * n_kv > 0x7fffffff) return hipErrorInvalidValue;
    if (kgrid > 0) {
        dim3 grid((unsigned)(kgrid * n_kv), a.t.H, a.t.A);
        switch (a.t.D / 64) {
        case 1: append_blocks<1><<<grid, 256, 0, s>>>(a); break;
        case 2: append_blocks<2><<<grid, 256, 0, s>>>(a); break;
        case 3: append_blocks<3><<<grid, 256, 0, s>>>(a); break;
        case 4: append_blocks<4><<<grid, 256, 0, s>>>(a); break;
        case 5: append_blocks<5><<<grid, 256, 0, s>>>(a); break;
        case 6: append_blocks<6><<<grid, 256, 0, s>>>(a); break;
        case 7: append_blocks<7><<<grid, 256, 0, s>>>(a); break;
        case 8: append_blocks<8><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.t.window_cap > 0 || a.rope_dim) {
        dim3 grid((unsigned)((a.t.D / 64 + (a.rope_dim ? 1 : 0)) * window_chunks(a.t.window_cap)), a.t.H, a.t.A);
        append_window<<<grid, 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.counts_in_window) return hipSuccess;
    }
    append_counts<<<(a.t.A + 255) / 256, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &args, hipStream_t s)
{
    const int64_t items = (int64_t)args.t.max_blocks + (args.t.window_cap + 63) / 64;
    if (args.t.D % 64 || args.t.D < 64 || args.t.D > 512) return hipErrorInvalidValue;
    DequantArgs a = args;
    for (int64_t j0 = 0; j0 < items; j0 += kGridY) {
        a.j0 = (int)j0;
        const int64_t left = items - j0;
        dim3 grid(a.t.H, (unsigned)(left < kGridY ? left : kGridY), a.t.A);
        switch (a.t.D / 64) {
        case 1: dequantize_kernel<1><<<grid, 256, 0, s>>>(a); break;
        case 2: dequantize_kernel<2><<<grid, 256, 0, s>>>(a); break;
        case 3: dequantize_kernel<3><<<grid, 256, 0, s>>>(a); break;
        case 4: dequantize_kernel<4><<<grid, 256, 0, s>>>(a); break;
        case 5: dequantize_kernel<5><<<grid, 256, 0, s>>>(a); break;
        case 6: dequantize_kernel<6><<<grid, 256, 0, s>>>(a); break;
        case 7: dequantize_kernel<7><<<grid, 256, 0, s>>>(a); break;
        default: dequantize_kernel<8><<<grid, 256, 0, s>>>(a); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvq
