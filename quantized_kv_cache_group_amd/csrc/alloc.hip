// Width allocation: block sensitivity on the GPU, budgeted greedy choice on
// the host (Coordinated Mixed-Precision KV Cache Quantization, arXiv
// 2611.10096, Abstract: sensitivity from a local attention-error bound using
// recent queries, keys and values; widths chosen jointly under a shared byte
// budget, for newly quantized blocks only).
//
// The bound (derived from the per-group reconstruction bound s/2, s = range
// / (2^b - 1)): for query head h (KV head g), a 64-token block quantized at
// width b changes attention restricted to the block by at most, to first
// order, c(b) * S_h with c(b) = 1 / (2 (2^b - 1)) and
//     S_h = 2 Vmax scale max_t sum_grp rK[t][grp] sum_{d in grp} |q_h[d]|
//           + 8 max_t sqrt(sum_grp rV[t][grp]^2)
// (rK, rV: max - min of a group, Vmax: the largest value-row norm of the
// block; 8 = sqrt(64) elements per group).  The block's sensitivity is
// S = sum_h S_h; the error of width b is estimated as c(b) S.
#include "kvq_internal.h"

#include <algorithm>
#include <queue>
#include <vector>

namespace kvq {
namespace {

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

constexpr int MAX_HQ = 1024;                         // query heads per workgroup pass
constexpr int MAX_QA = 8192;                         // Hq * (D/64) sums of |q| in LDS

// One workgroup per (block i, sequence a); a thread per (token t, KV head g)
// pair computes the group ranges of its K and V rows and the V row norm,
// then folds the per-head maxima into LDS (non-negative floats compare as
// integers).
__global__ __launch_bounds__(256) void block_sensitivity(const uint16_t *k, const uint16_t *v, int64_t seq_tokens,
                                                         int H, int D, const uint16_t *q, int Hq, float scale,
                                                         float *S, int n_blocks)
{
    __shared__ float qa[MAX_QA];                     // [h][grp] sum |q|
    __shared__ unsigned kmax[MAX_HQ];                // per query head: max_t sum_grp rK * qa
    __shared__ unsigned vstat[2 * MAX_HQ];           // per KV head: max_t |v_t|, max_t sqrt(sum rV^2)
    const int i = blockIdx.x, a = blockIdx.y, tid = threadIdx.x;
    const int NG = D / 64, G = Hq / H;
    for (int e = tid; e < Hq * NG; e += 256) {
        const int h = e / NG, grp = e % NG;
        const uint16_t *qr = q + ((size_t)a * Hq + h) * D + 64 * grp;
        float s = 0.f;
        for (int d = 0; d < 64; d++) s += fabsf(__uint_as_float((uint32_t)qr[d] << 16));
        qa[e] = s;
    }
    for (int e = tid; e < Hq; e += 256) kmax[e] = 0u;
    for (int e = tid; e < 2 * H; e += 256) vstat[e] = 0u;
    __syncthreads();
    for (int pr = tid; pr < 64 * H; pr += 256) {
        const int t = pr / H, g = pr % H;
        const size_t rowoff = (((size_t)a * seq_tokens + (size_t)64 * i + t) * H + g) * D;
        const uint4 *kr = reinterpret_cast<const uint4 *>(k + rowoff);
        const uint4 *vr = reinterpret_cast<const uint4 *>(v + rowoff);
        float rk[8], vss = 0.f, vn = 0.f;            // NG <= 8
        for (int grp = 0; grp < NG; grp++) {
            float kmn = INFINITY, kmx = -INFINITY, vmn = INFINITY, vmx = -INFINITY;
            for (int c = 0; c < 8; c++) {
                const uint4 kw = kr[8 * grp + c], vw = vr[8 * grp + c];
                const uint32_t ka[4] = {kw.x, kw.y, kw.z, kw.w}, va[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const float k0 = bf16lo(ka[u]), k1 = bf16hi(ka[u]);
                    const float v0 = bf16lo(va[u]), v1 = bf16hi(va[u]);
                    kmn = fminf(kmn, fminf(k0, k1));
                    kmx = fmaxf(kmx, fmaxf(k0, k1));
                    vmn = fminf(vmn, fminf(v0, v1));
                    vmx = fmaxf(vmx, fmaxf(v0, v1));
                    vn = __builtin_fmaf(v0, v0, __builtin_fmaf(v1, v1, vn));
                }
            }
            rk[grp] = kmx - kmn;
            vss = __builtin_fmaf(vmx - vmn, vmx - vmn, vss);
        }
        for (int hh = 0; hh < G; hh++) {
            const int h = g * G + hh;
            float sk = 0.f;
            for (int grp = 0; grp < NG; grp++) sk = __builtin_fmaf(rk[grp], qa[h * NG + grp], sk);
            atomicMax(&kmax[h], __float_as_uint(sk));
        }
        atomicMax(&vstat[2 * g], __float_as_uint(sqrtf(vn)));
        atomicMax(&vstat[2 * g + 1], __float_as_uint(sqrtf(vss)));
    }
    __syncthreads();
    if (tid == 0) {
        float total = 0.f;
        for (int h = 0; h < Hq; h++) {
            const int g = h / G;
            total += 2.0f * __uint_as_float(vstat[2 * g]) * fabsf(scale) * __uint_as_float(kmax[h]) +
                     8.0f * __uint_as_float(vstat[2 * g + 1]);
        }
        S[(size_t)a * n_blocks + i] = total;
    }
}

// The same statistics from a coalesced stream: a block's K (and V) rows are
// one contiguous region of 64*H*D bf16, read as units of one 64-element
// group, 8 lanes x 16 bytes per unit, with UNROLL units' K and V loads in
// flight per lane.  Group range and square sums go to LDS per (row, group);
// then a thread per (token, KV head) row folds its groups in order.  LDS
// (dynamic): qa [Hq][NG], rk / rv2 / vsq [64 H][NG], kmax [Hq], vstat [2H].
constexpr int SENS_UNROLL = 8;

__device__ __forceinline__ float octet_min(float x)
{
    x = fminf(x, __shfl_xor(x, 1));
    x = fminf(x, __shfl_xor(x, 2));
    return fminf(x, __shfl_xor(x, 4));
}
__device__ __forceinline__ float octet_max(float x)
{
    x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 2));
    return fmaxf(x, __shfl_xor(x, 4));
}
__device__ __forceinline__ float octet_sum(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    return x + __shfl_xor(x, 4);
}

__global__ __launch_bounds__(256) void block_sensitivity_stream(const uint16_t *k, const uint16_t *v,
                                                                int64_t seq_tokens, int H, int D, const uint16_t *q,
                                                                int Hq, float scale, float *S, int n_blocks)
{
    extern __shared__ float smem[];
    const int i = blockIdx.x, a = blockIdx.y, tid = threadIdx.x;
    const int NG = D / 64, G = Hq / H, NU = 64 * H * NG;
    const int oct = tid >> 3, sub = tid & 7;
    float *qa = smem, *rk = qa + Hq * NG, *rv2 = rk + NU, *vsq = rv2 + NU;
    unsigned *kmax = reinterpret_cast<unsigned *>(vsq + NU), *vstat = kmax + Hq;

    for (int u = oct; u < Hq * NG; u += 32) {         // sum |q| per (head, group)
        const uint4 w = *reinterpret_cast<const uint4 *>(q + (size_t)a * Hq * D + (size_t)u * 64 + 8 * sub);
        const uint32_t wa[4] = {w.x, w.y, w.z, w.w};
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 4; c++) s += fabsf(bf16lo(wa[c])) + fabsf(bf16hi(wa[c]));
        s = octet_sum(s);
        if (sub == 0) qa[u] = s;
    }
    for (int e = tid; e < Hq; e += 256) kmax[e] = 0u;
    for (int e = tid; e < 2 * H; e += 256) vstat[e] = 0u;

    const size_t base = ((size_t)a * seq_tokens + (size_t)64 * i) * H * D + 8 * sub;
    const uint4 *kb = reinterpret_cast<const uint4 *>(k + base);
    const uint4 *vb = reinterpret_cast<const uint4 *>(v + base);
    for (int u0 = oct; u0 < NU; u0 += 32 * SENS_UNROLL) {
        uint4 kw[SENS_UNROLL], vw[SENS_UNROLL];
#pragma unroll
        for (int r = 0; r < SENS_UNROLL; r++) {
            const int u = min(u0 + 32 * r, NU - 1);   // past the end: re-read the last unit, not stored
            kw[r] = kb[(size_t)u * 8];
            vw[r] = vb[(size_t)u * 8];
        }
#pragma unroll
        for (int r = 0; r < SENS_UNROLL; r++) {
            const uint32_t ka[4] = {kw[r].x, kw[r].y, kw[r].z, kw[r].w};
            const uint32_t va[4] = {vw[r].x, vw[r].y, vw[r].z, vw[r].w};
            float kmn = INFINITY, kmx = -INFINITY, vmn = INFINITY, vmx = -INFINITY, vs = 0.f;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const float k0 = bf16lo(ka[c]), k1 = bf16hi(ka[c]);
                const float v0 = bf16lo(va[c]), v1 = bf16hi(va[c]);
                kmn = fminf(kmn, fminf(k0, k1));
                kmx = fmaxf(kmx, fmaxf(k0, k1));
                vmn = fminf(vmn, fminf(v0, v1));
                vmx = fmaxf(vmx, fmaxf(v0, v1));
                vs = __builtin_fmaf(v0, v0, __builtin_fmaf(v1, v1, vs));
            }
            kmn = octet_min(kmn);
            kmx = octet_max(kmx);
            vmn = octet_min(vmn);
            vmx = octet_max(vmx);
            vs = octet_sum(vs);
            const int u = u0 + 32 * r;
            if (sub == 0 && u < NU) {
                rk[u] = kmx - kmn;
                rv2[u] = (vmx - vmn) * (vmx - vmn);
                vsq[u] = vs;
            }
        }
    }
    __syncthreads();
    for (int row = tid; row < 64 * H; row += 256) {   // row = token * H + KV head
        const int g = row % H;
        float vn = 0.f, vss = 0.f;
        for (int grp = 0; grp < NG; grp++) {
            vn += vsq[row * NG + grp];
            vss += rv2[row * NG + grp];
        }
        atomicMax(&vstat[2 * g], __float_as_uint(sqrtf(vn)));
        atomicMax(&vstat[2 * g + 1], __float_as_uint(sqrtf(vss)));
        for (int hh = 0; hh < G; hh++) {
            const int h = g * G + hh;
            float sk = 0.f;
            for (int grp = 0; grp < NG; grp++) sk = __builtin_fmaf(rk[row * NG + grp], qa[h * NG + grp], sk);
            atomicMax(&kmax[h], __float_as_uint(sk));
        }
    }
    __syncthreads();
    if (tid == 0) {
        float total = 0.f;
        for (int h = 0; h < Hq; h++) {
            const int g = h / G;
            total += 2.0f * __uint_as_float(vstat[2 * g]) * fabsf(scale) * __uint_as_float(kmax[h]) +
                     8.0f * __uint_as_float(vstat[2 * g + 1]);
        }
        S[(size_t)a * n_blocks + i] = total;
    }
}

size_t sensitivity_stream_lds(int H, int D, int Hq)
{
    const size_t NG = (size_t)D / 64;
    return 4 * ((size_t)Hq * NG + 3 * 64 * (size_t)H * NG + (size_t)Hq + 2 * (size_t)H);
}

}  // namespace

bool sensitivity_supported(int H, int D, int Hq) { return Hq <= MAX_HQ && Hq * (D / 64) <= MAX_QA && D / 64 <= 8 && H <= MAX_HQ; }

hipError_t launch_sensitivity(const uint16_t *k, const uint16_t *v, int A, int64_t seq_tokens, int n_blocks, int H,
                              int D, const uint16_t *q, int Hq, float scale, float *S, hipStream_t s)
{
    if (n_blocks == 0) return hipSuccess;
    const size_t lds = sensitivity_stream_lds(H, D, Hq);
    if (lds <= 48 * 1024 && ((uintptr_t)q & 15) == 0) {   // the stream reads q 16 bytes at a time
        block_sensitivity_stream<<<dim3(n_blocks, A), 256, lds, s>>>(k, v, seq_tokens, H, D, q, Hq, scale, S,
                                                                     n_blocks);
        return hipGetLastError();
    }
    block_sensitivity<<<dim3(n_blocks, A), 256, 0, s>>>(k, v, seq_tokens, H, D, q, Hq, scale, S, n_blocks);
    return hipGetLastError();
}

// Greedy: every block starts at 2 bits; repeatedly take the (block, next
// width) step with the largest S (c(b) - c(b')) per extra byte (equal
// ratios: lower block index first) among the steps that still fit.  A step
// that does not fit now never fits later (the bytes used only grow), so the
// heap simply drops it, and the block's later steps with it.
int allocate_widths(const float *S, int64_t n, uint64_t bytes2, uint64_t bytes3, uint64_t bytes4,
                    uint64_t bytes8, uint64_t budget, uint8_t *widths)
{
    static const int W[4] = {2, 3, 4, 8};
    const uint64_t bytes[4] = {bytes2, bytes3, bytes4, bytes8};
    if (n < 0 || (n > 0 && bytes2 > budget / (uint64_t)n)) return -1;   // all-2-bit size exceeds the budget
    uint64_t used = (uint64_t)n * bytes2;
    auto cost = [](int b) { return 1.0 / (2.0 * (double)((1 << b) - 1)); };
    struct Step {
        double r;
        int64_t i;
        int w;                                       // index of the current width
    };
    auto worse = [](const Step &x, const Step &y) { return x.r < y.r || (x.r == y.r && x.i > y.i); };
    std::priority_queue<Step, std::vector<Step>, decltype(worse)> pq(worse);
    std::vector<int> wi((size_t)n, 0);
    auto push = [&](int64_t i) {
        const int w = wi[(size_t)i];
        if (w + 1 >= 4) return;
        const double extra = (double)(bytes[w + 1] - bytes[w]);
        pq.push(Step{(double)S[i] * (cost(W[w]) - cost(W[w + 1])) / extra, i, w});
    };
    for (int64_t i = 0; i < n; i++) push(i);
    while (!pq.empty()) {
        const Step st = pq.top();
        pq.pop();
        const uint64_t extra = bytes[st.w + 1] - bytes[st.w];
        if (used + extra > budget) continue;
        used += extra;
        wi[(size_t)st.i] = st.w + 1;
        push(st.i);
    }
    for (int64_t i = 0; i < n; i++) widths[i] = (uint8_t)W[wi[(size_t)i]];
    return 0;
}

}  // namespace kvq
