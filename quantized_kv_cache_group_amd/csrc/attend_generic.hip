// Generic attention over a quantized cache (gfx950): any width mix, window,
// rope part, latent values, causal new tokens.  This is the straightforward
// kernel: it dequantizes each key/value tile to fp32 in LDS and computes
// scores and the value sum on the vector ALUs.  The tuned decode and chunk
// kernels handle the common shapes; this one covers everything else and
// serves as their in-library cross-check.
//
// Semantics (QKVShare, Metodologia: restore the quantized cache to 16-bit
// rows, then ordinary attention; Agent Memory Below the Prompt, Abstract:
// batched attention over several agents' caches and cross-phase chunks):
//   key set of query row (sequence a, query token i, head h):
//     64*n_blocks[a] dequantized tokens, n_window[a] bf16 tokens, and for a
//     chunk the new tokens 0..i; KV head h / G; scores scale * <q, k>.
// Work split: workgroup = (key split, row tile of <= 16 query rows of one KV
// head, sequence).  Each split writes (max, sum, weighted values) partials
// and a merge kernel combines the splits with the usual max-rescaling.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int NT = 256;     // lanes per workgroup
constexpr int RMAX = 16;    // query rows per tile
constexpr int TK = 8;       // keys per LDS tile

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

struct SeqLen {
    int nb, nw, T;
};

__device__ __forceinline__ SeqLen seq_len(const Tables &t, int a)
{
    SeqLen s;
    s.nb = clampi(t.n_blocks[a], 0, t.max_blocks);
    s.nw = t.n_window ? clampi(t.n_window[a], 0, t.window_cap) : 0;
    s.T = 64 * s.nb + s.nw;
    return s;
}

// Dequantized element d (< D) of KV head g, cached token t (< 64*nb).
__device__ __forceinline__ float cached_elem(const Tables &tb, const Store &st, int a, int g, int t, int d)
{
    const int j = t >> 6, r = t & 63;
    const int b = tb.bits[(size_t)a * tb.max_blocks + j];
    const uint8_t *blk = st.pool + st.offset[(size_t)a * tb.max_blocks + j];
    const int D = tb.D, H = tb.H, ng = D >> 6, grp = d >> 6, i = d & 63;
    const size_t code_row = (size_t)D * b / 8;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(blk + ((size_t)g * 64 + r) * code_row +
                                                           (size_t)grp * 8 * b);
    const int pos = b * i, wi = pos >> 5, o = pos & 31;
    uint32_t v = w[wi] >> o;
    if (o + b > 32) v |= w[wi + 1] << (32 - o);
    v &= (1u << b) - 1u;
    const uint32_t m = reinterpret_cast<const uint32_t *>(blk + (size_t)H * 64 * code_row)
        [((size_t)g * 64 + r) * ng + grp];
    return __builtin_fmaf((float)v, f16f((uint16_t)(m & 0xffffu)), f16f((uint16_t)(m >> 16)));
}

struct RowInfo {
    int valid;   // row exists
    int i;       // query token within the sequence
    int h;       // query head
    int lim;     // number of keys the row attends to
};

__device__ __forceinline__ RowInfo row_info(const AttnArgs &p, int g, int tile, int r, int T)
{
    RowInfo ri;
    ri.i = tile * p.tok_per_tile + r / p.G;
    ri.h = g * p.G + r % p.G;
    ri.valid = (r < p.tok_per_tile * p.G) && (ri.i < p.n_qtok);
    ri.lim = p.n_new ? T + ri.i + 1 : T;
    return ri;
}

__global__ __launch_bounds__(NT) void attend_split_generic(AttnArgs p)
{
    extern __shared__ float lds[];
    const int s = blockIdx.x, a = blockIdx.z;
    const int g = blockIdx.y / p.n_row_tiles, tile = blockIdx.y % p.n_row_tiles;
    const SeqLen L = seq_len(p.t, a);
    const int Dk = p.Dk, Dv = p.Dv, D = p.t.D, H = p.t.H;
    const int nrows = p.tok_per_tile * p.G;

    uint16_t *q_s = reinterpret_cast<uint16_t *>(lds);   // [RMAX][Dk] bf16 bits
    float *k_s = lds + RMAX * Dk / 2;       // [TK][Dk]
    float *v_s = k_s + TK * Dk;             // [TK][Dv]
    float *p_s = v_s + (p.v_is_k ? 0 : TK * Dv);   // [RMAX][TK]
    float *alpha_s = p_s + RMAX * TK;       // [RMAX]
    __shared__ int lim_s[RMAX];
    __shared__ int kmax_s;

    if (threadIdx.x == 0) kmax_s = 0;
    __syncthreads();
    if (threadIdx.x < RMAX) {
        RowInfo ri = row_info(p, g, tile, threadIdx.x, L.T);
        lim_s[threadIdx.x] = ri.valid ? ri.lim : 0;
        if (ri.valid) atomicMax(&kmax_s, ri.lim);
    }
    __syncthreads();
    const int k_begin = s * p.split_keys;
    const int k_end = min(k_begin + p.split_keys, kmax_s);
    if (k_begin >= k_end) return;            // no row needs this split

    // Query rows to LDS (bf16 bits; widened exactly when used).
    for (int e = threadIdx.x; e < RMAX * Dk; e += NT) {
        const int r = e / Dk, d = e % Dk;
        uint16_t v = 0;
        if (r < nrows && lim_s[r] > 0) {
            RowInfo ri = row_info(p, g, tile, r, L.T);
            v = p.q[(((size_t)a * p.n_qtok + ri.i) * p.Hq + ri.h) * Dk + d];
        }
        q_s[e] = v;
    }

    float m_run = -INFINITY, l_run = 0.0f;   // held by lane r < RMAX for row r
    constexpr int MAXACC = RMAX * 512 / NT;  // (row, dim) pairs per lane
    float acc[MAXACC];
#pragma unroll
    for (int k = 0; k < MAXACC; k++) acc[k] = 0.0f;
    const int npairs = nrows * Dv;

    for (int t0 = k_begin; t0 < k_end; t0 += TK) {
        __syncthreads();
        // Key tile (and value tile unless values alias the keys).
        for (int e = threadIdx.x; e < TK * Dk; e += NT) {
            const int r = e / Dk, d = e % Dk, t = t0 + r;
            float v = 0.0f;
            if (t < k_end) {
                if (d < D) {
                    if (t < 64 * L.nb) v = cached_elem(p.t, p.k, a, g, t, d);
                    else if (t < L.T) v = bf16f(p.k.window[(((size_t)a * p.t.window_cap + (t - 64 * L.nb)) * H + g) * D + d]);
                    else v = bf16f(p.k_new[(((size_t)a * p.n_new + (t - L.T)) * H + g) * D + d]);
                } else {
                    v = bf16f(p.rope[(((size_t)a * p.rope_tokens + t) * H + g) * p.rope_dim + (d - D)]);
                }
            }
            k_s[e] = v;
        }
        if (!p.v_is_k) {
            for (int e = threadIdx.x; e < TK * Dv; e += NT) {
                const int r = e / Dv, d = e % Dv, t = t0 + r;
                float v = 0.0f;
                if (t < k_end) {
                    if (t < 64 * L.nb) v = cached_elem(p.t, p.v, a, g, t, d);
                    else if (t < L.T) v = bf16f(p.v.window[(((size_t)a * p.t.window_cap + (t - 64 * L.nb)) * H + g) * D + d]);
                    else v = bf16f(p.v_new[(((size_t)a * p.n_new + (t - L.T)) * H + g) * D + d]);
                }
                v_s[e] = v;
            }
        }
        __syncthreads();
        // Scores: lane (r, t) for r < RMAX, t < TK.
        if (threadIdx.x < RMAX * TK) {
            const int r = threadIdx.x / TK, tt = threadIdx.x % TK, t = t0 + tt;
            float sc = -INFINITY;
            if (r < nrows && t < k_end && t < lim_s[r]) {
                float dot = 0.0f;
                for (int d = 0; d < Dk; d++) dot = __builtin_fmaf(bf16f(q_s[r * Dk + d]), k_s[tt * Dk + d], dot);
                sc = dot * p.scale;
            }
            p_s[r * TK + tt] = sc;
        }
        __syncthreads();
        // Online softmax update, one lane per row.
        if (threadIdx.x < RMAX) {
            const int r = threadIdx.x;
            float mt = -INFINITY;
            for (int tt = 0; tt < TK; tt++) mt = fmaxf(mt, p_s[r * TK + tt]);
            const float m_new = fmaxf(m_run, mt);
            float alpha = 1.0f, sum = 0.0f;
            if (m_new != -INFINITY) {
                alpha = expf(m_run - m_new);
                for (int tt = 0; tt < TK; tt++) {
                    const float e = expf(p_s[r * TK + tt] - m_new);
                    p_s[r * TK + tt] = e;
                    sum += e;
                }
            } else {
                for (int tt = 0; tt < TK; tt++) p_s[r * TK + tt] = 0.0f;
            }
            l_run = l_run * alpha + sum;
            m_run = m_new;
            alpha_s[r] = alpha;
        }
        __syncthreads();
        const float *vt = p.v_is_k ? k_s : v_s;
        const int vstride = p.v_is_k ? Dk : Dv;
#pragma unroll
        for (int k = 0; k < MAXACC; k++) {
            const int pi = threadIdx.x + k * NT;
            if (pi < npairs) {
                const int r = pi / Dv, d = pi % Dv;
                float o = acc[k] * alpha_s[r];
                for (int tt = 0; tt < TK; tt++) o = __builtin_fmaf(p_s[r * TK + tt], vt[tt * vstride + d], o);
                acc[k] = o;
            }
        }
    }

    // Partials of the rows that need this split.
    const size_t rstride = (size_t)p.n_splits * (Dv + 2);
#pragma unroll
    for (int k = 0; k < MAXACC; k++) {
        const int pi = threadIdx.x + k * NT;
        if (pi < npairs) {
            const int r = pi / Dv, d = pi % Dv;
            if (k_begin < lim_s[r]) {
                RowInfo ri = row_info(p, g, tile, r, L.T);
                const size_t row = ((size_t)a * p.n_qtok + ri.i) * p.Hq + ri.h;
                p.part[row * rstride + (size_t)s * (Dv + 2) + 2 + d] = acc[k];
            }
        }
    }
    if ((int)threadIdx.x < nrows && k_begin < lim_s[threadIdx.x]) {
        RowInfo ri = row_info(p, g, tile, threadIdx.x, L.T);
        const size_t row = ((size_t)a * p.n_qtok + ri.i) * p.Hq + ri.h;
        p.part[row * rstride + (size_t)s * (Dv + 2) + 0] = m_run;
        p.part[row * rstride + (size_t)s * (Dv + 2) + 1] = l_run;
    }
}

// One workgroup per output row: combine the splits that cover its keys.
__global__ __launch_bounds__(256) void attend_merge_generic(AttnArgs p)
{
    const size_t row = blockIdx.x;
    const int h = (int)(row % p.Hq);
    const int i = (int)((row / p.Hq) % p.n_qtok);
    const int a = (int)(row / ((size_t)p.Hq * p.n_qtok));
    const SeqLen L = seq_len(p.t, a);
    const int lim = p.n_new ? L.T + i + 1 : L.T;
    const int ns = (lim + p.split_keys - 1) / p.split_keys;
    const float *pr = p.part + row * (size_t)p.n_splits * (p.Dv + 2);
    float M = -INFINITY;
    for (int s = 0; s < ns; s++) M = fmaxf(M, pr[(size_t)s * (p.Dv + 2)]);
    float Lsum = 0.0f;
    for (int s = 0; s < ns; s++) {
        const float m = pr[(size_t)s * (p.Dv + 2)];
        if (m != -INFINITY) Lsum += expf(m - M) * pr[(size_t)s * (p.Dv + 2) + 1];
    }
    float *o = p.out + row * p.Dv;
    (void)h;
    for (int d = threadIdx.x; d < p.Dv; d += blockDim.x) {
        float acc = 0.0f;
        for (int s = 0; s < ns; s++) {
            const float m = pr[(size_t)s * (p.Dv + 2)];
            if (m != -INFINITY) acc += expf(m - M) * pr[(size_t)s * (p.Dv + 2) + 2 + d];
        }
        o[d] = (Lsum > 0.0f) ? acc / Lsum : 0.0f;
    }
}

}  // namespace

void generic_plan(int max_keys, int n_new, int G, int *tok_per_tile, int *split_keys, int *n_splits)
{
    *tok_per_tile = n_new ? (RMAX / G) : 1;
    int sk = n_new ? 2048 : 256;
    *split_keys = sk;
    *n_splits = max_keys > 0 ? (max_keys + sk - 1) / sk : 1;
}

hipError_t launch_attend_generic(const AttnArgs &p, hipStream_t s)
{
    // Dk is even (a multiple of 64 plus 0 or 64), so the bf16 query rows
    // take RMAX*Dk/2 floats of space.
    const size_t lds = sizeof(float) * ((size_t)RMAX * p.Dk / 2 + (size_t)TK * p.Dk +
                                        (p.v_is_k ? 0 : (size_t)TK * p.Dv) + (size_t)RMAX * TK + RMAX);
    dim3 grid(p.n_splits, p.t.H * p.n_row_tiles, p.t.A);
    hipLaunchKernelGGL(attend_split_generic, grid, dim3(NT), lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t rows = (size_t)p.t.A * p.n_qtok * p.Hq;
    hipLaunchKernelGGL(attend_merge_generic, dim3((unsigned)rows), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvq
