// attn_combine.hip -- the split-K (flash decoding) merge (Ferrum Infer README,
// "Key Optimizations": split-K for long-context decode).
//
// Split s of a query row left (m_s, l_s, o_s): its running max in log2 units,
// the sum of 2^(score - m_s) over its keys and the matching unnormalised
// weighted sum of V.  The row's result is
//     M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// over all S splits: a split with no key of the sequence, or none the row
// can see, carries l_s = 0, o_s = 0 and a very negative m_s, and drops out.
// Nothing here depends on the sequence lengths, so the merge costs one
// memory round trip.
//
// Fixed summation order, so results are bitwise reproducible.  Rows of
// padding tokens past a ragged chunk are left as they are.
#include "kvd_internal.h"

namespace kvd {
namespace {

// Up to eight splits (the common case), each thread reads everything it
// needs in one go; beyond that, one workgroup of COMBINE_THREADS per query
// row forms the split weights 2^(m_s - M) / sum once in LDS (lanes over
// splits, wave reductions), then each thread sums its splits with
// independent loads in flight.
constexpr int COMBINE_THREADS = 128;
constexpr int MAX_STAGED_SPLITS = 1024;

// Query row (b*T + t)*Hq + h belongs to a padding token of a ragged chunk
// (t >= q_lens[b]): its output is left as it is.
__device__ inline bool is_padding(const CacheView& c, size_t qrow) {
    if (!c.q_lens) return false;
    const size_t bt = qrow / c.Hq;
    return (int)(bt % c.T) >= c.q_lens[bt / c.T];
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Up to eight splits: D/4 threads a row, one float4 of it each, and as many
// rows as fill 256 threads in one workgroup (the same arithmetic as above,
// element by element).
constexpr int ROWS_THREADS = 256;
constexpr int ROWS_MAX_SPLITS = 8;

__global__ __launch_bounds__(ROWS_THREADS) void attn_combine_rows_kernel(AttnArgs a) {
    const CacheView& c = a.c;
    const int lq = __builtin_ctz(c.D) - 2;                 // threads a row: D / 4
    const int rpw = ROWS_THREADS >> lq;                    // rows a workgroup
    const size_t rows = (size_t)c.B * c.T * c.Hq;
    const size_t qrow = (size_t)blockIdx.x * rpw + (threadIdx.x >> lq);
    const int e4 = threadIdx.x & ((1 << lq) - 1);
    if (qrow >= rows || is_padding(c, qrow)) return;
    const int n = a.num_splits;
    const float2* ml = (const float2*)(a.part_ml + qrow * n * 2);
    const float4* po = (const float4*)(a.part_o + qrow * n * c.D) + e4;
    float2 w[ROWS_MAX_SPLITS];
    float4 o[ROWS_MAX_SPLITS];
#pragma unroll
    for (int s = 0; s < ROWS_MAX_SPLITS; ++s)
        if (s < n) {
            w[s] = ml[s];
            o[s] = po[(size_t)s * (c.D >> 2)];
        }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < ROWS_MAX_SPLITS; ++s)
        if (s < n) M = fmaxf(M, w[s].x);
    float Ls = 0.0f;
    float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int s = 0; s < ROWS_MAX_SPLITS; ++s)
        if (s < n) {
            const float f = exp2f(w[s].x - M);
            Ls += w[s].y * f;
            O.x += o[s].x * f;
            O.y += o[s].y * f;
            O.z += o[s].z * f;
            O.w += o[s].w * f;
        }
    *(float4*)(a.out + qrow * c.D + 4 * e4) =
        make_float4(finish_out(O.x, Ls), finish_out(O.y, Ls), finish_out(O.z, Ls), finish_out(O.w, Ls));
    if (a.lse && e4 == 0) a.lse[qrow] = finish_lse(M, Ls);
}

__global__ __launch_bounds__(COMBINE_THREADS) void attn_combine_kernel(AttnArgs a) {
    __shared__ float sm_w[MAX_STAGED_SPLITS];
    __shared__ float sm_red[2];
    const CacheView& c = a.c;
    const size_t qrow = blockIdx.x;                     // (b*T + t)*Hq + h
    if (is_padding(c, qrow)) return;
    const int S = a.num_splits;
    const int n = S;
    const float* ml = a.part_ml + qrow * S * 2;
    const float* po = a.part_o + qrow * S * c.D;

    if (threadIdx.x < 64) {
        // wave 0: the max and the weighted sum over splits, 64 at a time
        float M = -INFINITY;
        for (int s = threadIdx.x; s < n; s += 64) M = fmaxf(M, ml[2 * s]);
        M = wave_max(M);
        float Ls = 0.0f;
        for (int s = threadIdx.x; s < n; s += 64) {
            const float w = exp2f(ml[2 * s] - M);
            Ls += ml[2 * s + 1] * w;
            if (s < MAX_STAGED_SPLITS) sm_w[s] = w;
        }
        Ls = wave_sum(Ls);
        if (threadIdx.x == 0) {
            sm_red[0] = M;
            sm_red[1] = Ls > 0.0f ? 1.0f / Ls : 0.0f;
            if (a.lse) a.lse[qrow] = finish_lse(M, Ls);
        }
    }
    __syncthreads();
    const float M = sm_red[0], inv = sm_red[1];
    for (int d = threadIdx.x; d < c.D; d += COMBINE_THREADS) {
        float O = 0.0f;
#pragma unroll 8
        for (int s = 0; s < n; ++s) {
            const float w = s < MAX_STAGED_SPLITS ? sm_w[s] : exp2f(ml[2 * s] - M);
            O += po[(size_t)s * c.D + d] * w;
        }
        a.out[qrow * c.D + d] = O * inv;
    }
}

// Merge of context-parallel partials: one workgroup per row.  The parts'
// weights are exp(lse_p - M) (M = max_p lse_p), their sum S gives
// LSE = M + log S, and each element is the weighted sum over the parts with a
// nonzero weight (a part that saw no key is never used), scaled by 1/S.
// Beyond eight parts, wave 0 forms the weights in LDS first.  Fixed
// summation order.
constexpr int MAX_PARTS = 4096;

// Few parts (the usual count: one per GPU of a group): every thread loads all
// the parts' lse and its elements of all the parts at once, one memory round
// trip; the same weights, and parts of weight 0 are loaded but never used.
template <int NMAX>
__device__ inline bool merge_small(int n, int64_t rows, int D, const float* outs, const float* lses,
                                   float* out, float* lse_out) {
    if (n > NMAX) return false;
    const int64_t row = blockIdx.x;
    float l[NMAX];
#pragma unroll
    for (int p = 0; p < NMAX; ++p)
        if (p < n) l[p] = lses[p * rows + row];
    for (int d = threadIdx.x; d < D; d += COMBINE_THREADS) {
        float x[NMAX];
#pragma unroll
        for (int p = 0; p < NMAX; ++p)
            if (p < n) x[p] = outs[((size_t)p * rows + row) * D + d];
        float M = -INFINITY;
#pragma unroll
        for (int p = 0; p < NMAX; ++p)
            if (p < n) M = fmaxf(M, l[p]);
        float S = 0.0f, o = 0.0f;
#pragma unroll
        for (int p = 0; p < NMAX; ++p)
            if (p < n) {
                const float w = M == -INFINITY ? 0.0f : expf(l[p] - M);
                S += w;
                if (w > 0.0f) o += w * x[p];
            }
        out[(size_t)row * D + d] = o * (S > 0.0f ? 1.0f / S : 0.0f);
        if (lse_out && d == 0) lse_out[row] = S > 0.0f ? M + logf(S) : -INFINITY;
    }
    return true;
}

__global__ __launch_bounds__(COMBINE_THREADS) void merge_partials_kernel(int n, int64_t rows, int D,
                                                                        const float* outs,
                                                                        const float* lses, float* out,
                                                                        float* lse_out) {
    __shared__ float sm_w[MAX_PARTS];
    __shared__ float sm_red[2];
    if (merge_small<8>(n, rows, D, outs, lses, out, lse_out)) return;
    const int64_t row = blockIdx.x;
    if (threadIdx.x < 64) {
        float M = -INFINITY;
        for (int p = threadIdx.x; p < n; p += 64) M = fmaxf(M, lses[p * rows + row]);
        M = wave_max(M);
        float S = 0.0f;
        for (int p = threadIdx.x; p < n; p += 64) {
            const float w = M == -INFINITY ? 0.0f : expf(lses[p * rows + row] - M);
            sm_w[p] = w;
            S += w;
        }
        S = wave_sum(S);
        if (threadIdx.x == 0) {
            sm_red[0] = S > 0.0f ? M + logf(S) : -INFINITY;
            sm_red[1] = S > 0.0f ? 1.0f / S : 0.0f;
        }
    }
    __syncthreads();
    if (lse_out && threadIdx.x == 0) lse_out[row] = sm_red[0];
    const float inv = sm_red[1];
    for (int d = threadIdx.x; d < D; d += COMBINE_THREADS) {
        float o = 0.0f;
        for (int p = 0; p < n; ++p)
            if (sm_w[p] > 0.0f) o += sm_w[p] * outs[((size_t)p * rows + row) * D + d];
        out[(size_t)row * D + d] = o * inv;
    }
}

}  // namespace

hipError_t launch_merge_partials(int n_parts, int64_t rows, int D, const float* outs, const float* lses,
                                 float* out, float* lse_out, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(merge_partials_kernel, dim3((unsigned)rows), dim3(COMBINE_THREADS), 0, s, n_parts,
                       rows, D, outs, lses, out, lse_out);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s) {
    const size_t rows = (size_t)a.c.B * a.c.T * a.c.Hq;
    if (rows == 0) return hipSuccess;
    if (a.num_splits <= ROWS_MAX_SPLITS) {
        const size_t rpw = ROWS_THREADS / (a.c.D / 4);
        hipLaunchKernelGGL(attn_combine_rows_kernel, dim3((unsigned)((rows + rpw - 1) / rpw)),
                           dim3(ROWS_THREADS), 0, s, a);
    } else {
        hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)rows), dim3(COMBINE_THREADS), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kvd
