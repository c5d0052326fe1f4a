// attn_combine.hip -- the split-K (flash decoding) merge (Ferrum Infer README,
// "Key Optimizations": split-K for long-context decode).
//
// Split s of a query row left (m_s, l_s, o_s): its running max in log2 units,
// the sum of 2^(score - m_s) over its keys and the matching unnormalised
// weighted sum of V.  The row's result is
//     M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// over the splits that hold keys of this sequence (split s exists when
// s * split_keys < seq_lens[b]).  Splits whose keys the row cannot see carry
// l_s = 0 and a very negative m_s, and drop out.
//
// One 64-lane workgroup per query row; lanes stride over the head dimension.
// Fixed summation order, so results are bitwise reproducible.
#include "kvd_internal.h"

namespace kvd {
namespace {

__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
    const CacheView& c = a.c;
    const size_t qrow = blockIdx.x;                     // (b*T + t)*Hq + h
    const int b = (int)(qrow / ((size_t)c.T * c.Hq));
    const int L = c.seq_lens[b];
    const int S = a.num_splits;
    const int n = min(S, (L + a.split_keys - 1) / a.split_keys);
    const float* ml = a.part_ml + qrow * S * 2;
    const float* po = a.part_o + qrow * S * c.D;

    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, ml[2 * s]);
    float Ls = 0.0f;
    for (int s = 0; s < n; ++s) Ls += ml[2 * s + 1] * exp2f(ml[2 * s] - M);
    const float inv = 1.0f / Ls;
    for (int d = threadIdx.x; d < c.D; d += 64) {
        float O = 0.0f;
        for (int s = 0; s < n; ++s) O += po[(size_t)s * c.D + d] * exp2f(ml[2 * s] - M);
        a.out[qrow * c.D + d] = O * inv;
    }
}

}  // namespace

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s) {
    const size_t rows = (size_t)a.c.B * a.c.T * a.c.Hq;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)rows), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvd
