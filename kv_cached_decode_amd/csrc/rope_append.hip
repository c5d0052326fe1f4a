// rope_append.hip -- RoPE of the new q/k at each token's absolute position and
// the paged append of the new K/V rows (ferric-core generate.rs `step_gpu`:
// `rope_off_t` then the cache append; Ferrum Infer README: batched RoPE with
// per-item positions, paged KV through a block table).
//
// One workgroup per new token (b, t).  The token's position is
// seq_lens[b] - T + t.  The D/2 rotation angles pos * base^(-2i/D) are
// evaluated once per token in fp64 and shared through LDS; every head's pair
// is then rotated in fp64 and rounded once: to fp32 for q_rot and an fp32
// cache, to bf16 (round to nearest even) for a bf16 cache.  The volume is
// tiny (B*T*(Hq + 2*Hkv)*D elements), so the kernel is latency-bound and is
// kept simple: coalesced loads and stores along the head dimension.
#include "bf16_round.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

__device__ inline void pair_of(int i, int half, int interleaved, int& ia, int& ic) {
    if (interleaved) { ia = 2 * i; ic = 2 * i + 1; }
    else             { ia = i;     ic = i + half; }
}

__device__ inline void rotate(double x, double y, double c, double s, double& xr, double& yr) {
#pragma clang fp contract(off)
    xr = x * c - y * s;
    yr = x * s + y * c;
}

__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
    __shared__ double cs[128];
    __shared__ double sn[128];
    const CacheView& c = a.c;
    const int token = blockIdx.x;
    const int b = token / c.T, t = token - b * c.T;
    const int D = c.D, half = D >> 1;
    const int pos = c.seq_lens[b] - c.T + t;

    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        double theta = pow(a.base, -2.0 * (double)i / (double)D);
        double phi = (double)pos * theta;
        cs[i] = cos(phi);
        sn[i] = sin(phi);
    }
    __syncthreads();

    // queries -> q_rot (fp32); q and q_rot may alias: each pair is read and
    // written by the same thread.
    const float* q = a.q + (size_t)token * c.Hq * D;
    float* qr = a.q_rot + (size_t)token * c.Hq * D;
    for (int w = threadIdx.x; w < c.Hq * half; w += blockDim.x) {
        int h = w / half, i = w - h * half, ia, ic;
        pair_of(i, half, a.interleaved, ia, ic);
        double xr, yr;
        rotate(q[h * D + ia], q[h * D + ic], cs[i], sn[i], xr, yr);
        qr[h * D + ia] = (float)xr;
        qr[h * D + ic] = (float)yr;
    }

    // the cache slot of this token
    const int blk = c.table[(size_t)b * c.max_blocks + (pos >> c.log2_bs)];
    const int off = pos & ((1 << c.log2_bs) - 1);
    const size_t head_stride = (size_t)D << c.log2_bs;                 // one head of a block
    const size_t slot = ((size_t)blk * c.Hkv << c.log2_bs) * D + (size_t)off * D;
    const float* k = a.k + (size_t)token * c.Hkv * D;
    const float* v = a.v + (size_t)token * c.Hkv * D;

    for (int w = threadIdx.x; w < c.Hkv * half; w += blockDim.x) {
        int h = w / half, i = w - h * half, ia, ic;
        pair_of(i, half, a.interleaved, ia, ic);
        double xr, yr;
        rotate(k[h * D + ia], k[h * D + ic], cs[i], sn[i], xr, yr);
        size_t base = slot + h * head_stride;
        if (a.kv_bf16) {
            uint16_t* kc = (uint16_t*)c.k;
            kc[base + ia] = bf16_from_f64(xr);
            kc[base + ic] = bf16_from_f64(yr);
        } else {
            float* kc = (float*)c.k;
            kc[base + ia] = (float)xr;
            kc[base + ic] = (float)yr;
        }
    }
    for (int w = threadIdx.x; w < c.Hkv * D; w += blockDim.x) {
        int h = w / D, d = w - h * D;
        size_t idx = slot + h * head_stride + d;
        if (a.kv_bf16) ((uint16_t*)c.v)[idx] = bf16_from_f32(v[w]);
        else           ((float*)c.v)[idx] = v[w];
    }
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s) {
    const int tokens = a.c.B * a.c.T;
    if (tokens == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_append_kernel, dim3(tokens), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvd
