// stream_probe.hip -- a plain streaming-read kernel: what the HBM delivers in
// practice to a kernel that only reads, at a given grid shape.  Measurement
// only, not a step of the decode path: the decode kernels read the cache at
// close to this rate at best, so their achieved bandwidth is reported as a
// fraction of it beside the fraction of the 8 TB/s peak.
//
// Workgroup w reads its own contiguous share of the buffer, 16 bytes per lane
// per load, UNROLL loads in flight per lane per round (nontemporal, as the
// decode kernels load the cache), folding everything it reads into one word.
// The word is stored only when it equals a fixed pattern, so the loads
// cannot be dropped and nothing is written in practice.
#include "kvd_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL>
__global__ __launch_bounds__(1024) void stream_read_kernel(const u32x4* __restrict__ src, long long n,
                                                            unsigned* __restrict__ sink) {
    const long long per = (n + gridDim.x - 1) / gridDim.x;
    const long long lo = (long long)blockIdx.x * per;
    const long long hi = lo + per < n ? lo + per : n;
    const int stride = blockDim.x;
    unsigned acc = 0;
    long long i = lo + threadIdx.x;
    for (; i + (long long)(UNROLL - 1) * stride < hi; i += (long long)UNROLL * stride) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + (long long)u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" int32_t kvd_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups,
                                         int32_t threads, int32_t unroll, void* sink, void* stream) {
    if (!buf || !sink) return 1;
    if (((uintptr_t)buf & 15) || ((uintptr_t)sink & 3) || bytes % 16 != 0) return 2;
    if (workgroups < 1 || workgroups > (1 << 20)) return 2;
    if (threads < 64 || threads > 1024 || threads % 64 != 0) return 2;
    const long long n = (long long)(bytes / 16);
    const u32x4* src = (const u32x4*)buf;
    unsigned* out = (unsigned*)sink;
    hipStream_t s = (hipStream_t)stream;
    switch (unroll) {
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(workgroups), dim3(threads), 0, s, src, n, out); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(workgroups), dim3(threads), 0, s, src, n, out); break;
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(workgroups), dim3(threads), 0, s, src, n, out); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(workgroups), dim3(threads), 0, s, src, n, out); break;
        case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(workgroups), dim3(threads), 0, s, src, n, out); break;
        default: return 3;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
