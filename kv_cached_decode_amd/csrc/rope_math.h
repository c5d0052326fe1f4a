// rope_math.h -- the RoPE arithmetic shared by the stand-alone RoPE/append
// kernel and the fused decode-step kernel, so that both produce the same bits.
//
// Pair i < D/2 of a head vector at absolute position pos is turned by the
// angle pos * base^(-2i/D) (ferric-core generate.rs: `rope_off_t` at the
// token's position; the frequency formula is the usual one, the pages name
// only the base).  The frequency, the angle, its cosine and sine and the
// rotation are all evaluated in fp64; callers round the result once into
// their output type.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace kvd {

// Element indices of pair i: HALF pairs (i, i + D/2), INTERLEAVED (2i, 2i+1).
__device__ inline void rope_pair(int i, int half, int interleaved, int& ia, int& ic) {
    if (interleaved) { ia = 2 * i; ic = 2 * i + 1; }
    else             { ia = i;     ic = i + half; }
}

// The frequencies theta_i = base^(-2i/D) are evaluated once on the host (the
// same libm pow for every call) and passed to the kernels; a kernel forms the
// angle pos * theta_i and its cosine and sine in fp64.
__device__ inline void rope_angle(double theta, int pos, double& cs, double& sn) {
    const double phi = (double)pos * theta;
    sincos(phi, &sn, &cs);
}

// Element i (per thread) of a double table inside the kernel's by-value
// argument block, read in place.  The explicit kernel arguments start at the
// base of the kernarg segment (AMDGPU code-object ABI), so the table sits at
// offsetof(Args, table) there.  Indexing the by-value argument itself with a
// per-thread value would make the compiler copy the whole argument block to
// scratch memory first.
__device__ inline double kernarg_double(size_t table_offset, int i) {
    typedef const __attribute__((address_space(4))) char kchar;
    typedef const __attribute__((address_space(4))) double kdouble;
    kchar* base = (kchar*)__builtin_amdgcn_kernarg_segment_ptr();
    return ((kdouble*)(base + table_offset))[i];
}

// (x, y) turned by the angle whose cosine and sine are (c, s); no fused
// multiply-add, so every caller rounds the same products.
__device__ inline void rope_rotate(double x, double y, double c, double s, double& xr, double& yr) {
#pragma clang fp contract(off)
    xr = x * c - y * s;
    yr = x * s + y * c;
}

}  // namespace kvd
