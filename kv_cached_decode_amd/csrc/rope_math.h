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

// (x, y) turned by the angle whose cosine and sine are (c, s); no fused
// multiply-add, so every caller rounds the same products.
__device__ inline void rope_rotate(double x, double y, double c, double s, double& xr, double& yr) {
#pragma clang fp contract(off)
    xr = x * c - y * s;
    yr = x * s + y * c;
}

}  // namespace kvd
