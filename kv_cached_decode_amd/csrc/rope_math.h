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

#include <cmath>
#include <cstddef>

namespace kvd {

// Element indices of pair i: HALF pairs (i, i + D/2), INTERLEAVED (2i, 2i+1).
__device__ inline void rope_pair(int i, int half, int interleaved, int& ia, int& ic) {
    if (interleaved) { ia = 2 * i; ic = 2 * i + 1; }
    else             { ia = i;     ic = i + half; }
}

// Sine and cosine of a rotary angle in fp64, within about two units in the
// last place.  Cody and Waite's reduction by pi/2: k = nearest integer to
// x * 2/pi, r = x - k*pi/2 with pi/2 in three parts (the first two hold 33
// significant bits, so k times them is exact for k < 2^20; each step is one
// fused multiply-add, rounded once); then the Taylor series of sin and cos on
// |r| <= pi/4 up to r^17 / 17! and r^18 / 18! (truncation below 1e-19
// relative), and the quadrant k mod 4 picks signs and swaps.  Angles of 1.6e6
// and more (positions beyond about a million at frequency 1) take the library
// routine.  A few dozen fp64 operations instead of the library's general
// path, which dominated the fused step's set-up.
__host__ __device__ inline void rope_sincos(double x, double& sn, double& cs) {
    if (!(x > -1.6e6 && x < 1.6e6)) {
        sn = sin(x);
        cs = cos(x);
        return;
    }
    constexpr double C1 = 0x1.921fb544p+0;            // pi/2, leading 33 bits
    constexpr double C2 = 0x1.0b4611a6p-34;           // the next 33 bits
    constexpr double C3 = 0x1.3198a2e037073p-69;      // the rest, rounded
    constexpr double TWO_OVER_PI = 0x1.45f306dc9c883p-1;
    const double k = rint(x * TWO_OVER_PI);
    double r = fma(-k, C1, x);
    r = fma(-k, C2, r);
    r = fma(-k, C3, r);
    const double r2 = r * r;
    // sin r = r - r^3/3! + ... - r^15/15! + r^17/17!, Horner in r^2
    double ps = 1.0 / 355687428096000.0;
    ps = fma(ps, r2, -1.0 / 1307674368000.0);
    ps = fma(ps, r2, 1.0 / 6227020800.0);
    ps = fma(ps, r2, -1.0 / 39916800.0);
    ps = fma(ps, r2, 1.0 / 362880.0);
    ps = fma(ps, r2, -1.0 / 5040.0);
    ps = fma(ps, r2, 1.0 / 120.0);
    ps = fma(ps, r2, -1.0 / 6.0);
    const double s = fma(ps * r2, r, r);
    // cos r = 1 - r^2/2! + ... + r^16/16! - r^18/18!
    double pc = -1.0 / 6402373705728000.0;
    pc = fma(pc, r2, 1.0 / 20922789888000.0);
    pc = fma(pc, r2, -1.0 / 87178291200.0);
    pc = fma(pc, r2, 1.0 / 479001600.0);
    pc = fma(pc, r2, -1.0 / 3628800.0);
    pc = fma(pc, r2, 1.0 / 40320.0);
    pc = fma(pc, r2, -1.0 / 720.0);
    pc = fma(pc, r2, 1.0 / 24.0);
    pc = fma(pc, r2, -0.5);
    const double c = fma(pc, r2, 1.0);
    switch ((long long)k & 3) {
        case 0: sn = s;  cs = c;  break;
        case 1: sn = c;  cs = -s; break;
        case 2: sn = -s; cs = -c; break;
        default: sn = -c; cs = s; break;
    }
}

// The frequencies theta_i = base^(-2i/D) are evaluated once on the host (the
// same libm pow for every call) and passed to the kernels; a kernel forms the
// angle pos * theta_i and its cosine and sine in fp64.
__device__ inline void rope_angle(double theta, int pos, double& cs, double& sn) {
    const double phi = (double)pos * theta;
    rope_sincos(phi, sn, cs);
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
