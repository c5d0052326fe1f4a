// bf16_round.h -- rounding into the bf16 cache format (round to nearest even,
// a single rounding), usable from kernels and from host-side checks.
//
// bf16 keeps fp32's sign and 8 exponent bits and the top 7 fraction bits.
// Keys are rounded straight from the fp64 rotated value (no fp32 step, so no
// double rounding); values are rounded from their fp32 input.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

__host__ __device__ inline uint16_t bf16_from_f64(double x) {
    const uint64_t bits = __builtin_bit_cast(uint64_t, x);
    const uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    if (x != x) return sign | 0x7FC0u;
    const double ax = x < 0 ? -x : x;
    double r;
    if (ax < 0x1p-126) {
        // bf16 subnormals are multiples of 2^-133: scale, round to an integer
        // (ties to even), scale back -- every step exact in fp64.
        r = __builtin_rint(ax * 0x1p133) * 0x1p-133;
    } else {
        // Keep the top 7 of the 52 fraction bits.  Adding half an ulp of the
        // kept part minus one, plus the kept lsb, carries exactly when the
        // dropped part exceeds half an ulp or ties with an odd lsb; clearing
        // the dropped bits then truncates.  A carry out of the fraction bumps
        // the exponent, and one out of the largest binade reaches infinity.
        uint64_t u = __builtin_bit_cast(uint64_t, ax);
        const uint64_t drop = (1ull << 45) - 1;
        const uint64_t half_minus_one = (1ull << 44) - 1;
        u += half_minus_one + ((u >> 45) & 1ull);
        u &= ~drop;
        r = __builtin_bit_cast(double, u);
    }
    const float f = (float)r;   // exact: at most 8 significant bits (or +inf)
    return sign | (uint16_t)(__builtin_bit_cast(uint32_t, f) >> 16);
}

__host__ __device__ inline uint16_t bf16_from_f32(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) & 0x8000u) | 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);   // half an ulp minus one, plus the kept lsb
    return (uint16_t)(u >> 16);
}

}  // namespace kvd
