// Scalar arithmetic of the fused kernels that the GPU tests also run on their own
// (tests/hw_conversions.hip, over every input class these functions are used on), so that the
// tests check the kernels' own code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace farn_math {

// 1/sqrt(m) for 2^-1000 <= m <= 2^1000: the hardware reciprocal square root (about 24 correct
// bits, measured) refined by two Newton steps, y += y * (1/2 - m y^2 / 2); the result sits
// within two fp64 units of the correctly rounded 1/sqrt (one step leaves up to ~20).
__device__ __forceinline__ double rsq_newton(double m) {
    const double hm = 0.5 * m;
    const double y0 = __builtin_amdgcn_rsq(m);
    const double y1 = __builtin_fma(y0, __builtin_fma(-hm * y0, y0, 0.5), y0);
    return __builtin_fma(y1, __builtin_fma(-hm * y1, y1, 0.5), y1);
}

// RN(1/448).
constexpr float kInv448 = 0x1.24924ap-9f;

// The FP8 group scale amax/448 for amax = the fp32 with bit pattern `amax` (a bf16 magnitude
// pattern shifted left 16): q0 = amax * RN(1/448) corrected by one FMA of the remainder,
// q0 + (amax - q0 * 448) * RN(1/448). Over every finite bf16 amax (32,640 values, zero and
// subnormals included) this is the correctly rounded quotient (checked in exact rational
// arithmetic and on the GPU); inf and NaN take q0 (inf, or the quieted NaN).
__device__ __forceinline__ float fp8_scale(uint32_t amax) {
    const float a = __uint_as_float(amax);
    const float q0 = a * kInv448;
    const float r = __builtin_fmaf(-q0, 448.0f, a);
    return amax < 0x7f800000u ? __builtin_fmaf(r, kInv448, q0) : q0;
}

// 1/s for the (rescaled) scale s of an FP8 group: the hardware reciprocal refined by one
// Newton step, y + y * (1 - s * y), which is the correctly rounded reciprocal for every scale
// a bf16 amax gives (checked on the GPU for all of them); for inf and NaN the hardware
// reciprocal itself (0, NaN). The caller handles s = 0.
__device__ __forceinline__ float fp8_recip(float s) {
    const float y = __builtin_amdgcn_rcpf(s);
    const float yn = __builtin_fmaf(__builtin_fmaf(-s, y, 1.0f), y, y);
    return __builtin_isfinite(s) ? yn : y;
}

}  // namespace farn_math
