/*
 * Test kernels for the GPU conversion instructions the FP8 and MXFP4 paths rely on
 * (tests/test_gpu_conversions.py): v_cvt_pk_fp8_f32 over a range of fp32 bit patterns,
 * v_cvt_scalef32_pk_fp4_f32 over a list of values under every E8M0 block exponent, the
 * fused kernels' reciprocal square root (v_rsq_f64 and two Newton steps), and their FP8 group
 * scale and its reciprocal (an FMA-corrected product by 1/448; v_rcp_f32 and one Newton step).
 * Built by tp_all_reduce_amd/build.py; not part of the library.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../tp_all_reduce_amd/csrc/farn_device_math.h"

// out[i] = E4M3 code of the fp32 with bit pattern base + i, i < n (n even)
__global__ void fp8_of_bits(uint32_t base, uint8_t *out, uint32_t n) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (2 * i + 1 >= n) return;
    const float a = __uint_as_float(base + 2 * i), b = __uint_as_float(base + 2 * i + 1);
    const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    out[2 * i] = (uint8_t)(w & 0xffu);
    out[2 * i + 1] = (uint8_t)((w >> 8) & 0xffu);
}

// out[(s + 127) * n + i] = E2M1 code of x[i] * 2^-s, for s = -127 .. 127 (blockIdx.y), n even;
// the scale operand is the fp32 whose exponent field is the E8M0 byte s + 127
__global__ void fp4_all_scales(const float *x, uint8_t *out, uint32_t n) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (2 * i + 1 >= n) return;
    const float sc = __uint_as_float(blockIdx.y << 23);
    const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[2 * i], x[2 * i + 1], sc, 0);
    const size_t base = (size_t)blockIdx.y * n;
    out[base + 2 * i] = (uint8_t)(w & 0xfu);
    out[base + 2 * i + 1] = (uint8_t)((w >> 4) & 0xfu);
}

// out[2i] = the hardware reciprocal square root (v_rsq_f64) of m[i], out[2i+1] = 1/sqrt(m[i]) as
// the fused kernels form it for 2^-1000 <= m <= 2^1000 (farn_math::rsq_newton, the kernels' own
// function)
__global__ void rsq_newton(const double *m, double *out, uint32_t n) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    out[2 * i] = __builtin_amdgcn_rsq(m[i]);
    out[2 * i + 1] = farn_math::rsq_newton(m[i]);
}

// For amax = the fp32 whose bits are amax_bits[i] (a bf16 magnitude pattern shifted left 16):
// out[3i] = scale = amax/448 and out[3i+1] = 1/(scale * k) as the FP8 quant forms them, with k =
// 2^64 for scale < 2^-64 (else 1) and 0 for a zero scale; out[3i+2] = scale * k. The kernels'
// own functions (farn_math::fp8_scale, farn_math::fp8_recip) and the quant's rescaling rule.
__global__ void fp8_scale_inv(const uint32_t *amax_bits, float *out, uint32_t n) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float scale = farn_math::fp8_scale(amax_bits[i]);
    const float k = scale < 0x1p-64f ? 0x1p64f : 1.0f;
    const float sk = scale * k;
    out[3 * i] = scale;
    out[3 * i + 1] = scale == 0.0f ? 0.0f : farn_math::fp8_recip(sk);
    out[3 * i + 2] = sk;
}

extern "C" int hwconv_fp8_scale_inv(const void *amax_bits, void *out, uint32_t n, void *stream) {
    if (n == 0 || n > (1u << 20)) return 1;
    const uint32_t block = 256, grid = (n + block - 1) / block;
    hipLaunchKernelGGL(fp8_scale_inv, dim3(grid), dim3(block), 0, (hipStream_t)stream, (const uint32_t *)amax_bits,
                       (float *)out, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int hwconv_rsq_newton(const void *m, void *out, uint32_t n, void *stream) {
    if (n == 0 || n > (1u << 26)) return 1;
    const uint32_t block = 256, grid = (n + block - 1) / block;
    hipLaunchKernelGGL(rsq_newton, dim3(grid), dim3(block), 0, (hipStream_t)stream, (const double *)m, (double *)out, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int hwconv_fp8_of_bits(uint32_t base, void *out, uint32_t n, void *stream) {
    if (n == 0 || (n & 1u) || n > (1u << 28) || (uint64_t)base + n > 0x100000000ull) return 1;
    const uint32_t block = 256, grid = (n / 2 + block - 1) / block;
    hipLaunchKernelGGL(fp8_of_bits, dim3(grid), dim3(block), 0, (hipStream_t)stream, base, (uint8_t *)out, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int hwconv_fp4_all_scales(const void *x, void *out, uint32_t n, void *stream) {
    if (n == 0 || (n & 1u) || n > (1u << 20)) return 1;
    const uint32_t block = 256, grid = (n / 2 + block - 1) / block;
    hipLaunchKernelGGL(fp4_all_scales, dim3(grid, 255), dim3(block), 0, (hipStream_t)stream, (const float *)x,
                       (uint8_t *)out, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
