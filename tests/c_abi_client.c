/*
 * A plain C client of include/farn.h: HIP runtime for memory, no Python, no torch.
 * It runs the FP8 call on a case whose results have a closed form and checks them.
 *
 * Case (R = 2, T = 3, H = 256): P_1 = -P_0 bit for bit, so the rank sum is +0 and
 * residual_out equals the residual, the constant 2; out = 2 / sqrt(4 + eps) * gamma is
 * gamma times (1 - 1.25e-7), which rounds to gamma in bf16; gamma is 1.5 in group 0 and
 * 0.75 in group 1, so each group's amax is its gamma, its scale fl32(gamma / 448) and every
 * code the largest finite E4M3 value 448 (0x7E). A call with group size 64 must be
 * rejected with FARN_ERR_SHAPE.
 * Exit status 0 when every check holds.
 *
 * Built by tp_all_reduce_amd/build.py; run by tests/test_gpu_parity.py.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/farn.h"

#define T 3
#define H 256
#define CHECK_HIP(x)                                                         \
    do {                                                                     \
        hipError_t e_ = (x);                                                 \
        if (e_ != hipSuccess) {                                              \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__); \
            return 2;                                                        \
        }                                                                    \
    } while (0)

static uint16_t bf16_of(float f) { /* exact for the values used here */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void) {
    if (farn_abi_version() != FARN_ABI_VERSION) return 3;
    static uint16_t p0[T * H], p1[T * H], res[T * H], gamma[H];
    for (int i = 0; i < T * H; ++i) {
        float v = (float)((i * 37) % 101 - 50) * 0.125f;
        p0[i] = bf16_of(v);
        p1[i] = (uint16_t)(p0[i] ^ 0x8000u);
        res[i] = bf16_of(2.0f);
    }
    for (int h = 0; h < H; ++h) gamma[h] = bf16_of(h < 128 ? 1.5f : 0.75f);

    void *d_p0, *d_p1, *d_res, *d_g, *d_ro, *d_out, *d_q, *d_s;
    CHECK_HIP(hipMalloc(&d_p0, sizeof p0));
    CHECK_HIP(hipMalloc(&d_p1, sizeof p1));
    CHECK_HIP(hipMalloc(&d_res, sizeof res));
    CHECK_HIP(hipMalloc(&d_g, sizeof gamma));
    CHECK_HIP(hipMalloc(&d_ro, sizeof res));
    CHECK_HIP(hipMalloc(&d_out, sizeof res));
    CHECK_HIP(hipMalloc(&d_q, T * H));
    CHECK_HIP(hipMalloc(&d_s, T * (H / 128) * sizeof(float)));
    CHECK_HIP(hipMemcpy(d_p0, p0, sizeof p0, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_p1, p1, sizeof p1, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_res, res, sizeof res, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_g, gamma, sizeof gamma, hipMemcpyHostToDevice));

    const void *partials[2] = {d_p0, d_p1};
    /* a rejected call enqueues nothing and says why */
    farn_status bad = farn_reduce_add_rmsnorm_quant_group(partials, 2, d_res, d_g, 1e-6f, T, H, 64,
                                                          d_ro, d_out, d_q, (float *)d_s, NULL);
    if (bad != FARN_ERR_SHAPE) {
        fprintf(stderr, "expected FARN_ERR_SHAPE, got %d (%s)\n", (int)bad, farn_status_string(bad));
        return 4;
    }
    farn_status st = farn_reduce_add_rmsnorm_quant_group(partials, 2, d_res, d_g, 1e-6f, T, H, 128,
                                                         d_ro, d_out, d_q, (float *)d_s, NULL);
    if (st != FARN_OK) {
        fprintf(stderr, "call failed: %s\n", farn_status_string(st));
        return 5;
    }
    CHECK_HIP(hipDeviceSynchronize());

    static uint16_t ro[T * H], out[T * H];
    static uint8_t q[T * H];
    static float s[T * (H / 128)];
    CHECK_HIP(hipMemcpy(ro, d_ro, sizeof ro, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(q, d_q, sizeof q, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(s, d_s, sizeof s, hipMemcpyDeviceToHost));

    int errors = 0;
    for (int i = 0; i < T * H; ++i) {
        if (ro[i] != res[i]) ++errors;
        if (out[i] != gamma[i % H]) ++errors;
        if (q[i] != 0x7Eu) ++errors;
    }
    for (int t = 0; t < T; ++t) {
        if (s[t * 2 + 0] != 1.5f / 448.0f) ++errors;
        if (s[t * 2 + 1] != 0.75f / 448.0f) ++errors;
    }
    hipFree(d_p0);
    hipFree(d_p1);
    hipFree(d_res);
    hipFree(d_g);
    hipFree(d_ro);
    hipFree(d_out);
    hipFree(d_q);
    hipFree(d_s);
    printf("c_abi_client: %d mismatches\n", errors);
    return errors == 0 ? 0 : 1;
}
