// Host-side driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the C-ABI
// layer (tp_all_reduce_amd/csrc/farn_api.cpp) with the kernel launcher replaced by a stub
// that records the launch it was asked for. Every entry point is called with well-formed
// and malformed arguments over fake host addresses (the layer never dereferences device
// pointers). Exit status 0 means every expectation held; the sanitizers abort on any
// memory or undefined-behaviour error.
#include <stdint.h>
#include <stdio.h>
#include <math.h>

#include "../include/farn.h"
#include "../tp_all_reduce_amd/csrc/farn_internal.h"

namespace {
int g_launches = 0;
farn::Call g_last;
int g_last_variant = 0;
}  // namespace

namespace farn {
int launch(const Call &c, int variant) {
    ++g_launches;
    g_last = c;
    g_last_variant = variant;
    return 0;
}
}  // namespace farn

static int failures = 0;
#define EXPECT(cond)                                                       \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static void *A(uint64_t slot, uint64_t off = 0) { return (void *)(uintptr_t)(0x1000000000ull + slot * (1ull << 28) + off); }
// addresses 2^40 bytes apart, for calls whose arrays are larger than A's spacing
static void *B(uint64_t slot) { return (void *)(uintptr_t)((1ull << 44) + slot * (1ull << 40)); }

int main() {
    const void *parts[8];
    for (int r = 0; r < 8; ++r) parts[r] = A(r);
    const float eps = 1e-6f;
    // accepted calls reach the launcher once, with the arguments passed through
    int before = g_launches;
    EXPECT(farn_reduce_add_rmsnorm(parts, 8, A(10), A(11), eps, 64, 7168, A(12), A(13), nullptr) == FARN_OK);
    EXPECT(g_launches == before + 1 && g_last.R == 8 && g_last.T == 64 && g_last.H == 7168 && g_last.q == nullptr);
    EXPECT(farn_reduce_add_rmsnorm_quant_group(parts, 4, nullptr, A(11), eps, 16, 4096, 128, A(12), nullptr, A(14),
                                               (float *)A(15), nullptr) == FARN_OK);
    EXPECT(g_last.residual == nullptr && g_last.out == nullptr && g_last.q == A(14) && !g_last.mxfp4);
    EXPECT(farn_reduce_add_rmsnorm_mxfp4(parts, 2, A(10), A(11), eps, 5, 96, A(12), A(13), A(14), A(15), nullptr) ==
           FARN_OK);
    EXPECT(g_last.mxfp4);
    EXPECT(farn_reduce_add_rmsnorm_quant_group_ex(parts, 8, A(10), A(11), eps, 8192, 7168, 128, A(12), A(13), A(14),
                                                  (float *)A(15), nullptr, FARN_VARIANT_LATENCY | FARN_SCALES_COL_MAJOR) ==
           FARN_OK);
    EXPECT(g_last.scale_cols && g_last_variant == FARN_VARIANT_LATENCY);
    EXPECT(farn_reduce(parts, 3, 7, 1024, A(12), nullptr) == FARN_OK);
    EXPECT(farn_quant_group(A(12), 7, 1024, 128, A(14), (float *)A(15), nullptr) == FARN_OK);
    // in place: residual_out == residual
    EXPECT(farn_reduce_add_rmsnorm(parts, 8, A(10), A(11), eps, 64, 7168, A(10), A(13), nullptr) == FARN_OK);
    // T == 0: OK, nothing launched
    before = g_launches;
    EXPECT(farn_reduce_add_rmsnorm(parts, 8, nullptr, A(11), eps, 0, 7168, nullptr, nullptr, nullptr) == FARN_OK);
    EXPECT(farn_reduce(parts, 8, 0, 7168, nullptr, nullptr) == FARN_OK);
    EXPECT(farn_quant_group(nullptr, 0, 1024, 128, nullptr, nullptr, nullptr) == FARN_OK);
    EXPECT(g_launches == before);
    // rejected calls never reach the launcher
    before = g_launches;
    EXPECT(farn_reduce_add_rmsnorm(nullptr, 8, A(10), A(11), eps, 4, 256, A(12), A(13), nullptr) == FARN_ERR_NULL);
    EXPECT(farn_reduce_add_rmsnorm(parts, 9, A(10), A(11), eps, 4, 256, A(12), A(13), nullptr) == FARN_ERR_SHAPE);
    EXPECT(farn_reduce_add_rmsnorm(parts, 0, A(10), A(11), eps, 4, 256, A(12), A(13), nullptr) == FARN_ERR_SHAPE);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), eps, -1, 256, A(12), A(13), nullptr) == FARN_ERR_SHAPE);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), eps, (int64_t)1 << 41, 256, A(12), A(13), nullptr) ==
           FARN_ERR_SHAPE);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), eps, 4, 260, A(12), A(13), nullptr) == FARN_ERR_SHAPE);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), eps, 4, FARN_MAX_H + 8, A(12), A(13), nullptr) ==
           FARN_ERR_SHAPE);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), NAN, 4, 256, A(12), A(13), nullptr) == FARN_ERR_EPS);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), -1.0f, 4, 256, A(12), A(13), nullptr) == FARN_ERR_EPS);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10, 4), A(11), eps, 4, 256, A(12), A(13), nullptr) == FARN_ERR_ALIGN);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), eps, 4, 256, A(12), A(0, 64), nullptr) == FARN_ERR_ALIAS);
    EXPECT(farn_reduce_add_rmsnorm(parts, 2, A(10), A(11), eps, 4, 256, A(10, 16), A(13), nullptr) == FARN_ERR_ALIAS);
    EXPECT(farn_reduce_add_rmsnorm_ex(parts, 2, A(10), A(11), eps, 4, 256, A(12), A(13), nullptr, 3) ==
           FARN_ERR_VARIANT);
    EXPECT(farn_reduce_add_rmsnorm_ex(parts, 2, A(10), A(11), eps, 4, 256, A(12), A(13), nullptr,
                                      FARN_SCALES_COL_MAJOR) == FARN_ERR_VARIANT);
    EXPECT(farn_reduce_add_rmsnorm_quant_group(parts, 2, A(10), A(11), eps, 4, 256, 64, A(12), A(13), A(14),
                                               (float *)A(15), nullptr) == FARN_ERR_SHAPE);
    const void *big[8];
    for (int r = 0; r < 8; ++r) big[r] = B(r);
    EXPECT(farn_reduce_add_rmsnorm_quant_group_ex(big, 8, B(10), B(11), eps, (int64_t)1 << 21, 32768, 128, B(12),
                                                  B(13), B(14), (float *)B(15), nullptr, FARN_SCALES_COL_MAJOR) ==
           FARN_ERR_SHAPE);
    EXPECT(farn_reduce_add_rmsnorm_mxfp4(parts, 2, A(10), A(11), eps, 4, 48, A(12), A(13), A(14), A(15), nullptr) ==
           FARN_ERR_SHAPE);
    EXPECT(farn_reduce(parts, 2, 4, 256, A(0, 32), nullptr) == FARN_ERR_ALIAS);
    EXPECT(farn_quant_group(A(12), 4, 256, 128, A(12, 64), (float *)A(15), nullptr) == FARN_ERR_ALIAS);
    EXPECT(g_launches == before);
    // LDS reserved to hold the narrow kernels of long rows (H = 6152 .. 8192) at two workgroups
    // per compute unit: FP8 / MXFP4 with R >= 6 above 512 rows and R = 4, 5 from 2048 rows; the
    // plain call with R = 4 .. 7 from 2048 rows; never for the small-call schedule, the plain
    // call with R = 8 or R < 4, or the wide shape
    struct LdsCase { int R; int64_t T, H; int quant; int variant; unsigned want; };
    const LdsCase lds_cases[] = {
        {8, 8192, 7168, 1, 0, 56u << 10}, {8, 8192, 7168, 2, 0, 56u << 10}, {8, 8192, 7168, 0, 0, 0},
        {8, 512, 7168, 1, 0, 0},          {8, 513, 7168, 1, 0, 56u << 10}, {6, 1024, 6272, 1, 0, 56u << 10},
        {5, 1024, 7168, 1, 0, 0},         {4, 2048, 7168, 1, 0, 56u << 10}, {4, 2047, 7168, 2, 0, 0},
        {2, 8192, 7168, 1, 0, 0},         {8, 8192, 6144, 1, 0, 0},          {8, 8192, 8192, 1, 0, 56u << 10},
        {8, 8192, 7168, 1, FARN_VARIANT_WIDE, 0}, {8, 8192, 8192, 0, FARN_VARIANT_NARROW, 0},
        {6, 2048, 7168, 0, 0, 56u << 10}, {4, 2048, 6656, 0, 0, 56u << 10}, {4, 2047, 7168, 0, 0, 0},
        {7, 8192, 7168, 0, 0, 56u << 10}, {3, 8192, 7168, 0, 0, 0},          {6, 4096, 8192, 0, 0, 0},
        {6, 4096, 8192, 0, FARN_VARIANT_NARROW, 56u << 10}, {6, 2048, 8192, 0, 0, 56u << 10},
        {7, 8192, 6144, 0, 0, 0},
    };
    for (const LdsCase &lc : lds_cases) {
        farn_status st;
        if (lc.quant == 1)
            st = farn_reduce_add_rmsnorm_quant_group_ex(parts, lc.R, A(10), A(11), eps, lc.T, lc.H, 128, B(12), B(13),
                                                        B(14), (float *)B(15), nullptr, lc.variant);
        else if (lc.quant == 2)
            st = farn_reduce_add_rmsnorm_mxfp4_ex(parts, lc.R, A(10), A(11), eps, lc.T, lc.H, B(12), B(13), B(14),
                                                  B(15), nullptr, lc.variant);
        else
            st = farn_reduce_add_rmsnorm_ex(parts, lc.R, A(10), A(11), eps, lc.T, lc.H, B(12), B(13), nullptr,
                                            lc.variant);
        if (st != FARN_OK)
            fprintf(stderr, "R=%d T=%lld H=%lld quant=%d: status %d\n", lc.R, (long long)lc.T, (long long)lc.H, lc.quant,
                    (int)st);
        EXPECT(st == FARN_OK);
        if (g_last.lds_reserve != lc.want)
            fprintf(stderr, "lds_reserve R=%d T=%lld H=%lld quant=%d variant=%d: %u, want %u\n", lc.R, (long long)lc.T,
                    (long long)lc.H, lc.quant, lc.variant, g_last.lds_reserve, lc.want);
        EXPECT(g_last.lds_reserve == lc.want);
    }
    // the dispatch rule and the status strings over a grid, extreme sizes included
    const int64_t Ts[] = {1, 2, 63, 64, 511, 512, 1023, 1024, 2047, 2048, 4096, 8191, 8192, (int64_t)1 << 40};
    for (int R = 1; R <= 8; ++R)
        for (int64_t H = 8; H <= FARN_MAX_H; H += (H < 1024 ? 8 : 264))
            for (int64_t T : Ts)
                for (int quant = 0; quant < 2; ++quant) {
                    const int v = farn_select_variant(R, T, H, quant);
                    EXPECT(v == FARN_VARIANT_LATENCY || v == FARN_VARIANT_BANDWIDTH);
                }
    for (int s = -2; s < 12; ++s) EXPECT(farn_status_string(s) != nullptr);
    EXPECT(farn_abi_version() == FARN_ABI_VERSION);
    printf("%d launches, %d failures\n", g_launches, failures);
    return failures == 0 ? 0 : 1;
}
