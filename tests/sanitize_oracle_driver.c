/* Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU oracle
 * (oracle/farn_oracle.c): every entry point on small seeded inputs, one and several
 * threads, with and without residual and bf16 output, including rows fewer than threads.
 * Exit status 0 = every call returned 0 and the threaded results equal the one-thread
 * ones; the sanitizers abort on any memory or undefined-behaviour error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_reduce_add_rmsnorm(const uint16_t *const *, int, const uint16_t *, const uint16_t *, float, int64_t,
                              int64_t, uint16_t *, uint16_t *, int);
int oracle_reduce_add_rmsnorm_quant_group(const uint16_t *const *, int, const uint16_t *, const uint16_t *, float,
                                          int64_t, int64_t, int, uint16_t *, uint16_t *, uint8_t *, float *, int);
int oracle_reduce_add_rmsnorm_mxfp4(const uint16_t *const *, int, const uint16_t *, const uint16_t *, float, int64_t,
                                    int64_t, uint16_t *, uint16_t *, uint8_t *, uint8_t *, int);
int oracle_reduce(const uint16_t *const *, int, int64_t, int64_t, uint16_t *);
int oracle_quant_group(const uint16_t *, int64_t, int64_t, int, uint8_t *, float *);
uint16_t oracle_bf16_from_double(double);
uint8_t oracle_e4m3fn_from_double(double);
uint8_t oracle_e2m1_from_double(double);

static uint32_t state = 12345u;
static uint16_t rnd_bf16(void) {
    state = state * 1664525u + 1013904223u; /* a plain LCG: test inputs only */
    uint16_t b = (uint16_t)(state >> 16);
    if ((b & 0x7F80u) == 0x7F80u) b &= 0xBFFFu; /* keep inputs finite */
    return b;
}

int main(void) {
    int failures = 0;
    const int shapes[][3] = {{1, 1, 256}, {2, 5, 128}, {8, 17, 384}, {3, 3, 1024}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        const int R = shapes[s][0], T = shapes[s][1], H = shapes[s][2];
        const size_t n = (size_t)T * H;
        uint16_t *P[8];
        for (int r = 0; r < R; ++r) {
            P[r] = malloc(n * 2);
            for (size_t i = 0; i < n; ++i) P[r][i] = rnd_bf16();
        }
        uint16_t *res = malloc(n * 2), *g = malloc((size_t)H * 2);
        for (size_t i = 0; i < n; ++i) res[i] = rnd_bf16();
        for (int h = 0; h < H; ++h) g[h] = (uint16_t)(0x3F00u + (rnd_bf16() & 0x7Fu));
        uint16_t *ro1 = malloc(n * 2), *o1 = malloc(n * 2), *ro = malloc(n * 2), *o = malloc(n * 2);
        uint8_t *q1 = malloc(n), *q = malloc(n), *mq1 = malloc(n / 2), *mq = malloc(n / 2);
        float *sc1 = malloc(n / 128 * 4 + 4), *sc = malloc(n / 128 * 4 + 4);
        uint8_t *ms1 = malloc(n / 32), *ms = malloc(n / 32);
        for (int withres = 0; withres < 2; ++withres) {
            const uint16_t *rp = withres ? res : NULL;
            failures += oracle_reduce_add_rmsnorm((const uint16_t *const *)P, R, rp, g, 1e-6f, T, H, ro1, o1, 1) != 0;
            failures += oracle_reduce_add_rmsnorm_quant_group((const uint16_t *const *)P, R, rp, g, 1e-6f, T, H, 128,
                                                              ro1, o1, q1, sc1, 1) != 0;
            failures += oracle_reduce_add_rmsnorm_mxfp4((const uint16_t *const *)P, R, rp, g, 1e-6f, T, H, ro1, NULL,
                                                        mq1, ms1, 1) != 0;
            for (int th = 2; th <= 9; th += 7) {
                memset(ro, 0xA5, n * 2);
                memset(o, 0xA5, n * 2);
                memset(q, 0xA5, n);
                failures += oracle_reduce_add_rmsnorm_quant_group((const uint16_t *const *)P, R, rp, g, 1e-6f, T, H,
                                                                  128, ro, o, q, sc, th) != 0;
                failures += memcmp(ro, ro1, n * 2) != 0 || memcmp(o, o1, n * 2) != 0 || memcmp(q, q1, n) != 0 ||
                            memcmp(sc, sc1, n / 128 * 4) != 0;
                failures += oracle_reduce_add_rmsnorm_mxfp4((const uint16_t *const *)P, R, rp, g, 1e-6f, T, H, ro, o,
                                                            mq, ms, th) != 0;
                failures += memcmp(mq, mq1, n / 2) != 0 || memcmp(ms, ms1, n / 32) != 0;
            }
        }
        failures += oracle_reduce((const uint16_t *const *)P, R, T, H, ro) != 0;
        failures += oracle_quant_group(o1, T, H, 128, q, sc) != 0;
        for (int r = 0; r < R; ++r) free(P[r]);
        free(res); free(g); free(ro1); free(o1); free(ro); free(o); free(q1); free(q);
        free(mq1); free(mq); free(sc1); free(sc); free(ms1); free(ms);
    }
    /* encoders over special values */
    const double xs[] = {0.0, -0.0, 1e-45, -1e-45, 1e-300, 3.4e38, -3.4e38, 1e39, 448.0, 464.0, 6.0, 7.0, 1.0 / 0.0};
    for (size_t i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
        (void)oracle_bf16_from_double(xs[i]);
        (void)oracle_e4m3fn_from_double(xs[i]);
        (void)oracle_e2m1_from_double(xs[i]);
    }
    printf("%d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
