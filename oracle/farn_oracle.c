/*
 * CPU ORACLE for the fused reduce + residual-add + RMSNorm (+ per-group FP8 quant)
 * op. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
 * baseline leg use it to judge the GPU path. The product library never links,
 * loads or calls it, and it shares no code, header or table with the GPU path.
 *
 * It is the plain definition of the op, written out element by element, in the
 * order of the steps:
 *
 *   1. reduce     acc = P_0; acc = fl32(acc + P_r) for r = 1..R-1   (fp32 adds,
 *                 fixed rank order)
 *   2. residual   y32 = fl32(acc + residual)        (skipped when residual is NULL)
 *   3. round      residual_out = bf16_rne(y32)
 *   4. stats      rstd = 1 / sqrt(sum_h y_h^2 / H + eps), y = residual_out as
 *                 double, sum in double
 *   5. normalise  out = bf16_rne(y * rstd * gamma), product in double, one rounding
 *   6. quant      per row and 128-channel group: amax = max |out|,
 *                 scale = fl32(amax / 448), v = fl32(out / scale) (IEEE single
 *                 division), q = e4m3fn_rne_satfinite(v); scale == 0 gives q = 0.
 *
 * Where the pages support these steps:
 *   - all-reduce then RMSNorm of the all-reduce output, returning both
 *     (the normalised value and the all-reduce/residual output):
 *     "ROCm AITER fused all-reduce + RMSNorm" (vLLM #37646 summary), snippet
 *     AiterAllreduceFusedRMSNormPattern (pattern / replacement) and the
 *     fused_add_rms_norm pattern named in the implementation breakdown;
 *   - residual passed in and returned next to the normalised output:
 *     "AMD fused AllReduce-RMSNorm quant kernel" (sglang #24651 summary),
 *     layernorm.py snippet _forward_with_allreduce_fusion_quant_per_group;
 *   - quant applied to the bf16 normalised activation (fused_out[0]) in
 *     groups of 128 ("per-1x128"): same snippet, attempt 2.
 * The pages print no formula; the definition above (fp32 fold in rank order,
 * residual last, bf16 rounding points, RMSNorm of the rounded value, eps inside
 * the square root, scale = amax/448) is the stated op, and every choice the
 * pages leave open is taken at its plainest reading:
 *   - rank order 0..R-1, residual added last, fp32 adds, no FMA;
 *   - RNE for bf16 and e4m3fn; NaN stays NaN;
 *   - statistics over the bf16 residual_out, mean over all H channels;
 *   - one rounding of y*rstd*gamma;
 *   - quant input is the bf16 `out`; no floor on the scale; all-zero group gives
 *     scale 0 and codes 0;
 *   - out / scale is a binary32 division (the division an fp32 framework performs
 *     before casting to e4m3fn), and that quotient is rounded once more, to e4m3fn;
 *   - e4m3fn saturates to +-448 (it never has to for finite input, since
 *     |out/scale| <= 448 up to one fp32 rounding);
 *   - a NULL residual means "no residual" (zeros, the zero not added);
 *   - scales are fp32 [T, H/group] row-major.
 *
 * Number formats are written from their public definitions:
 *   bfloat16 = the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent
 *   bits with bias 127, 7 mantissa bits, subnormals, +-inf, NaN);
 *   E4M3 of the OCP 8-bit floating point specification (OFP8): 1 sign bit,
 *   4 exponent bits (bias 7), 3 mantissa bits, subnormals 2^-6 * m/8, no
 *   infinities, S.1111.111 = NaN, largest finite 448.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread (no fast
 * math: the fp32 fold must be plain IEEE single adds).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bits -> exact binary64 value (every bf16 is a binary32, every binary32 a binary64). */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Round a binary64 value to the nearest bfloat16, ties to even, in one rounding.
 * The value is scaled by its bf16 quantum (a power of two, so the scaling is
 * exact), rounded to an integer with nearbyint (ties to even in the default
 * rounding mode), and scaled back. Below the smallest normal (2^-126) the
 * quantum stays 2^-133 (bf16 subnormals). Results at or above 2^128 are +-inf.
 * NaN returns the quiet NaN of the same sign.
 */
uint16_t oracle_bf16_from_double(double x) {
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);           /* a in [2^(e2-1), 2^e2) */
    int ex = e2 - 1;
    if (ex < -126) ex = -126; /* subnormal bf16: fixed quantum 2^-133 */
    double quantum = ldexp(1.0, ex - 7);
    double r = nearbyint(a / quantum) * quantum;
    if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits and is in binary32 range */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/*
 * Round a binary64 value to the nearest OCP E4M3 code, ties to even, saturating
 * finite values (and +-inf) to +-448. The quantum of E4M3 is 2^(e-3) for |v| in
 * [2^e, 2^(e+1)) with e >= -6, and 2^-9 below 2^-6 (subnormals).
 */
uint8_t oracle_e4m3fn_from_double(double x) {
    const uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
    double a = fabs(x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;
    if (ex < -6) ex = -6;
    double quantum = ldexp(1.0, ex - 3);
    double r = nearbyint(a / quantum) * quantum; /* in [0, 448] */
    if (r == 0.0) return sign;
    frexp(r, &e2);
    int er = e2 - 1;
    if (er < -6) /* subnormal code: r = m * 2^-9, m in 1..7 */
        return (uint8_t)(sign | (uint8_t)(r * 512.0));
    int mant = (int)(r / ldexp(1.0, er - 3)) - 8; /* 0..7 */
    return (uint8_t)(sign | (uint8_t)(((er + 7) << 3) | mant));
}

typedef struct {
    const uint16_t *const *partials;
    int R;
    const uint16_t *residual;
    const uint16_t *gamma;
    float eps;
    int64_t T, H;
    int group; /* 0 = no quant */
    uint16_t *residual_out;
    uint16_t *out;
    uint8_t *q;
    float *scales;
    int nthreads;
    int tid;
} job_t;

/* One token row: steps 1-6 of the header, in order. `o` is an H-long scratch row. */
static void one_row(const job_t *j, int64_t t, uint16_t *o) {
    const int64_t H = j->H;
    const int64_t base = t * H;

    /* steps 1-3: fp32 fold in rank order, residual last, round to bf16 */
    for (int64_t h = 0; h < H; ++h) {
        float acc = bf16_to_float(j->partials[0][base + h]);
        for (int r = 1; r < j->R; ++r) acc = acc + bf16_to_float(j->partials[r][base + h]);
        float y32 = acc;
        if (j->residual) y32 = acc + bf16_to_float(j->residual[base + h]);
        j->residual_out[base + h] = oracle_bf16_from_double((double)y32);
    }

    /* step 4: mean of squares of the bf16 values, in double */
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        double y = bf16_to_double(j->residual_out[base + h]);
        ss += y * y;
    }
    double rstd = 1.0 / sqrt(ss / (double)H + (double)j->eps);

    /* step 5: normalise and scale by gamma, one rounding to bf16 */
    for (int64_t h = 0; h < H; ++h) {
        double y = bf16_to_double(j->residual_out[base + h]);
        o[h] = oracle_bf16_from_double(y * rstd * bf16_to_double(j->gamma[h]));
        if (j->out) j->out[base + h] = o[h];
    }

    /* step 6: per-group FP8 quant of the bf16 out */
    if (j->group > 0) {
        const int64_t G = H / j->group;
        for (int64_t g = 0; g < G; ++g) {
            const int64_t h0 = g * j->group;
            double amax = 0.0;
            for (int64_t h = h0; h < h0 + j->group; ++h) {
                double v = fabs(bf16_to_double(o[h]));
                if (v > amax || isnan(v)) amax = v;
                if (isnan(amax)) break;
            }
            /* amax/448 in binary64 then to binary32: a bf16 divided by 448 = 7*64 has a
               non-terminating binary expansion, so this equals the correctly rounded fp32 quotient */
            float scale = (float)(amax / 448.0);
            j->scales[t * G + g] = scale;
            for (int64_t h = h0; h < h0 + j->group; ++h) {
                if (scale == 0.0f)
                    j->q[base + h] = 0x00u;
                else
                    j->q[base + h] = oracle_e4m3fn_from_double((double)(bf16_to_float(o[h]) / scale));
            }
        }
    }
}

static void *worker(void *arg) {
    const job_t *j = (const job_t *)arg;
    uint16_t *o = (uint16_t *)malloc((size_t)j->H * sizeof(uint16_t));
    if (!o) return (void *)1;
    for (int64_t t = j->tid; t < j->T; t += j->nthreads) one_row(j, t, o);
    free(o);
    return NULL;
}

static int run(job_t *proto) {
    if (!proto->partials || proto->R < 1 || !proto->gamma || !proto->residual_out || proto->T < 0 ||
        proto->H < 1)
        return -1;
    for (int r = 0; r < proto->R; ++r)
        if (!proto->partials[r]) return -1;
    if (proto->group > 0 && (proto->H % proto->group != 0 || !proto->q || !proto->scales)) return -1;
    if (proto->group == 0 && !proto->out) return -1;
    int n = proto->nthreads < 1 ? 1 : proto->nthreads;
    if (n > 256) n = 256;
    if ((int64_t)n > proto->T) n = proto->T > 0 ? (int)proto->T : 1;
    job_t jobs[256];
    pthread_t th[256];
    int rc = 0;
    for (int k = 0; k < n; ++k) {
        jobs[k] = *proto;
        jobs[k].nthreads = n;
        jobs[k].tid = k;
    }
    /* threads that did start are always joined before returning: they use `jobs` */
    int started = 1;
    for (int k = 1; k < n; ++k) {
        if (pthread_create(&th[k], NULL, worker, &jobs[k]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    if (rc == 0 && worker(&jobs[0]) != NULL) rc = -3;
    for (int k = 1; k < started; ++k) {
        void *ret = NULL;
        pthread_join(th[k], &ret);
        if (ret != NULL && rc == 0) rc = -3;
    }
    return rc;
}

/* residual may be NULL (no residual); residual_out may equal residual (in place). Returns 0 on success. */
int oracle_reduce_add_rmsnorm(const uint16_t *const *partials, int R, const uint16_t *residual,
                              const uint16_t *gamma, float eps, int64_t T, int64_t H,
                              uint16_t *residual_out, uint16_t *out, int nthreads) {
    job_t j = {partials, R, residual, gamma, eps, T, H, 0, residual_out, out, NULL, NULL, nthreads, 0};
    return run(&j);
}

/* As above plus step 6; `out` may be NULL (bf16 output not kept). Returns 0 on success. */
int oracle_reduce_add_rmsnorm_quant_group(const uint16_t *const *partials, int R,
                                          const uint16_t *residual, const uint16_t *gamma, float eps,
                                          int64_t T, int64_t H, int group, uint16_t *residual_out,
                                          uint16_t *out, uint8_t *q, float *scales, int nthreads) {
    if (group < 1) return -1;
    job_t j = {partials, R, residual, gamma, eps, T, H, group, residual_out, out, q, scales, nthreads, 0};
    return run(&j);
}

/* Array forms of the two encoders, so tests can sweep many inputs in one call. */
void oracle_bf16_from_double_array(const double *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_bf16_from_double(x[i]);
}

void oracle_e4m3fn_from_double_array(const double *x, uint8_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_e4m3fn_from_double(x[i]);
}

/*
 * Unfused building blocks, for the two- and three-kernel compositions the fused call
 * replaces ("AMD fused AllReduce-RMSNorm quant kernel", sglang #24651 summary: the
 * fallback chain runs AR + RMSNorm and then a separate per-1x128 quant, and the
 * benchmark compares 3-, 2- and 1-kernel variants; "ROCm AITER fused all-reduce +
 * RMSNorm", vLLM #37646 summary: the unfused pattern is tensor_model_parallel_all_reduce
 * followed by rms_norm).
 */

/* All-reduce alone: out = bf16_rne(P_0 + P_1 + ... + P_{R-1}), fp32 left fold in rank order. */
int oracle_reduce(const uint16_t *const *partials, int R, int64_t T, int64_t H, uint16_t *out) {
    if (!partials || R < 1 || !out || T < 0 || H < 1) return -1;
    for (int r = 0; r < R; ++r)
        if (!partials[r]) return -1;
    for (int64_t i = 0; i < T * H; ++i) {
        float acc = bf16_to_float(partials[0][i]);
        for (int r = 1; r < R; ++r) acc = acc + bf16_to_float(partials[r][i]);
        out[i] = oracle_bf16_from_double((double)acc);
    }
    return 0;
}

/* Per-group quant alone, of a bf16 [T,H] input: step 6 of the header on x. */
int oracle_quant_group(const uint16_t *x, int64_t T, int64_t H, int group, uint8_t *q,
                       float *scales) {
    if (!x || !q || !scales || T < 0 || H < 1 || group < 1 || H % group != 0) return -1;
    const int64_t G = H / group;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t g = 0; g < G; ++g) {
            const uint16_t *o = x + t * H + g * group;
            double amax = 0.0;
            for (int64_t h = 0; h < group; ++h) {
                double v = fabs(bf16_to_double(o[h]));
                if (v > amax || isnan(v)) amax = v;
                if (isnan(amax)) break;
            }
            float scale = (float)(amax / 448.0);
            scales[t * G + g] = scale;
            for (int64_t h = 0; h < group; ++h)
                q[t * H + g * group + h] =
                    scale == 0.0f ? 0x00u : oracle_e4m3fn_from_double((double)(bf16_to_float(o[h]) / scale));
        }
    }
    return 0;
}

/*
 * MXFP4 output (the third one-stage variant named in "Fix: add missing end_sync barrier
 * in fused allreduce+rmsnorm kernel", Copilot overview: the MXFP4 1-stage variant). The
 * pages name the format only; it is written here from the OCP Microscaling Formats (MX)
 * v1.0 specification:
 *   - blocks of 32 consecutive elements along H share one scale X = 2^s of type E8M0
 *     (an 8-bit biased exponent, bias 127, 0xFF = NaN);
 *   - s = floor(log2(max |V_i|)) - emax, emax = 2 for the FP4 E2M1 element type (its
 *     largest normal is 6 = 1.5 * 2^2), clamped to the E8M0 range [-127, 127];
 *   - each element P_i = V_i / X rounded to E2M1 (1 sign, 2 exponent bits with bias 1,
 *     1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), round to nearest even, magnitudes
 *     above 6 clamped to 6.
 * Readings (the spec or the pages leave these open): V is the bf16 `out`; an all-zero
 * block gets s = -127 (byte 0x00) and zero codes; a block holding a NaN gets the NaN
 * scale 0xFF and zero codes; two codes per byte, element 2i in the low nibble; scales
 * are bytes [T, H/32] row-major.
 */

/* E2M1 code of a binary64 value, one rounding to nearest even, saturating to +-6. */
uint8_t oracle_e2m1_from_double(double x) {
    const uint8_t sign = signbit(x) ? 0x8u : 0u;
    double a = fabs(x);
    if (isnan(x)) return 0; /* not reached: NaN blocks are handled by the caller */
    if (a >= 6.0) return (uint8_t)(sign | 0x7u);
    /* quantum: 0.5 below 2, 1 in [2,4), 2 in [4,8) */
    double quantum = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
    double r = nearbyint(a / quantum) * quantum; /* ties to even multiple of the quantum */
    static const double values[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (uint8_t c = 0; c < 8; ++c)
        if (values[c] == r) return (uint8_t)(sign | c);
    return (uint8_t)(sign | 0x7u); /* r == 8 (from [7, 8)): clamp to 6 */
}

void oracle_e2m1_from_double_array(const double *x, uint8_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_e2m1_from_double(x[i]);
}

/* MXFP4 of a bf16 [T,H] input: q [T, H/2] bytes (two codes each), scales [T, H/32] E8M0 bytes. */
int oracle_mxfp4(const uint16_t *x, int64_t T, int64_t H, uint8_t *q, uint8_t *scales) {
    if (!x || !q || !scales || T < 0 || H < 32 || H % 32 != 0) return -1;
    const int64_t B = H / 32;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < B; ++b) {
            const uint16_t *v = x + t * H + b * 32;
            double amax = 0.0;
            int has_nan = 0;
            for (int i = 0; i < 32; ++i) {
                double a = fabs(bf16_to_double(v[i]));
                if (isnan(a)) has_nan = 1;
                else if (a > amax) amax = a;
            }
            uint8_t codes[32];
            if (has_nan) {
                scales[t * B + b] = 0xFFu;
                for (int i = 0; i < 32; ++i) codes[i] = 0;
            } else if (amax == 0.0) {
                scales[t * B + b] = 0x00u;
                for (int i = 0; i < 32; ++i) codes[i] = 0;
            } else {
                int e2;
                frexp(amax, &e2);       /* amax in [2^(e2-1), 2^e2) */
                int s = (e2 - 1) - 2;   /* floor(log2 amax) - emax */
                if (s < -127) s = -127;
                if (s > 127) s = 127;
                scales[t * B + b] = (uint8_t)(s + 127);
                for (int i = 0; i < 32; ++i) codes[i] = oracle_e2m1_from_double(ldexp(bf16_to_double(v[i]), -s));
            }
            for (int i = 0; i < 16; ++i)
                q[t * (H / 2) + b * 16 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
    return 0;
}

/* The fused call with MXFP4 output: steps 1-5, then MXFP4 of the bf16 out. `out` may be NULL. */
int oracle_reduce_add_rmsnorm_mxfp4(const uint16_t *const *partials, int R, const uint16_t *residual,
                                    const uint16_t *gamma, float eps, int64_t T, int64_t H,
                                    uint16_t *residual_out, uint16_t *out, uint8_t *q, uint8_t *scales,
                                    int nthreads) {
    if (H % 32 != 0 || !q || !scales) return -1;
    uint16_t *o = out ? out : (uint16_t *)malloc((size_t)(T * H > 0 ? T * H : 1) * sizeof(uint16_t));
    if (!o) return -2;
    int rc = oracle_reduce_add_rmsnorm(partials, R, residual, gamma, eps, T, H, residual_out, o, nthreads);
    if (rc == 0) rc = oracle_mxfp4(o, T, H, q, scales);
    if (!out) free(o);
    return rc;
}
