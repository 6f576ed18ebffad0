/*
 * farn.h - C ABI of the fused reduce + residual-add + RMSNorm (+ per-group FP8
 * quant) op for AMD Instinct MI355X (gfx950).
 *
 * The op is the per-GPU body of a tensor-parallel all-reduce fused with the
 * residual add and RMSNorm that follows it, with the R rank partial-sum buffers
 * read from device memory. The pages' Python forms of the call are:
 *   - fused_ar_rms(inp, res_inp, *, w, eps, registered, use_1stage) returning
 *     (normalised output, all-reduce + residual output):
 *     "ROCm AITER fused all-reduce + RMSNorm" (vLLM #37646 summary),
 *     AiterCustomAllreduceProto and _rocm_aiter_fused_allreduce_rmsnorm_impl;
 *   - tensor_model_parallel_fused_allreduce_rmsnorm_quant_per_group(x, residual,
 *     weight, eps, group_size=128, emit_bf16) returning FP8 codes, per-group
 *     scales, the residual output and optionally the bf16 output, or None when
 *     the fused path cannot run: "AMD fused AllReduce-RMSNorm quant kernel"
 *     (sglang #24651 summary), layernorm.py snippet.
 * This ABI keeps their arguments, replaces the communicator with R explicit
 * partial pointers and the returned tuples with named output pointers, and
 * replaces "return None" with a status code.
 *
 * Arithmetic of one call, per token row t (h = 0..H-1):
 *   acc   = P_0[t,h]; acc += P_r[t,h] for r = 1..R-1     fp32 adds, rank order
 *   y     = acc + residual[t,h]                          fp32 (no add if residual == NULL)
 *   residual_out[t,h] = bf16_rne(y)
 *   rstd  = 1 / sqrt(sum_h residual_out[t,h]^2 / H + eps)   fp64: sum in a fixed reduction
 *           tree, the mean by one fp64 FMA, the reciprocal square root within two fp64 units
 *   out[t,h] = bf16_rne((residual_out[t,h] * rstd) * gamma[h])   one rounding of the product
 *           (formed in fp32 where that provably gives the same bf16 value, else in fp64)
 * and for the quant call, per group g of 128 channels:
 *   scale[t,g] = amax_g |out| / 448  (fp32, correctly rounded)
 *   q[t,h]     = e4m3fn_rne(fl32(out[t,h] / scale[t,g]))  (OCP E4M3, satfinite; 0 when
 *                scale == 0; the quotient as an IEEE single division gives it, then one
 *                rounding to E4M3; a -0 out gives the -0 code 0x80; a group holding a NaN
 *                out has a NaN scale and NaN codes, 0x7F or 0xFF)
 *
 * Layout: every [T,H] buffer is row-major and contiguous (row stride H
 * elements); bf16 values are passed as raw 16-bit patterns; q holds one E4M3
 * byte per element; scales is fp32 [T, H/128] row-major.
 *
 * Ownership: the caller allocates and frees every buffer; the library never
 * allocates, frees, synchronises, or keeps state between calls. Work is
 * enqueued asynchronously on `stream` (a hipStream_t; NULL = default stream).
 *
 * Errors: every argument check runs on the host before anything is enqueued; a
 * non-OK status means no work was enqueued (the analogue of the pages' "None,
 * caller falls back"). T == 0 returns FARN_OK and enqueues nothing; the [T,H]
 * buffers may then be NULL (gamma and the partials array may not).
 * FARN_ERR_LAUNCH is returned when a kernel launch itself fails. A call whose
 * rows need more than one launch (T x lanes above 2^32 - 1 work-items, e.g.
 * T >= 4,194,304 at H = 8192) may then have enqueued its earlier row chunks.
 */
#ifndef FARN_H
#define FARN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum farn_status {
    FARN_OK = 0,
    FARN_ERR_NULL = 1,    /* a required pointer is NULL */
    FARN_ERR_SHAPE = 2,   /* R not in [1, FARN_MAX_R]; T < 0 or T > 2^40; H <= 0, H % 8 != 0 or
                             H > FARN_MAX_H; FP8 quant: group_size != 128 or H % 128 != 0;
                             MXFP4: H % 32 != 0 */
    FARN_ERR_ALIGN = 3,   /* a bf16 / q buffer is not 16-byte aligned, or scales not 4-byte aligned */
    FARN_ERR_ALIAS = 4,   /* an output overlaps an input or another output (the one allowed
                             overlap: residual_out == residual exactly, in place) */
    FARN_ERR_EPS = 5,     /* eps is not finite or is negative */
    FARN_ERR_LAUNCH = 6,  /* the kernel launch failed */
    FARN_ERR_VARIANT = 7  /* unknown variant or option bit in an _ex call, or column-major
                             scales asked of a call without FP8 scales */
} farn_status;

/* Largest TP degree the pages run is 8 ("[AMD] Support --enable-aiter-allreduce-fusion
   on AMD GPUs", Commands Used: --tp 8). */
#define FARN_MAX_R 8
/* A row is held in registers: up to 1024 lanes x 4 vectors of 8 bf16. */
#define FARN_MAX_H 32768
/* Quant group along H ("per-1x128", group_size=128 in the sglang #24651 summary). */
#define FARN_GROUP 128
/* MXFP4 block along H (OCP Microscaling Formats (MX) v1.0: 32 elements per shared scale). */
#define FARN_MX_BLOCK 32
#define FARN_ABI_VERSION 4

/*
 * Plain call: reduce + residual add + RMSNorm.
 *   partials      host array of R device pointers, each bf16 [T,H]; may alias each other
 *   R             number of rank partials, 1..FARN_MAX_R
 *   residual      device bf16 [T,H], or NULL for no residual
 *   gamma         device bf16 [H]
 *   eps           added to the mean of squares inside the square root (1e-6 typical)
 *   T, H          tokens and hidden size
 *   residual_out  device bf16 [T,H]; may equal residual (in place)
 *   out           device bf16 [T,H]
 *   stream        hipStream_t or NULL
 */
farn_status farn_reduce_add_rmsnorm(const void *const *partials, int R, const void *residual,
                                    const void *gamma, float eps, int64_t T, int64_t H,
                                    void *residual_out, void *out, void *stream);

/*
 * FP8 call: the plain call, then per-group E4M3 quant of the bf16 output.
 *   group_size    must be FARN_GROUP (128); H % 128 == 0
 *   residual_out  device bf16 [T,H]; may equal residual
 *   out           device bf16 [T,H], or NULL to not write the bf16 output (emit_bf16 off)
 *   q             device uint8 [T,H], E4M3 codes
 *   scales        device fp32 [T, H/128]
 */
farn_status farn_reduce_add_rmsnorm_quant_group(const void *const *partials, int R,
                                                const void *residual, const void *gamma, float eps,
                                                int64_t T, int64_t H, int group_size,
                                                void *residual_out, void *out, void *q,
                                                float *scales, void *stream);

/*
 * MXFP4 call: the plain call, then MXFP4 of the bf16 output - the third one-stage
 * variant of the fused kernel ("Fix: add missing end_sync barrier in fused
 * allreduce+rmsnorm kernel", Copilot overview, names it). Format from the OCP
 * Microscaling Formats (MX) v1.0 specification: per row and block b of 32 channels,
 *   scales[t,b] = E8M0 byte s + 127, s = floor(log2(max |out|)) - 2, clamped to
 *                 [-127, 127]; 0xFF (NaN) if the block holds a NaN; 0x00 if it is all zero
 *   code        = E2M1 of out / 2^s, round to nearest even, magnitudes above 6 clamped to 6
 *                 (0 for NaN and zero blocks)
 *   q[t, i]     = code of channel 2i in bits 0-3, code of channel 2i+1 in bits 4-7
 *   H % 32 == 0; q device uint8 [T, H/2] (16-byte aligned); scales device uint8 [T, H/32];
 *   out device bf16 [T,H] or NULL (bf16 output not written).
 */
farn_status farn_reduce_add_rmsnorm_mxfp4(const void *const *partials, int R, const void *residual,
                                          const void *gamma, float eps, int64_t T, int64_t H,
                                          void *residual_out, void *out, void *q, void *scales,
                                          void *stream);

/* Launch shapes of the one kernel (one workgroup per token row; H/8 16-byte vectors per row):
 *   FARN_VARIANT_WIDE   (1, also named FARN_VARIANT_LATENCY): one vector per lane, H/8 lanes
 *                       rounded up to a multiple of 64 (up to 1024 lanes at H = 8192); beyond
 *                       H = 8192, two vectors per lane up to H = 16384 and four beyond, on H/16
 *                       or H/32 lanes rounded up to a multiple of 64 (at most 1024). The fewest
 *                       instructions per lane.
 *   FARN_VARIANT_NARROW (2, also named FARN_VARIANT_BANDWIDTH): about half as many lanes with
 *                       two vectors each, for 1024 < H <= 8192 (the WIDE launch otherwise):
 *                       twice the loads in flight per lane, half the waves per row.
 * The older names describe launch widths, not regimes: both shapes serve every T. AUTO
 * (farn_select_variant) picks by measurement on MI355X. It takes NARROW for
 *   - 6144 < H <= 8192, except the plain call with H > 7168 from T = 4096;
 *   - 4608 < H <= 5120 with 768 <= T < 2048;
 *   - the FP8 call with 2048 < H <= 6144 and T < 768, when H <= 3712 from T = 80 or
 *     256 <= T < 512;
 *   - R <= 4 and 2048 < H <= 6144 with 512 <= T < 768 (R <= 2: T < 1536);
 * and WIDE everywhere else. Both compute the same results (their fp64 sums of squares differ
 * only in the order of additions). */
typedef enum farn_variant {
    FARN_VARIANT_AUTO = 0,
    FARN_VARIANT_WIDE = 1,
    FARN_VARIANT_NARROW = 2,
    FARN_VARIANT_LATENCY = FARN_VARIANT_WIDE,
    FARN_VARIANT_BANDWIDTH = FARN_VARIANT_NARROW
} farn_variant;

/* Option bit of the _ex calls, or-ed into `variant`: FP8 scales laid out column-major,
   scales[g * T + t] for group g of row t ([H/128, T], the transposed per-token-group
   layout FP8 GEMMs read; the sglang #24651 summary's consumers take (fp8, scale) pairs
   and its related-PR notes mention scale layout utilities for AMD FP8). Requires
   T * H/128 * 4 < 2^31 bytes. */
#define FARN_SCALES_COL_MAJOR 0x100

/* As the calls above, with the launch shape forced (variant: a farn_variant, or-ed with
   option bits). For tests, the bench and callers that need an option. */
farn_status farn_reduce_add_rmsnorm_ex(const void *const *partials, int R, const void *residual,
                                       const void *gamma, float eps, int64_t T, int64_t H,
                                       void *residual_out, void *out, void *stream, int variant);
farn_status farn_reduce_add_rmsnorm_quant_group_ex(const void *const *partials, int R,
                                                   const void *residual, const void *gamma,
                                                   float eps, int64_t T, int64_t H, int group_size,
                                                   void *residual_out, void *out, void *q,
                                                   float *scales, void *stream, int variant);
farn_status farn_reduce_add_rmsnorm_mxfp4_ex(const void *const *partials, int R, const void *residual,
                                             const void *gamma, float eps, int64_t T, int64_t H,
                                             void *residual_out, void *out, void *q, void *scales,
                                             void *stream, int variant);

/*
 * Unfused building blocks: the kernels the fused calls replace. The sglang #24651
 * summary ("AMD fused AllReduce-RMSNorm quant kernel", layernorm.py snippet and
 * benchmark file list) falls back from the one-kernel AR + RMSNorm + quant to AR +
 * RMSNorm followed by a separate per-1x128 quant, and benchmarks 3-, 2- and 1-kernel
 * variants; the vLLM #37646 summary's unfused pattern is all-reduce then rms_norm.
 * With these, the 2-kernel path is farn_reduce_add_rmsnorm + farn_quant_group and the
 * 3-kernel path is farn_reduce + farn_reduce_add_rmsnorm (R = 1, the all-reduce output
 * as its one partial) + farn_quant_group. Results follow each block's own definition,
 * so the 3-kernel path rounds the all-reduce output to bf16 before the residual add.
 */

/* All-reduce alone: out[t,h] = bf16_rne(P_0 + ... + P_{R-1}), fp32 adds in rank order.
 *   partials  host array of R device pointers, bf16 [T,H]; out device bf16 [T,H] (may not
 *   overlap a partial). Same checks and status codes as the fused calls. */
farn_status farn_reduce(const void *const *partials, int R, int64_t T, int64_t H, void *out,
                        void *stream);

/* Per-group quant alone of a bf16 [T,H] input x: scales[t,g] = amax/448 over channels
 * [128g, 128g+128) of row t, q = E4M3 codes of fl32(x/scale) (as in the FP8 call;
 * satfinite, 0 for a zero group). group_size must be 128; H % 128 == 0; q and scales may not overlap x. */
farn_status farn_quant_group(const void *x, int64_t T, int64_t H, int group_size, void *q,
                             float *scales, void *stream);

/* The variant AUTO would run for this shape (no validation; pure function of its arguments).
 * quant: 0 for the plain call, 1 for the FP8 call, 2 for the MXFP4 call. */
int farn_select_variant(int R, int64_t T, int64_t H, int quant);

/* Static, NUL-terminated description of a status code. */
const char *farn_status_string(int status);

int farn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FARN_H */
