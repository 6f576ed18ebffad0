// HIP kernels for gfx950 (CDNA4): fused reduce of R rank partials + residual add +
// RMSNorm (+ per-128-channel E4M3 quant, or MXFP4), one token row at a time.
//
// The op is the per-GPU body of the fused tensor-parallel all-reduce + RMSNorm of
// "ROCm AITER fused all-reduce + RMSNorm" (vLLM #37646 summary: all-reduce, then
// rms_norm of its output, both returned) and of the per-group FP8 variant in "AMD
// fused AllReduce-RMSNorm quant kernel" (sglang #24651 summary: group_size 128,
// quant of the bf16 normalised output). Here the R partial buffers sit in local HBM.
//
// Work mapping:
//   One workgroup per token row, grid = T (in several launches of consecutive rows when
//   T x L exceeds a dispatch's 2^32 - 1 work-items). A row of H bf16 is NV = H/8 16-byte vectors,
//   spread over L lanes (a multiple of 64, <= 1024) with VPL vectors per lane,
//   lane-strided: lane l holds vectors l, l+L, l+2L, ... So every load instruction of a
//   wave is 64 lanes x 16 B = 1 KiB contiguous, and a 128-channel quant group is
//   exactly 16 consecutive lanes (one DPP row) of one vector slot.
//   Per lane: with one or two slots the source issues the loads of all of them before
//   consuming any (the compiler may still sink some below the first slot's fold; rows
//   beyond 16384 channels, four slots, load one slot at a time); the partials are summed
//   in fp32 in rank order, the residual added last, the sum rounded to bf16
//   (residual_out) and kept packed in registers. The sum of squares
//   (fp64) goes lane -> 16-lane DPP butterfly -> 4 rows via readlane -> one double
//   per wave through LDS -> each lane reads one wave's value and a 16-lane butterfly
//   adds them (the same fixed order in every wave); the
//   normalisation product is rounded once to bf16 (formed in fp32 where that provably
//   gives the same value, else in fp64). The row never passes through LDS; only one
//   double per wave does.
//
// Two launch shapes of the same kernel (chosen by the host from R, T and H, as measured):
//   wide   - the widest row mapping (L up to 1024, one vector per lane up to H = 8192; beyond,
//            two or four per lane on as few lanes as cover the row): the fewest instructions
//            per lane.
//   narrow - L about NV/2, two vectors per lane: half the waves per row, twice the loads in
//            flight per lane. On MI355X it is the faster one for H = 6152 .. 8192 (the FP8
//            prefill call at H = 7168 by 3-4 %, decode by 5-9 %), at H = 4616 .. 5120 for
//            768 <= T < 2048, for much of the FP8 call at H = 2056 .. 6144 below T = 768, and
//            with up to four ranks at mid-size T.
// The fp64 statistics make the two shapes agree bit for bit in practice (their sums of
// squares differ only in the order of fp64 additions). The two-slot quant kernels also have
// two store schedules, one for many rows and one for few (do_row). The host may reserve LDS
// that the kernel does not use (Call::lds_reserve) to bound how many workgroups share a
// compute unit: the streaming FP8 and MXFP4 two-slot kernels run faster at large T with two
// per compute unit than with the three their registers allow.
//
// No MFMA: nothing here is a contraction; the op is HBM-bound (about 0.5 flop per
// byte against a ridge of ~20 flop/byte).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "farn_device_math.h"
#include "farn_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

struct Params {
    const void *p[8];   // rank partials, bf16 [T,H]
    const void *res;    // residual or null
    const void *gamma;  // [H]
    void *res_out;
    void *out;          // null: bf16 output not written (quant call only)
    void *q;            // E4M3 codes [T,H] (FP8), or E2M1 code pairs [T,H/2] (MXFP4)
    void *scales;       // fp32 [T, H/128] (FP8), or E8M0 bytes [T, H/32] (MXFP4)
    const void *x;      // bf16 [T,H] input of the standalone quant kernel
    int scale_cols;     // FP8 scales column-major [H/128, T] (else row-major [T, H/128])
    int64_t T;
    int64_t t0;         // row of this launch's first workgroup
    int nvec;           // H / 8
    int ngroups;        // H / 128
    double h;           // H (mean divisor)
    double inv_h;       // 1 / H
    float eps;
};

constexpr int kMaxWaves = 16;
static_assert(kMaxWaves == 16, "the per-wave values are read by one 16-lane DPP row");

// Output quant modes of the fused kernel.
constexpr int kQuantNone = 0;   // bf16 out only
constexpr int kQuantFp8 = 1;    // + E4M3 codes and fp32 scales per 128 channels
constexpr int kQuantMxfp4 = 2;  // + E2M1 code pairs and E8M0 scales per 32 channels

// ---------------------------------------------------------------- buffer access
// Every global access goes through a buffer resource covering exactly one row of one
// array. The hardware range check turns a load past the end of the row (lanes beyond
// H/8, or a row >= T, whose resource has 0 records) into zeros and drops such a store,
// so no access needs a branch: the loads of a row are issued straight-line and the
// compiler's vmcnt bookkeeping stays exact across the software pipeline.
// dword3 0x00020000: 32-bit data format, the raw-buffer setting for CDNA.
constexpr int kRsrcFlags = 0x00020000;
// Cache policies (gfx950 cache-policy bits: sc0 = 1, nt = 2, sc1 = 16), chosen by
// measurement of this traffic mix (9 read streams, 2 bf16 write streams, 1 byte
// stream) on MI355X: row loads non-temporal, bf16 stores system-scope (sc1), E4M3 code
// stores non-temporal. With no arithmetic at all this mix then moves 80% of peak
// HBM bandwidth, against 75% with every access non-temporal and 66% with none.
constexpr int kLoadPolicy = 2;
// gamma is read by every row's workgroup: default policy, so it stays in L2. Non-temporal
// gamma loads (re-fetched per row) measured 2-14 % slower at decode sizes from HBM and
// 0.6 % on the FP8 prefill chunk.
constexpr int kGammaLoadPolicy = 0;
constexpr int kStoreBf16Policy = 16;
constexpr int kStoreCodePolicy = 2;
// FP8 codes and scales of the two-slot kernel's small-call schedule (few rows): sc1.
constexpr int kStoreCodeSmallPolicy = 16;
// MXFP4 codes and scale bytes: sc1 (measured: -0.4 % on the prefill chunk, -3.5 % at decode
// against non-temporal; for the FP8 codes non-temporal is the faster one by 3.5-7 %).
constexpr int kStoreMxPolicy = 16;
constexpr uint32_t kDropOffset = 0x80000000u;  // beyond any row: store dropped

__device__ __forceinline__ rsrc_t row_rsrc(const void *base, int64_t byte_off, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + byte_off), (short)0,
                                             nbytes, kRsrcFlags);
}
__device__ __forceinline__ u32x4 ld16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadPolicy);
}
__device__ __forceinline__ void st16(u32x4 v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStoreBf16Policy);
}
template <int P>
__device__ __forceinline__ void st8(u32x2 v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, P);
}
template <int P>
__device__ __forceinline__ void st4(float v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, P);
}
__device__ __forceinline__ void st4_mx(uint32_t v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kStoreMxPolicy);
}
__device__ __forceinline__ void st1_mx(uint32_t v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, r, off, 0, kStoreMxPolicy);
}

// ---------------------------------------------------------------- number formats
// Float classes for v_cmp_class: positive normal, and normal of either sign.
constexpr int kClassPosNormal = 1 << 8;
constexpr int kClassNormal = (1 << 3) | (1 << 8);
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = bf16x2{(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// fp64 -> fp32 rounded to odd: truncate toward zero, then set the last bit if anything
// was dropped. A value rounded to odd with 24 bits and then to nearest-even with 8 bits
// lands where one direct rounding to 8 bits would, so fp64 -> bf16 rounds once.
// Branch-free: the nearest-even result steps back one unit when it rounded away from
// zero, and the sticky bit is or-ed in when the conversion was inexact.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
    const float f = (float)d;  // nearest even
    const double back = (double)f;
    const uint32_t inexact = back != d ? 1u : 0u;
    const uint32_t away = __builtin_fabs(back) > __builtin_fabs(d) ? 1u : 0u;
    return __uint_as_float((__float_as_uint(f) - away) | inexact);
}

// Two fp64 -> packed bf16 pair, each rounded once to nearest even.
__device__ __forceinline__ uint32_t pack_bf16_d(double lo, double hi) {
    return pack_bf16(f64_to_f32_odd(lo), f64_to_f32_odd(hi));
}

// FP8 and FP4 codes come from gfx950's conversion instructions:
//   v_cvt_pk_fp8_f32 (two fp32 -> two OCP E4M3 codes): round to nearest even; values at
//     or above 464 in magnitude, inf and NaN give a NaN code (no saturation).
//   v_cvt_scalef32_pk_fp4_f32 (two fp32 times 2^-e -> two OCP E2M1 codes, e the exponent
//     of the scale operand): round to nearest even code, magnitudes above 6 saturate to 6.
// Both were checked exhaustively against the format definitions on MI355X: every
// non-negative fp32 value below 464 (and the negatives down to -464) for E4M3, every bf16
// value under every block exponent -127..127 for E2M1 (tests/test_gpu_conversions.py
// repeats the checks).

// The binary32 quotient o / scale without a divide (inv = 1/scale): q0 = o * inv, the
// remainder by one FMA, one correction by another (Markstein's FMA correction of a
// reciprocal product). The result can sit one fp32 unit off the correctly rounded
// quotient, but never where that changes its E4M3 code: for every bf16 amax and every bf16
// o the group can hold (tiny groups rescaled by the caller) the codes agree (checked on the
// CPU over all 1.07e9 such pairs, tests/test_encoder_models.py).
// The remainder is taken negated, nr = q0 * scale - o, and the correction is q0 - nr * inv:
// the same value as q0 + (o - q0 * scale) * inv for every o (round to nearest is symmetric),
// and a -0 input keeps its sign (-0 - (+0) = -0, where -0 + (+0) would give +0), so its code
// is the -0 code 0x80, as the division gives.
// scale_r is scale, or the largest finite float for an inf scale (so that the remainder of
// a finite o is -o rather than 0 * inf = NaN).
__device__ __forceinline__ float fp32_quotient(float o, float scale_r, float inv) {
#pragma clang fp contract(off)
    const float q0 = o * inv;
    const float nr = __builtin_fmaf(q0, scale_r, -o);
    return __builtin_fmaf(-nr, inv, q0);
}

// ---------------------------------------------------------------- cross-lane
// DPP controls (gfx9): quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140. After the four steps every lane of a
// 16-lane row holds the row's total, identical in every lane (each step adds the
// same pair in both lanes, and fp32 addition is commutative).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// fp64 through DPP: the two 32-bit halves move with the same control. Every control used
// here reads a lane inside the same 16-lane row, so all lanes are written and no previous
// value of the destination is needed (bound_ctrl set, full masks).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double row16_sum_d(double x) {
    x = x + dpp_d<0xB1>(x);
    x = x + dpp_d<0x4E>(x);
    x = x + dpp_d<0x141>(x);
    x = x + dpp_d<0x140>(x);
    return x;
}

__device__ __forceinline__ double readlane_d(double x, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Wave total: the four 16-lane row totals, read as scalars and added in a fixed order.
__device__ __forceinline__ double wave_sum_d(double x) {
    x = row16_sum_d(x);
    return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}

// ---------------------------------------------------------------- one row
// The loads of one vector slot: R partials and the residual (zeros when absent).
template <int R>
struct SlotIn {
    u32x4 p[R];
    u32x4 res;
};

// Issue the R+1 loads of slot byte offset `off` of row t. A row t >= T loads zeros.
template <int R>
__device__ __forceinline__ void load_slot(SlotIn<R> &in, const Params &k, int64_t t, uint32_t off) {
    const int rb = t < k.T ? k.nvec * 16 : 0;
    const int64_t ro = t * (int64_t)k.nvec * 16;
#pragma unroll
    for (int r = 0; r < R; ++r) in.p[r] = ld16(row_rsrc(k.p[r], ro, rb), off);
    in.res = ld16(row_rsrc(k.res, k.res ? ro : 0, k.res ? rb : 0), off);
}

// Forms of the fold (the same sums; they differ in instructions and so in how the compiler
// schedules the row's loads around them):
//   kFoldSelect  - the residual term added, then the sum with or without it selected
//   kFoldNegZero - with no residual the zero words loaded in its place are unpacked as -0 (the
//                  sign bit or-ed in; x + (-0) is x for every x, -0 and NaN included), no select
//   kFoldNegZeroReg - the same with the high-half mask in a register, so that mask-and-or is one
//                  instruction (a three-operand instruction cannot take the 32-bit constant
//                  itself on this target)
//   kFoldNoResidual - no residual term (the standalone all-reduce)
// Chosen per kernel by measurement on MI355X (do_row).
constexpr int kFoldSelect = 0;
constexpr int kFoldNegZero = 1;
constexpr int kFoldNegZeroReg = 2;
constexpr int kFoldNoResidual = 3;

// fp32 sum of the partials in rank order, residual last (a missing residual adds nothing, so a
// -0 sum stays -0), rounded to bf16: four packed pairs. Lanes past the row end see zeros.
template <int R, int kFold>
__device__ __forceinline__ u32x4 fold_slot(const SlotIn<R> &in, bool has_res) {
    const uint32_t zsign = has_res ? 0u : 0x80000000u;
    uint32_t hmask = 0xffff0000u;
    if constexpr (kFold == kFoldNegZeroReg) __asm__("v_mov_b32 %0, 0xffff0000" : "=v"(hmask));
    u32x4 packed;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float lo = bf_lo(in.p[0][w]);
        float hi = bf_hi(in.p[0][w]);
#pragma unroll
        for (int r = 1; r < R; ++r) {
            lo = lo + bf_lo(in.p[r][w]);
            hi = hi + bf_hi(in.p[r][w]);
        }
        if constexpr (kFold == kFoldSelect) {
            const float lo_r = lo + bf_lo(in.res[w]);
            const float hi_r = hi + bf_hi(in.res[w]);
            lo = has_res ? lo_r : lo;
            hi = has_res ? hi_r : hi;
        } else if constexpr (kFold != kFoldNoResidual) {
            lo = lo + __uint_as_float((in.res[w] << 16) | zsign);
            hi = hi + __uint_as_float((in.res[w] & hmask) | zsign);
        }
        packed[w] = pack_bf16(lo, hi);
    }
    return packed;
}

// fold_slot, stored as residual_out here (kStoreNow) or by the caller later, with the squares
// of the rounded values added to ss (fp64; zeros from lanes past the row end add nothing).
template <int R, bool kStoreNow, int kFold>
__device__ __forceinline__ u32x4 reduce_slot(const SlotIn<R> &in, const Params &k, rsrc_t ro_out,
                                             uint32_t off, double &ss) {
    const u32x4 packed = fold_slot<R, kFold>(in, k.res != nullptr);
    if constexpr (kStoreNow) st16(packed, ro_out, off);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const double a = (double)bf_lo(packed[w]);
        const double b = (double)bf_hi(packed[w]);
        ss = __builtin_fma(a, a, ss);  // bf16 squares are exact in fp64
        ss = __builtin_fma(b, b, ss);
    }
    return packed;
}

// Row statistics in fp64: wave DPP tree, one double per wave through `slot` (kMaxWaves
// doubles; wave 0 sets the slots past the row's waves to zero), one barrier, then lane l of
// every wave reads slot l mod 16 and the 16-lane DPP butterfly adds them, in one fixed order
// for every wave and lane (one LDS read after the barrier rather than one per wave, read one
// after another: 1-5 % off a decode call); then rstd = 1/sqrt(m) for m = ss/H + eps. fp64
// statistics put `out` on the bf16 value the exact statistics give (an fp32 tree moves about
// one element in 10^4 by one bf16 step, and when that element is a group's amax its scale
// moves by up to 2^-7); MI355X runs fp64 vector FMAs at the rate of unpacked fp32 ones.
// m is formed as ss * (1/H) + eps by one FMA, and 1/sqrt(m) as the hardware reciprocal
// square root (about 24 correct bits, measured) refined by two Newton steps
// (y += y * (1/2 - m y^2 / 2)): the result sits within two fp64 units of the correctly
// rounded 1/sqrt (one step leaves up to ~20), far below what the bf16 outputs resolve, and
// the row's dependent chain after the barrier is some 25 fp64 operations shorter than with a
// division and a square root. Outside 2^-1000 <= m <= 2^1000 (and for an inf or NaN m) the
// division and square root are used.
__device__ __forceinline__ double row_rstd(double ss, const Params &k, double *slot) {
    const int lane = (int)threadIdx.x & 63;
    const int wave = (int)threadIdx.x >> 6;
    const int nwaves = (int)blockDim.x >> 6;
    const double wsum = wave_sum_d(ss);
    if (lane == 0) slot[wave] = wsum;
    if (wave == 0 && lane >= nwaves && lane < kMaxWaves) slot[lane] = 0.0;
    __syncthreads();
    const double tot = row16_sum_d(slot[lane & (kMaxWaves - 1)]);
    const double m = __builtin_fma(tot, k.inv_h, (double)k.eps);
    double r;
    if (m >= 0x1p-1000 && m <= 0x1p1000) {  // the same in every lane of the row
        r = farn_math::rsq_newton(m);
    } else {
        __asm__ volatile("" ::: "memory");  // keeps this rare path a branch, not computed beside the other
        r = 1.0 / __builtin_sqrt(tot / k.h + (double)k.eps);
    }
    return r;
}

// E4M3 codes of N vector slots (8 bf16 values each, two per word of `ob`) and, from one lane
// per 16-lane group, each group's scale, stored at byte sbase + group * sstride of r_sc. The
// slots' steps are written side by side, so their dependent chains (group max, scale,
// reciprocal) overlap.
// The group's amax is a packed 16-bit max of the magnitude patterns (bf16 magnitudes
// order as unsigned integers, inf included, and a NaN, above inf, wins and propagates
// into the scale). Each code is the conversion of the binary32 quotient o / scale, sign
// included: for a finite scale |quotient| <= 448 * (1 + 2^-23) < 464, so the conversion
// never reaches its NaN range; an inf scale gives 0 for finite o and NaN for infinite o,
// a NaN scale NaN codes. An all-zero group has scale 0 and every code +0: inv = 0 keeps
// its lanes on the arithmetic path (their quotients are +-0) and a mask clears the signs.
// A group whose scale is below 2^-64 is quantised from o and scale both times 2^64 (exact;
// the quotient is the same), so that 1/scale and the remainder stay normal numbers; the
// stored scale is the unscaled one. 1/scale is the hardware reciprocal refined by one Newton
// step (y + y * (1 - s * y)), which equals the correctly rounded reciprocal for every scale
// a bf16 amax can produce (checked on the GPU for all of them); 1/inf = 0 and NaN come from
// the hardware reciprocal itself.
// kSkipRescale: when no group of the wave needs the 2^64 rescaling (every k is 1), a
// wave-uniform branch forms the quotients without the multiplications by k (the same values).
// Measured on MI355X for the one-slot kernels: FP8 calls at decode sizes 2.7-5 % faster; in
// the two-slot small-call kernel it gained nothing (-1.8 .. +2.6 %), so that one keeps the
// straight code.
template <int P, int N, bool kSkipRescale = false>
__device__ __forceinline__ void quant_slots(const u32x4 (&ob)[N], rsrc_t r_q, rsrc_t r_sc, const uint32_t (&off)[N],
                                            uint32_t sbase, uint32_t sstride) {
    uint32_t amax[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        u16x2 m = u16x2{0, 0};
#pragma unroll
        for (int w = 0; w < 4; ++w)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, ob[n][w] & 0x7fff7fffu));
        amax[n] = max((uint32_t)m[0], (uint32_t)m[1]);
    }
    // 16 lanes = one 128-channel group: a DPP butterfly of unsigned maxima (the magnitude
    // patterns of non-negative floats order as integers), slot by slot
#pragma unroll
    for (int n = 0; n < N; ++n) amax[n] = max(amax[n], dpp_u<0xB1>(amax[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) amax[n] = max(amax[n], dpp_u<0x4E>(amax[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) amax[n] = max(amax[n], dpp_u<0x141>(amax[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) amax[n] = max(amax[n], dpp_u<0x140>(amax[n])) << 16;
    float scale[N], k[N], inv[N], sr[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        scale[n] = farn_math::fp8_scale(amax[n]);  // amax/448, correctly rounded
        k[n] = scale[n] < 0x1p-64f ? 0x1p64f : 1.0f;
        const float sk = scale[n] * k[n];
        inv[n] = scale[n] == 0.0f ? 0.0f : farn_math::fp8_recip(sk);
        sr[n] = min(sk, 0x1.fffffep127f);
    }
    bool rescale = false;
    if constexpr (kSkipRescale) {
#pragma unroll
        for (int n = 0; n < N; ++n) rescale = rescale || k[n] != 1.0f;
        rescale = __builtin_amdgcn_ballot_w64(rescale) != 0;
    }
#pragma unroll
    for (int n = 0; n < N; ++n) {
        float v[8];
        if (kSkipRescale && !rescale) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                v[2 * w] = fp32_quotient(bf_lo(ob[n][w]), sr[n], inv[n]);
                v[2 * w + 1] = fp32_quotient(bf_hi(ob[n][w]), sr[n], inv[n]);
            }
        } else {
            // keeps the rare path a branch, not computed beside the other
            if constexpr (kSkipRescale) __asm__ volatile("" ::: "memory");
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                v[2 * w] = fp32_quotient(bf_lo(ob[n][w]) * k[n], sr[n], inv[n]);
                v[2 * w + 1] = fp32_quotient(bf_hi(ob[n][w]) * k[n], sr[n], inv[n]);
            }
        }
        const uint32_t keep = scale[n] == 0.0f ? 0u : 0xffffffffu;
        u32x2 codes;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d], v[4 * d + 1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d + 2], v[4 * d + 3], word, true);
            codes[d] = (uint32_t)word & keep;
        }
        st8<P>(codes, r_q, off[n] >> 1);
        // one lane per group writes the scale; the others aim past the row (dropped)
        const uint32_t soff = ((int)threadIdx.x & 15) == 0 ? sbase + (off[n] >> 8) * sstride : kDropOffset;
        st4<P>(scale[n], r_sc, soff);
    }
}

template <int P, bool kSkipRescale = false>
__device__ __forceinline__ void quant_slot(u32x4 ob, rsrc_t r_q, rsrc_t r_sc, uint32_t off, uint32_t sbase,
                                           uint32_t sstride) {
    const u32x4 obs[1] = {ob};
    const uint32_t offs[1] = {off};
    quant_slots<P, 1, kSkipRescale>(obs, r_q, r_sc, offs, sbase, sstride);
}

// MXFP4 of N vector slots from their packed bf16 values, the slots' steps written side by
// side: the 32-channel block spans the 4 lanes of a quad. Shared scale 2^s with
// s = floor(log2 amax) - 2 (E2M1's largest exponent), clamped to the E8M0 range; a block
// holding a NaN gets the NaN scale 0xFF and zero codes, an all-zero block scale 2^-127
// (byte 0) and zero codes. The block max is a packed 16-bit max of the bf16 magnitude
// patterns (they order as integers, and a NaN, above inf, wins), then two DPP steps. The
// conversion takes the scale as an fp32 whose exponent field is the E8M0 byte (s = -127 is
// the bit pattern 0), scales each value by 2^-s exactly and rounds it to E2M1; element 2i goes
// to the low nibble of its byte.
template <int N>
__device__ __forceinline__ void mxfp4_slots(const u32x4 (&ob)[N], rsrc_t r_q, rsrc_t r_sc,
                                            const uint32_t (&off)[N]) {
    uint32_t amax[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        u16x2 m = u16x2{0, 0};
#pragma unroll
        for (int w = 0; w < 4; ++w)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, ob[n][w] & 0x7fff7fffu));
        amax[n] = max((uint32_t)m[0], (uint32_t)m[1]) << 16;
    }
#pragma unroll
    for (int n = 0; n < N; ++n) amax[n] = max(amax[n], dpp_u<0xB1>(amax[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) amax[n] = max(amax[n], dpp_u<0x4E>(amax[n]));
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const bool nan_blk = amax[n] > 0x7f800000u;
        const bool zero_blk = amax[n] == 0u;
        int sexp = __builtin_amdgcn_frexp_expf(__uint_as_float(amax[n])) - 1 - 2;  // floor(log2 amax) - 2
        sexp = sexp < -127 ? -127 : (sexp > 127 ? 127 : sexp);
        const float sc = __uint_as_float((uint32_t)(sexp + 127) << 23);
        uint32_t word = 0u;
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf_lo(ob[n][0]), bf_hi(ob[n][0]), sc, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf_lo(ob[n][1]), bf_hi(ob[n][1]), sc, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf_lo(ob[n][2]), bf_hi(ob[n][2]), sc, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf_lo(ob[n][3]), bf_hi(ob[n][3]), sc, 3);
        const uint32_t keep = (nan_blk || zero_blk) ? 0u : 0xffffffffu;
        st4_mx(word & keep, r_q, off[n] >> 2);
        const uint32_t sbyte = nan_blk ? 0xffu : (zero_blk ? 0u : (uint32_t)(sexp + 127));
        // one lane per quad writes the scale byte; the others aim past the row (dropped)
        st1_mx(sbyte, r_sc, ((int)threadIdx.x & 3) == 0 ? (off[n] >> 6) : kDropOffset);
    }
}

// Normalised values of one vector slot, (y * rstd) * gamma each rounded once to bf16, packed.
// Fast path in fp32: yg = y * gamma is exact when it is a normal number (two 8-bit
// significands), and p = fl32(yg * fl32(rstd)) then lies within 1.5 fp32 units of the fp64
// product (one rounding of rstd, one of the product; at most one more unit where p and the
// fp64 value straddle a power of two), so the bf16 rounding of p is the one-rounding result
// unless p is within 3 fp32 units of a bf16 midpoint: low 16 bits 0x7FFD .. 0x8003 (fp32
// subnormal results included, whose error is below one unit). When any lane of the wave
// has such a p, a yg that is not a normal number (zero, subnormal, inf, NaN) or the row an
// rstd whose fp32 rounding is not normal, the wave redoes the slot in fp64: the product in
// fp64, rounded to odd to fp32, then to nearest-even bf16 (one rounding). On random data
// about one slot in twenty takes that path.
__device__ __forceinline__ u32x4 norm_slot(u32x4 yb, u32x4 gam, double rstd, float r32, bool r32_ok) {
    u32x4 packed;
    bool ok = r32_ok;
    uint16_t near_mid = 0xffff;  // min over the slot of (low 16 bits of p) - 0x7FFD, mod 2^16
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float ylo = bf_lo(yb[w]) * bf_lo(gam[w]);
        const float yhi = bf_hi(yb[w]) * bf_hi(gam[w]);
        ok = ok && __builtin_amdgcn_classf(ylo, kClassNormal) && __builtin_amdgcn_classf(yhi, kClassNormal);
        const float plo = ylo * r32;
        const float phi = yhi * r32;
        near_mid = min(near_mid, (uint16_t)(__float_as_uint(plo) - 0x7FFDu));
        near_mid = min(near_mid, (uint16_t)(__float_as_uint(phi) - 0x7FFDu));
        packed[w] = pack_bf16(plo, phi);
    }
    if (__builtin_amdgcn_ballot_w64(!ok || near_mid <= 6) != 0) {
        __asm__ volatile("" ::: "memory");  // keeps the fp64 path a branch, not computed beside the fast one
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const double lo = ((double)bf_lo(yb[w]) * rstd) * (double)bf_lo(gam[w]);
            const double hi = ((double)bf_hi(yb[w]) * rstd) * (double)bf_hi(gam[w]);
            packed[w] = pack_bf16_d(lo, hi);
        }
    }
    return packed;
}

// Normalise one vector slot and store it as out; returns the packed bf16 values (the FP8 and
// MXFP4 quants' input).
__device__ __forceinline__ u32x4 norm_store(u32x4 yb, u32x4 gam, double rstd, float r32, bool r32_ok,
                                            rsrc_t r_out, uint32_t off) {
    const u32x4 packed = norm_slot(yb, gam, rstd, r32, r32_ok);
    st16(packed, r_out, off);
    return packed;
}

// gamma of the vector slot at byte offset `off`. The four-slot kernels (rows beyond 16384
// channels, launch bound 1024 lanes, so at most 128 VGPRs per lane) load it slot by slot when they
// normalise instead of holding all four slots' gamma through the row: measured on MI355X, that
// removes their register spills (28-44 bytes per lane) and makes them 3-10 % faster.
__device__ __forceinline__ u32x4 gamma_slot(const Params &k, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(k.gamma, 0, k.nvec * 16), off, 0, kGammaLoadPolicy);
}

// Whole row t with the loads of slot 0 already issued into `in0`. With two slots per
// lane the source issues the second slot's loads before reducing the first; with four
// (rows beyond 16384 channels) the slots are loaded and reduced one after the other, and each
// slot's gamma is loaded when it is normalised, to bound register use.
template <int R, int VPL, int QM, bool kSmall>
__device__ __forceinline__ void do_row(const SlotIn<R> &in0, const u32x4 (&gam)[VPL],
                                       const Params &k, int64_t t, double *slot) {
    const uint32_t L16 = blockDim.x * 16u;
    const uint32_t off0 = threadIdx.x * 16u;
    const int rb = k.nvec * 16;
    const int64_t ro = t * (int64_t)rb;
    const rsrc_t r_ro = row_rsrc(k.res_out, ro, rb);
    // Store schedule, chosen by measurement on MI355X. The plain two-slot kernel stores
    // residual_out with out, after the statistics, rather than between the two slots' folds
    // while slot 1's loads are in flight: 5-8 % faster at decode sizes (H = 7168, 8192),
    // 2-14 % at T = 128 .. 2048 (R = 8, H = 7168; at H = 8192 3.6-11 % up to T = 384, within
    // 0.7 % from T = 512) and ~1 % on the prefill chunk. The one-slot kernels store it as soon
    // as it is folded (1-3 % faster that way). The two-slot quant kernels have two schedules: the streaming one
    // (immediate residual_out, each slot's codes right after its out, FP8 codes
    // non-temporal) for many rows, and kSmall (residual_out after the statistics, FP8: all of
    // out before the codes, codes and scales sc1) for few rows, where it is 4-15 % faster
    // (T = 16 .. 256) and from T = 1024 2-6 % slower.
    constexpr bool kDefer = VPL == 2 && (QM == kQuantNone || kSmall);
    constexpr bool kOutsFirst = kSmall && QM == kQuantFp8 && VPL == 2;
    constexpr int kCodeP = kSmall ? kStoreCodeSmallPolicy : kStoreCodePolicy;
    // Fold form (measured, interleaved, median of 5, against the select in every kernel): the -0
    // unpack takes 1-3 % off FP8 and MXFP4 calls at decode sizes (up to 6 % at R = 4, T = 16,
    // H = 4096 from HBM) and 1-7 % off few-rank plain calls there; with the mask in a register in
    // the plain kernels, R = 8 calls of the two-slot kernel ran 1-4 % slower (other register
    // allocation); the two-slot streaming quant kernels keep the select (with the -0 unpack
    // 0.6 % slower on the FP8 and MXFP4 prefill chunk), and so does the plain kernel of a single
    // rank (0.4-3 % slower with it at H = 7168, T = 2048 and 8192). The four-slot kernels (rows
    // beyond 16384 channels, not measured) take the forms of the one-slot ones.
    constexpr int kFold = QM == kQuantNone ? (R == 1 ? kFoldSelect : kFoldNegZero)
                                           : (VPL == 2 && !kSmall ? kFoldSelect : kFoldNegZeroReg);
    double ss = 0.0;
    u32x4 yb[VPL];
    if constexpr (VPL == 2) {
        SlotIn<R> in1;
        load_slot<R>(in1, k, t, off0 + L16);
        yb[0] = reduce_slot<R, !kDefer, kFold>(in0, k, r_ro, off0, ss);
        yb[1] = reduce_slot<R, !kDefer, kFold>(in1, k, r_ro, off0 + L16, ss);
    } else {
        yb[0] = reduce_slot<R, true, kFold>(in0, k, r_ro, off0, ss);
#pragma unroll
        for (int v = 1; v < VPL; ++v) {
            SlotIn<R> in;
            load_slot<R>(in, k, t, off0 + v * L16);
            yb[v] = reduce_slot<R, true, kFold>(in, k, r_ro, off0 + v * L16, ss);
        }
    }
    const double rstd = row_rstd(ss, k, slot);
    const float r32 = (float)rstd;
    const bool r32_ok = __builtin_amdgcn_classf(r32, kClassPosNormal);
    const rsrc_t r_out = row_rsrc(k.out, k.out ? ro : 0, k.out ? rb : 0);
    // per-row code and scale bytes: FP8 H and 4*H/128; MXFP4 H/2 and H/32
    const int qb = QM == kQuantFp8 ? k.nvec * 8 : (QM == kQuantMxfp4 ? k.nvec * 4 : 0);
    const int sb = QM == kQuantFp8 ? k.ngroups * 4 : (QM == kQuantMxfp4 ? k.nvec / 4 : 0);
    const rsrc_t r_q = row_rsrc(k.q, t * (int64_t)qb, qb);
    // FP8 scales row-major: this row's H/128 floats; column-major: the whole [H/128, T]
    // array (the host keeps it under 2^31 bytes), row t's scale of group g at (g*T + t)*4
    const bool cols = QM == kQuantFp8 && k.scale_cols;
    const rsrc_t r_sc = cols ? row_rsrc(k.scales, 0, (int)(k.T * k.ngroups * 4))
                             : row_rsrc(k.scales, t * (int64_t)sb, sb);
    const uint32_t sbase = cols ? (uint32_t)t * 4u : 0u;
    const uint32_t sstride = cols ? (uint32_t)k.T * 4u : 4u;
    if constexpr (kOutsFirst) {
        u32x4 ob[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            st16(yb[v], r_ro, off0 + v * L16);
            ob[v] = norm_store(yb[v], gam[v], rstd, r32, r32_ok, r_out, off0 + v * L16);
        }
        uint32_t offs[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) offs[v] = off0 + v * L16;
        quant_slots<kCodeP, VPL>(ob, r_q, r_sc, offs, sbase, sstride);
    } else if constexpr (QM == kQuantMxfp4) {
        u32x4 ob[VPL];
        uint32_t offs[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            if constexpr (kDefer) st16(yb[v], r_ro, off0 + v * L16);
            const u32x4 g = VPL == 4 ? gamma_slot(k, off0 + v * L16) : gam[v];
            ob[v] = norm_store(yb[v], g, rstd, r32, r32_ok, r_out, off0 + v * L16);
            offs[v] = off0 + v * L16;
        }
        mxfp4_slots<VPL>(ob, r_q, r_sc, offs);
    } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            if constexpr (kDefer) st16(yb[v], r_ro, off0 + v * L16);
            const u32x4 g = VPL == 4 ? gamma_slot(k, off0 + v * L16) : gam[v];
            const u32x4 ob = norm_store(yb[v], g, rstd, r32, r32_ok, r_out, off0 + v * L16);
            if constexpr (QM == kQuantFp8) quant_slot<kCodeP, VPL == 1>(ob, r_q, r_sc, off0 + v * L16, sbase, sstride);
        }
    }
}

template <int VPL>
__device__ __forceinline__ void load_gamma(u32x4 (&gam)[VPL], const Params &k) {
    const rsrc_t rg = row_rsrc(k.gamma, 0, k.nvec * 16);
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        gam[v] = __builtin_amdgcn_raw_buffer_load_b128(rg, (v * blockDim.x + threadIdx.x) * 16u, 0,
                                                       kGammaLoadPolicy);
}

// ---------------------------------------------------------------- kernels
template <int R, int VPL, int QM, bool kSmall>
__global__ __launch_bounds__(1024) void farn_rows(const Params k) {
    __shared__ double slot[kMaxWaves];
    const int64_t t = k.t0 + blockIdx.x;
    SlotIn<R> in;
    load_slot<R>(in, k, t, threadIdx.x * 16u);
    u32x4 gam[VPL];
    if constexpr (VPL != 4) load_gamma<VPL>(gam, k);  // four slots: gamma_slot, slot by slot
    do_row<R, VPL, QM, kSmall>(in, gam, k, t, slot);
}

// Unfused building blocks (the compositions the fused call replaces): the all-reduce
// alone, and the per-group quant alone of a bf16 tensor. Same row mapping, loads and
// arithmetic as the fused kernel's corresponding steps.
template <int R, int VPL>
__global__ __launch_bounds__(1024) void farn_reduce_rows(const Params k) {
    const int64_t t = k.t0 + blockIdx.x;
    const int rb = k.nvec * 16;
    const rsrc_t r_out = row_rsrc(k.res_out, t * (int64_t)rb, rb);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const uint32_t off = (v * blockDim.x + threadIdx.x) * 16u;
        SlotIn<R> in;
        load_slot<R>(in, k, t, off);
        st16(fold_slot<R, kFoldNoResidual>(in, false), r_out, off);
    }
}

template <int VPL>
__global__ __launch_bounds__(1024) void farn_quant_rows(const Params k) {
    const int64_t t = k.t0 + blockIdx.x;
    const int rb = k.nvec * 16;
    const rsrc_t r_x = row_rsrc(k.x, t * (int64_t)rb, rb);
    const rsrc_t r_q = row_rsrc(k.q, t * (int64_t)k.nvec * 8, k.nvec * 8);
    const rsrc_t r_sc = row_rsrc(k.scales, t * (int64_t)k.ngroups * 4, k.ngroups * 4);
    u32x4 xv[VPL];  // (the standalone quant is the FP8 group quant)
#pragma unroll
    for (int v = 0; v < VPL; ++v) xv[v] = ld16(r_x, (v * blockDim.x + threadIdx.x) * 16u);
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        quant_slot<kStoreCodePolicy>(xv[v], r_q, r_sc, (v * blockDim.x + threadIdx.x) * 16u, 0u, 4u);
}

// ---------------------------------------------------------------- dispatch tables
typedef void (*KernelFn)(const Params);

// Entries: one, two and four vector slots per lane, then the two-slot small-call schedule
// (the plain kernel has one schedule: its entry 3 is entry 1).
template <int R, int QM>
struct Row {
    static constexpr KernelFn fn[4] = {farn_rows<R, 1, QM, false>, farn_rows<R, 2, QM, false>,
                                       farn_rows<R, 4, QM, false>, farn_rows<R, 2, QM, QM != kQuantNone>};
};

template <int R>
struct RedRow {
    static constexpr KernelFn fn[3] = {farn_reduce_rows<R, 1>, farn_reduce_rows<R, 2>,
                                       farn_reduce_rows<R, 4>};
};
constexpr KernelFn kQuantRows[3] = {farn_quant_rows<1>, farn_quant_rows<2>, farn_quant_rows<4>};

KernelFn pick_reduce(int R, int vi) {
    switch (R) {
#define FARN_CASE(n) \
    case n: return RedRow<n>::fn[vi];
        FARN_CASE(1) FARN_CASE(2) FARN_CASE(3) FARN_CASE(4)
        FARN_CASE(5) FARN_CASE(6) FARN_CASE(7) FARN_CASE(8)
#undef FARN_CASE
        default: return nullptr;
    }
}

template <int QM>
KernelFn pick(int R, int vi) {
    switch (R) {
#define FARN_CASE(n) \
    case n: return Row<n, QM>::fn[vi];
        FARN_CASE(1) FARN_CASE(2) FARN_CASE(3) FARN_CASE(4)
        FARN_CASE(5) FARN_CASE(6) FARN_CASE(7) FARN_CASE(8)
#undef FARN_CASE
        default: return nullptr;
    }
}

}  // namespace

namespace farn {

static Params make_params(const Call &c) {
    Params k;
    for (int r = 0; r < 8; ++r) k.p[r] = c.partials[r];
    k.res = c.residual;
    k.gamma = c.gamma;
    k.res_out = c.residual_out;
    k.out = c.out;
    k.q = c.q;
    k.scales = c.scales;
    k.x = c.x;
    k.scale_cols = c.scale_cols ? 1 : 0;
    k.T = c.T;
    k.t0 = 0;
    k.nvec = (int)(c.H / 8);
    k.ngroups = (int)(c.H / 128);
    k.h = (double)c.H;
    k.inv_h = 1.0 / (double)c.H;
    k.eps = c.eps;
    return k;
}

int launch(const Call &c, int variant) {
    const RowShape rs = row_shape(c.H, c.kind == Kind::kFused ? variant : 1);
    int vi = rs.vpl == 1 ? 0 : (rs.vpl == 2 ? 1 : 2);
    if (c.kind == Kind::kFused && c.q != nullptr && rs.vpl == 2 && c.T <= kSmallCallRows) vi = 3;
    KernelFn fn = nullptr;
    if (c.kind == Kind::kReduce) {
        fn = pick_reduce(c.R, vi);
    } else if (c.kind == Kind::kQuant) {
        fn = kQuantRows[vi];
    } else {
        fn = c.q == nullptr ? pick<kQuantNone>(c.R, vi)
                            : (c.mxfp4 ? pick<kQuantMxfp4>(c.R, vi) : pick<kQuantFp8>(c.R, vi));
    }
    if (!fn) return 1;

    // A dispatch holds at most 2^32 - 1 work-items: very tall arrays go out as several
    // launches of consecutive rows (rows are independent).
    const int64_t max_rows = (int64_t)(UINT32_MAX / (uint32_t)rs.lanes);
    // hipLaunchKernel returns this launch's own status (hipGetLastError would also report,
    // and clear, an earlier error of the caller's).
    Params k = make_params(c);
    void *args[] = {&k};
    for (int64_t t0 = 0; t0 < c.T; t0 += max_rows) {
        k.t0 = t0;
        const int64_t n = c.T - t0 < max_rows ? c.T - t0 : max_rows;
        if (hipLaunchKernel((const void *)fn, dim3((uint32_t)n), dim3((uint32_t)rs.lanes), args,
                            c.lds_reserve, (hipStream_t)c.stream) != hipSuccess)
            return 1;
    }
    return 0;
}

}  // namespace farn
