// C-ABI entry points: argument checks on the host, variant choice, then one launch.
// This file makes no HIP call; every check runs before anything is enqueued, so a
// rejected call leaves the stream untouched (the analogue of the pages' fused path
// returning None so the caller falls back: "AMD fused AllReduce-RMSNorm quant
// kernel", sglang #24651 summary, layernorm.py snippet).
#include <math.h>
#include <stdint.h>

#include "../../include/farn.h"
#include "farn_internal.h"

namespace farn {

RowShape row_shape(int64_t H, int variant) {
    const int64_t nvec = H / 8;
    RowShape s;
    if (variant == FARN_VARIANT_NARROW && nvec > 128 && nvec <= 1024) {
        s.lanes = (int)((((nvec + 1) / 2) + 63) / 64 * 64);  // about NV/2 lanes, two vectors each
        s.vpl = 2;
    } else if (nvec <= 1024) {
        s.lanes = (int)(((nvec + 63) / 64) * 64);
        s.vpl = 1;
    } else if (nvec <= 2048) {
        // two or four vectors per lane on as few lanes as cover the row: measured on MI355X
        // against 1024 lanes at every such H (identical outputs), 5-25 % faster where 1024
        // lanes would leave vector slots empty (H = 8320 .. 13312, 16512 .. 28672; decode and
        // streaming), the same where the row nearly fills them (H = 14336 .. 16384, 32768)
        s.lanes = (int)((((nvec + 1) / 2) + 63) / 64 * 64);
        s.vpl = 2;
    } else {
        s.lanes = (int)((((nvec + 3) / 4) + 63) / 64 * 64);
        s.vpl = 4;
    }
    return s;
}

}  // namespace farn

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void *p, int64_t bytes) {
    uintptr_t lo = (uintptr_t)p;
    return Range{lo, lo + (uintptr_t)bytes};
}

// Output quant mode of a fused call.
enum Quant { kNone = 0, kFp8 = 1, kMxfp4 = 2 };

// Full check of one fused call.
farn_status check(const void *const *partials, int R, const void *residual, const void *gamma,
                  float eps, int64_t T, int64_t H, int group_size, Quant quant, void *residual_out,
                  void *out, void *q, void *scales) {
    if (R < 1 || R > FARN_MAX_R) return FARN_ERR_SHAPE;
    if (T < 0 || T > ((int64_t)1 << 40) || H <= 0 || H % 8 != 0 || H > FARN_MAX_H)
        return FARN_ERR_SHAPE;
    if (quant == kFp8 && (group_size != FARN_GROUP || H % FARN_GROUP != 0)) return FARN_ERR_SHAPE;
    if (quant == kMxfp4 && H % FARN_MX_BLOCK != 0) return FARN_ERR_SHAPE;
    if (!(eps >= 0.0f) || isinf(eps)) return FARN_ERR_EPS;
    if (!partials || !gamma) return FARN_ERR_NULL;
    if (T == 0) return FARN_OK;  // no row buffer is touched; empty tensors may have NULL data
    for (int r = 0; r < R; ++r)
        if (!partials[r]) return FARN_ERR_NULL;
    if (!residual_out) return FARN_ERR_NULL;
    if (quant != kNone) {
        if (!q || !scales) return FARN_ERR_NULL;
    } else if (!out) {
        return FARN_ERR_NULL;
    }

    auto a16 = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
    for (int r = 0; r < R; ++r)
        if (!a16(partials[r])) return FARN_ERR_ALIGN;
    if ((residual && !a16(residual)) || !a16(gamma) || !a16(residual_out) || (out && !a16(out)))
        return FARN_ERR_ALIGN;
    if (quant != kNone && !a16(q)) return FARN_ERR_ALIGN;
    if (quant == kFp8 && ((uintptr_t)scales & 3u) != 0) return FARN_ERR_ALIGN;

    const int64_t tile = T * H * 2;
    Range ins[FARN_MAX_R + 2];
    int n_in = 0;
    for (int r = 0; r < R; ++r) ins[n_in++] = range_of(partials[r], tile);
    ins[n_in++] = range_of(gamma, H * 2);
    Range res_in = residual ? range_of(residual, tile) : Range{0, 0};

    Range outs[4];
    int n_out = 0;
    outs[n_out++] = range_of(residual_out, tile);
    if (out) outs[n_out++] = range_of(out, tile);
    if (quant == kFp8) {
        outs[n_out++] = range_of(q, T * H);
        outs[n_out++] = range_of(scales, T * (H / FARN_GROUP) * 4);
    } else if (quant == kMxfp4) {
        outs[n_out++] = range_of(q, T * H / 2);
        outs[n_out++] = range_of(scales, T * (H / FARN_MX_BLOCK));
    }
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (overlaps(outs[i], ins[j])) return FARN_ERR_ALIAS;
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i], outs[j])) return FARN_ERR_ALIAS;
        if (residual && overlaps(outs[i], res_in)) {
            const bool in_place = (i == 0 && residual_out == residual);
            if (!in_place) return FARN_ERR_ALIAS;
        }
    }
    return FARN_OK;
}

// AUTO rule, from interleaved measurements of both launch shapes on MI355X (graph replay,
// median of 5; cache-hot for calls up to 128 MiB, streaming from HBM above). By vectors per
// row, nvec = H/8 (the wide shape runs one vector per lane, the narrow shape half as many
// lanes with two vectors each). Set on about 820 points (R = 2..8, H = 1024..8192,
// T = 16..8192, plain and FP8: grids over H x T x R and the points of earlier rules, five
// boxes), its edges adjusted on 320 random points (R = 2..8, H a multiple of 128, T
// log-uniform over 16..8192; plain, FP8 and MXFP4). Time of the narrow shape against the wide
// one:
//   1. nvec in (768, 1024] (H = 6152 .. 8192): narrow, median -3.2 % (decode -5 .. -9 %,
//      T = 1024 -9 %, T = 8192 -3.3 .. -4.5 %; ties at H = 8192, T = 2048); except the plain
//      call with nvec > 896 (H > 7168) from T = 4096, where the wide shape is 0.5-2 % faster
//      at R = 8.
//   2. nvec in (576, 640] (H = 4616 .. 5120) at 768 <= T < 2048: narrow, -3 .. -14 % at
//      T = 768 .. 1024 (two of 16 points +1.3 and +2.1 %), -2.8 .. +1.5 % at T = 1400 .. 2000.
//   3. The FP8 call with nvec in (256, 768] (H = 2056 .. 6144) below T = 768, when
//      nvec <= 464 (H <= 3712) from T = 80, or 256 <= T < 512: narrow, median -5.7 %, down to
//      -21 %, in five of six points faster; the two-slot kernel overlaps each slot's group
//      reductions and scale with the other slot's loads. From T = 768 the wide shape is up to
//      10 % faster at H = 2560. Below T = 80 the one-slot kernel, which skips the rescale
//      multiplies, is the faster one at H <= 3712 (on a grid of 180 points, R = 2..8,
//      H = 2176 .. 3712, T = 8 .. 256, cache-hot: narrow +0.7 .. +4.8 % by median up to T = 48,
//      even at T = 64, -1.6 % from T = 96; the bound takes the rule's loss there from 1.50 % to
//      0.22 %, on 80 further random points streaming from HBM from 4.17 % to 1.63 %). The MXFP4
//      call is not in this band: its narrow shape is 3-7 % slower below T = 100 there.
//   4. R <= 4, nvec in (256, 768] at 512 <= T < 768 (two ranks: T < 1536): narrow, median
//      -3.2 %, down to -20 % (FP8, T = 512), up to +10 % at H = 2560. With few ranks the wide
//      shape keeps only R + 1 loads in flight per lane; the narrow one doubles that. At T = 768
//      with four ranks the wide shape is 2-10 % faster; at T = 384 the two are even on average.
//   Everything else: wide (the narrow shape median 3.9 % slower, up to 36 % at small T and
//   H <= 2048).
// Against the faster shape at each point the rule loses 0.48 % on average over the 820 points,
// 0.50 .. 0.58 % over the 320 random ones, and 0.28 .. 0.49 % (at most 10.6 .. 16.5 %, mostly at
// R = 3, H = 4608, T = 434, plain) over 160 further random points measured after it was fixed,
// in four timings on three boxes. The previous rule, without
// band 3 and with a band for H = 1544 .. 2048 from T = 4096 (-1 .. -5 %), lost 1.19 %,
// 0.95 .. 1.18 % and 1.05 % (at most 19 % on the last set).
int select(int R, int64_t T, int64_t H, int quant) {
    const int64_t nvec = H / 8;
    if (nvec > 768 && nvec <= 1024)
        return (quant == kNone && nvec > 896 && T >= 4096) ? FARN_VARIANT_WIDE : FARN_VARIANT_NARROW;
    if (nvec > 576 && nvec <= 640 && T >= 768 && T < 2048) return FARN_VARIANT_NARROW;
    if (quant == kFp8 && nvec > 256 && nvec <= 768 && T < 768 && ((nvec <= 464 && T >= 80) || (T >= 256 && T < 512)))
        return FARN_VARIANT_NARROW;
    if (R <= 4 && nvec > 256 && nvec <= 768 && T >= 512 && T < (R <= 2 ? 1536 : 768)) return FARN_VARIANT_NARROW;
    return FARN_VARIANT_WIDE;
}

// Workgroups per compute unit of the narrow shape at nvec in (768, 1024] (7 or 8 waves per
// row) in calls of many rows: at most two. Registers allow three for the streaming FP8 and
// MXFP4 kernels (78-79 VGPRs) and for the plain kernel with up to seven ranks (80; with eight,
// 91 VGPRs hold it at two), and two stream faster: reserving 56 KiB of LDS per workgroup (of
// 160 KiB per compute unit), which the kernel does not use, leaves room for two.
// Measured on MI355X (interleaved, median of 5, H = 7168 unless stated), against no
// reservation: FP8 and MXFP4, R = 8: T = 1024 -1.4 %, T = 2048 -4.0 %, T = 8192 -2.7 .. -3.1 %;
// R = 6: -1.4 .. -3.8 %; R = 5 and 4 from T = 2048: -1.0 .. -3.5 %, but +0.6 .. +5.9 % at
// T = 1024. Plain, R = 4..7 from T = 2048: -0.9 .. -3.3 % at H = 6656 and 7168 (-2.9 ..
// +1.8 % at H = 8192, where the wide shape runs the plain call from T = 4096); at T = 1024
// 0 .. +4.7 %, and with two ranks +0.2 .. +3.5 % from T = 2048. The small-call schedule (T <= 512)
// holds 82-83 VGPRs, so two is already its limit.
constexpr unsigned kLdsTwoPerCu = 56u * 1024u;

unsigned lds_reserve(int R, int64_t T, int64_t H, Quant quant, int shape) {
    const int64_t nvec = H / 8;
    if (shape != FARN_VARIANT_NARROW || nvec <= 768 || nvec > 1024) return 0u;
    if (quant != kNone)
        return (T > farn::kSmallCallRows && (R >= 6 || (R >= 4 && T >= 2048))) ? kLdsTwoPerCu : 0u;
    return (R >= 4 && R <= 7 && T >= 2048) ? kLdsTwoPerCu : 0u;
}

farn_status run(const void *const *partials, int R, const void *residual, const void *gamma,
                float eps, int64_t T, int64_t H, int group_size, Quant quant, void *residual_out,
                void *out, void *q, void *scales, void *stream, int options) {
    const int variant = options & 0xff;
    const bool cols = (options & FARN_SCALES_COL_MAJOR) != 0;
    if ((options & ~(0xff | FARN_SCALES_COL_MAJOR)) != 0) return FARN_ERR_VARIANT;
    if (variant < FARN_VARIANT_AUTO || variant > FARN_VARIANT_NARROW) return FARN_ERR_VARIANT;
    if (cols && quant != kFp8) return FARN_ERR_VARIANT;
    farn_status st = check(partials, R, residual, gamma, eps, T, H, group_size, quant,
                           residual_out, out, q, scales);
    if (st != FARN_OK || T == 0) return st;
    // column-major scales are addressed through one 32-bit buffer range (T and H are in
    // range here, so the product cannot overflow)
    if (cols && T * (H / FARN_GROUP) * 4 >= ((int64_t)1 << 31)) return FARN_ERR_SHAPE;
    const int shape = variant == FARN_VARIANT_AUTO ? select(R, T, H, quant) : variant;
    farn::Call c;
    for (int r = 0; r < 8; ++r) c.partials[r] = r < R ? partials[r] : nullptr;
    c.R = R;
    c.residual = residual;
    c.gamma = gamma;
    c.eps = eps;
    c.T = T;
    c.H = H;
    c.residual_out = residual_out;
    c.out = out;
    c.q = quant != kNone ? q : nullptr;
    c.scales = quant != kNone ? scales : nullptr;
    c.mxfp4 = quant == kMxfp4;
    c.scale_cols = cols;
    c.stream = stream;
    c.lds_reserve = lds_reserve(R, T, H, quant, shape);
    return farn::launch(c, shape) == 0 ? FARN_OK : FARN_ERR_LAUNCH;
}

// Checks of the standalone all-reduce: partials -> out.
farn_status check_reduce(const void *const *partials, int R, int64_t T, int64_t H, void *out) {
    if (R < 1 || R > FARN_MAX_R) return FARN_ERR_SHAPE;
    if (T < 0 || T > ((int64_t)1 << 40) || H <= 0 || H % 8 != 0 || H > FARN_MAX_H) return FARN_ERR_SHAPE;
    if (!partials) return FARN_ERR_NULL;
    if (T == 0) return FARN_OK;
    for (int r = 0; r < R; ++r)
        if (!partials[r]) return FARN_ERR_NULL;
    if (!out) return FARN_ERR_NULL;
    auto a16 = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
    for (int r = 0; r < R; ++r)
        if (!a16(partials[r])) return FARN_ERR_ALIGN;
    if (!a16(out)) return FARN_ERR_ALIGN;
    const Range o = range_of(out, T * H * 2);
    for (int r = 0; r < R; ++r)
        if (overlaps(o, range_of(partials[r], T * H * 2))) return FARN_ERR_ALIAS;
    return FARN_OK;
}

// Checks of the standalone quant: x -> (q, scales).
farn_status check_quant(const void *x, int64_t T, int64_t H, int group_size, void *q, float *scales) {
    if (T < 0 || T > ((int64_t)1 << 40) || H <= 0 || H > FARN_MAX_H || group_size != FARN_GROUP ||
        H % FARN_GROUP != 0)
        return FARN_ERR_SHAPE;
    if (T == 0) return FARN_OK;
    if (!x || !q || !scales) return FARN_ERR_NULL;
    if (((uintptr_t)x & 15u) || ((uintptr_t)q & 15u) || ((uintptr_t)scales & 3u)) return FARN_ERR_ALIGN;
    const Range rx = range_of(x, T * H * 2), rq = range_of(q, T * H),
                rs = range_of(scales, T * (H / FARN_GROUP) * 4);
    if (overlaps(rq, rx) || overlaps(rs, rx) || overlaps(rq, rs)) return FARN_ERR_ALIAS;
    return FARN_OK;
}

farn::Call blank_call(void *stream) {
    farn::Call c;
    for (int r = 0; r < 8; ++r) c.partials[r] = nullptr;
    c.R = 0;
    c.residual = nullptr;
    c.gamma = nullptr;
    c.eps = 0.0f;
    c.T = 0;
    c.H = 0;
    c.residual_out = nullptr;
    c.out = nullptr;
    c.q = nullptr;
    c.scales = nullptr;
    c.x = nullptr;
    c.stream = stream;
    c.lds_reserve = 0;
    return c;
}

}  // namespace

extern "C" {

farn_status farn_reduce(const void *const *partials, int R, int64_t T, int64_t H, void *out,
                        void *stream) {
    farn_status st = check_reduce(partials, R, T, H, out);
    if (st != FARN_OK || T == 0) return st;
    farn::Call c = blank_call(stream);
    c.kind = farn::Kind::kReduce;
    for (int r = 0; r < R; ++r) c.partials[r] = partials[r];
    c.R = R;
    c.T = T;
    c.H = H;
    c.residual_out = out;
    return farn::launch(c, FARN_VARIANT_WIDE) == 0 ? FARN_OK : FARN_ERR_LAUNCH;
}

farn_status farn_quant_group(const void *x, int64_t T, int64_t H, int group_size, void *q,
                             float *scales, void *stream) {
    farn_status st = check_quant(x, T, H, group_size, q, scales);
    if (st != FARN_OK || T == 0) return st;
    farn::Call c = blank_call(stream);
    c.kind = farn::Kind::kQuant;
    c.T = T;
    c.H = H;
    c.x = x;
    c.q = q;
    c.scales = scales;
    return farn::launch(c, FARN_VARIANT_WIDE) == 0 ? FARN_OK : FARN_ERR_LAUNCH;
}

farn_status farn_reduce_add_rmsnorm(const void *const *partials, int R, const void *residual,
                                    const void *gamma, float eps, int64_t T, int64_t H,
                                    void *residual_out, void *out, void *stream) {
    return run(partials, R, residual, gamma, eps, T, H, 0, kNone, residual_out, out, nullptr,
               nullptr, stream, FARN_VARIANT_AUTO);
}

farn_status farn_reduce_add_rmsnorm_quant_group(const void *const *partials, int R,
                                                const void *residual, const void *gamma, float eps,
                                                int64_t T, int64_t H, int group_size,
                                                void *residual_out, void *out, void *q,
                                                float *scales, void *stream) {
    return run(partials, R, residual, gamma, eps, T, H, group_size, kFp8, residual_out, out, q,
               scales, stream, FARN_VARIANT_AUTO);
}

farn_status farn_reduce_add_rmsnorm_ex(const void *const *partials, int R, const void *residual,
                                       const void *gamma, float eps, int64_t T, int64_t H,
                                       void *residual_out, void *out, void *stream, int variant) {
    return run(partials, R, residual, gamma, eps, T, H, 0, kNone, residual_out, out, nullptr,
               nullptr, stream, variant);
}

farn_status farn_reduce_add_rmsnorm_quant_group_ex(const void *const *partials, int R,
                                                   const void *residual, const void *gamma,
                                                   float eps, int64_t T, int64_t H, int group_size,
                                                   void *residual_out, void *out, void *q,
                                                   float *scales, void *stream, int variant) {
    return run(partials, R, residual, gamma, eps, T, H, group_size, kFp8, residual_out, out, q,
               scales, stream, variant);
}

farn_status farn_reduce_add_rmsnorm_mxfp4(const void *const *partials, int R, const void *residual,
                                          const void *gamma, float eps, int64_t T, int64_t H,
                                          void *residual_out, void *out, void *q, void *scales,
                                          void *stream) {
    return run(partials, R, residual, gamma, eps, T, H, 0, kMxfp4, residual_out, out, q, scales,
               stream, FARN_VARIANT_AUTO);
}

farn_status farn_reduce_add_rmsnorm_mxfp4_ex(const void *const *partials, int R, const void *residual,
                                             const void *gamma, float eps, int64_t T, int64_t H,
                                             void *residual_out, void *out, void *q, void *scales,
                                             void *stream, int variant) {
    return run(partials, R, residual, gamma, eps, T, H, 0, kMxfp4, residual_out, out, q, scales,
               stream, variant);
}

int farn_select_variant(int R, int64_t T, int64_t H, int quant) { return select(R, T, H, quant); }

const char *farn_status_string(int status) {
    switch (status) {
        case FARN_OK: return "ok";
        case FARN_ERR_NULL: return "a required pointer is NULL";
        case FARN_ERR_SHAPE: return "unsupported shape (R, T, H or group size)";
        case FARN_ERR_ALIGN: return "a buffer is not aligned (16 bytes; scales 4 bytes)";
        case FARN_ERR_ALIAS: return "an output overlaps an input or another output";
        case FARN_ERR_EPS: return "eps is not finite or is negative";
        case FARN_ERR_LAUNCH: return "kernel launch failed";
        case FARN_ERR_VARIANT: return "unknown variant or option";
        default: return "unknown status";
    }
}

int farn_abi_version(void) { return FARN_ABI_VERSION; }

}  // extern "C"
