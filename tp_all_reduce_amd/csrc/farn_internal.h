// Internal interface between the C-ABI layer (argument checks, variant choice)
// and the HIP kernels. Not installed; callers use include/farn.h.
#pragma once

#include <stdint.h>

namespace farn {

enum class Kind { kFused, kReduce, kQuant };

// One validated call, raw device pointers. q / scales are null for the plain call.
// kReduce writes the all-reduce alone into residual_out; kQuant reads x.
struct Call {
    Kind kind = Kind::kFused;
    const void *partials[8];
    int R;
    const void *residual;  // null: no residual
    const void *gamma;
    float eps;
    int64_t T, H;
    void *residual_out;
    void *out;     // null only for the quant call with the bf16 output off
    void *q;       // quant calls only
    void *scales;  // quant calls only (fp32 for FP8, E8M0 bytes for MXFP4)
    bool mxfp4 = false;       // q / scales hold MXFP4 (else FP8 group-128)
    bool scale_cols = false;  // FP8 scales column-major [H/128, T]
    const void *x = nullptr;  // kQuant input
    void *stream;
    // Bytes of LDS reserved per workgroup beyond what the kernel declares (unused by it):
    // bounds how many workgroups share a compute unit (0 = no bound).
    unsigned lds_reserve = 0;
};

// Lanes per token row (= workgroup size) and 16-byte vectors per lane for hidden size
// H and variant (1 = wide: widest mapping; 2 = narrow: about half the lanes,
// two vectors per lane).
struct RowShape {
    int lanes;  // multiple of 64, <= 1024
    int vpl;    // vectors per lane: 1, 2 or 4
};
RowShape row_shape(int64_t H, int variant);

// Rows up to which the two-slot quant kernels run their small-call store schedule (measured
// on MI355X: faster up to T = 256, slower from T = 1024); above it, the streaming schedule.
constexpr int64_t kSmallCallRows = 512;

// Enqueue one workgroup per row. variant: 1 = wide, 2 = narrow (already resolved
// from AUTO; the unfused blocks use 1). Returns 0 on success, nonzero when the launch failed.
int launch(const Call &c, int variant);

}  // namespace farn
