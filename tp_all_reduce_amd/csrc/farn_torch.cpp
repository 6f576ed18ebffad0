// Tensor-level binding of the C ABI (include/farn.h) for Python: checks that every tensor
// is where and what the call needs (a GPU tensor of the right dtype, shape and layout, all
// on one device), then passes raw pointers to the extern "C" entry points of libfarn.so.
// Argument marshalling only; every step of the op runs in the library's kernels. The
// Python wrappers in __init__.py allocate missing outputs and turn a non-OK status into
// an exception. Written in C++ because the same checks in Python cost about 5 us per call.
#include <torch/extension.h>

#include <initializer_list>
#include <vector>

#include "../../include/farn.h"

namespace {

void check_tensor(const std::string &name, const at::Tensor &t, at::ScalarType dt, at::IntArrayRef shape,
                  const at::Device &dev) {
    TORCH_CHECK_VALUE(t.scalar_type() == dt && t.sizes() == shape && t.is_contiguous() && t.device() == dev,
                      name, ": expected contiguous ", dt, " ", shape, " on ", dev, ", got ", t.scalar_type(), " ",
                      t.sizes(), " on ", t.device());
}

// A code or scale buffer: contiguous, of one of `dts`, `numel` elements, on `dev`.
void check_buf(const char *name, const at::Tensor &t, std::initializer_list<at::ScalarType> dts, int64_t numel,
               const at::Device &dev) {
    bool dt_ok = false;
    for (auto d : dts) dt_ok = dt_ok || t.scalar_type() == d;
    TORCH_CHECK_VALUE(dt_ok && t.numel() == numel && t.is_contiguous() && t.device() == dev, name,
                      ": expected a contiguous tensor of ", numel, " elements of the call's dtype on ", dev,
                      ", got ", t.scalar_type(), " ", t.sizes(), " on ", t.device());
}

// The GPU of the call (that of its first input): the library takes plain pointers and cannot
// tell host memory from device memory, so host tensors are refused here.
at::Device gpu_of(const char *name, const at::Tensor &t) {
    TORCH_CHECK_VALUE(t.is_cuda(), name, ": expected a tensor on the GPU, got one on ", t.device());
    return t.device();
}

std::vector<const void *> checked_partials(const std::vector<at::Tensor> &partials, at::IntArrayRef shape,
                                           const at::Device &dev) {
    std::vector<const void *> ptrs(partials.size());
    for (size_t i = 0; i < partials.size(); ++i) {
        check_tensor("partials[" + std::to_string(i) + "]", partials[i], at::kBFloat16, shape, dev);
        ptrs[i] = partials[i].data_ptr();
    }
    return ptrs;
}

const void *opt_ptr(const c10::optional<at::Tensor> &t) { return t.has_value() ? t->data_ptr() : nullptr; }

// Modes of the fused call.
constexpr int64_t kPlain = 0, kFp8 = 1, kMxfp4 = 2;

// One fused call: plain (q and scales absent), FP8 (variant may carry FARN_SCALES_COL_MAJOR)
// or MXFP4. `stream` is the raw hipStream_t. Returns the farn_status.
int64_t fused(const std::vector<at::Tensor> &partials, const c10::optional<at::Tensor> &residual,
              const at::Tensor &gamma, double eps, const at::Tensor &residual_out,
              const c10::optional<at::Tensor> &out, const c10::optional<at::Tensor> &q,
              const c10::optional<at::Tensor> &scales, int64_t mode, int64_t group_size, int64_t variant,
              int64_t stream) {
    TORCH_CHECK_VALUE(!partials.empty(), "partials: expected at least one tensor");
    const at::Device dev = gpu_of("partials[0]", partials[0]);
    const at::IntArrayRef shape = partials[0].sizes();
    TORCH_CHECK_VALUE(shape.size() == 2, "partials[0]: expected a [T, H] tensor, got ", shape);
    const int64_t T = shape[0], H = shape[1];
    const std::vector<const void *> ptrs = checked_partials(partials, shape, dev);
    if (residual.has_value()) check_tensor("residual", *residual, at::kBFloat16, shape, dev);
    check_tensor("gamma", gamma, at::kBFloat16, {H}, dev);
    check_tensor("residual_out", residual_out, at::kBFloat16, shape, dev);
    if (out.has_value()) check_tensor("out", *out, at::kBFloat16, shape, dev);
    if (mode == kFp8) {
        TORCH_CHECK_VALUE(q.has_value() && scales.has_value(), "the FP8 call needs q and scales");
        const int64_t G = group_size > 0 ? H / group_size : 0;
        check_buf("q", *q, {at::kByte, at::kFloat8_e4m3fn}, T * H, dev);
        check_buf("scales", *scales, {at::kFloat}, T * G, dev);
    } else if (mode == kMxfp4) {
        TORCH_CHECK_VALUE(q.has_value() && scales.has_value(), "the MXFP4 call needs q and scales");
        check_buf("q", *q, {at::kByte}, T * (H / 2), dev);
        check_buf("scales", *scales, {at::kByte}, T * (H / FARN_MX_BLOCK), dev);
    } else {
        TORCH_CHECK_VALUE(mode == kPlain && out.has_value(), "the plain call needs out");
    }
    // HIP launches on the current device
    const c10::DeviceGuard guard(dev);
    void *s = reinterpret_cast<void *>(stream);
    const void *res = opt_ptr(residual);
    void *ro = residual_out.data_ptr();
    void *o = out.has_value() ? out->data_ptr() : nullptr;
    const int R = (int)partials.size();
    const float e = (float)eps;
    if (mode == kFp8)
        return farn_reduce_add_rmsnorm_quant_group_ex(ptrs.data(), R, res, gamma.data_ptr(), e, T, H,
                                                      (int)group_size, ro, o, q->data_ptr(),
                                                      static_cast<float *>(scales->data_ptr()), s, (int)variant);
    if (mode == kMxfp4)
        return farn_reduce_add_rmsnorm_mxfp4_ex(ptrs.data(), R, res, gamma.data_ptr(), e, T, H, ro, o,
                                                q->data_ptr(), scales->data_ptr(), s, (int)variant);
    return farn_reduce_add_rmsnorm_ex(ptrs.data(), R, res, gamma.data_ptr(), e, T, H, ro, o, s, (int)variant);
}

// The all-reduce alone: partials -> out.
int64_t reduce(const std::vector<at::Tensor> &partials, const at::Tensor &out, int64_t stream) {
    TORCH_CHECK_VALUE(!partials.empty(), "partials: expected at least one tensor");
    const at::Device dev = gpu_of("partials[0]", partials[0]);
    const at::IntArrayRef shape = partials[0].sizes();
    TORCH_CHECK_VALUE(shape.size() == 2, "partials[0]: expected a [T, H] tensor, got ", shape);
    const std::vector<const void *> ptrs = checked_partials(partials, shape, dev);
    check_tensor("out", out, at::kBFloat16, shape, dev);
    const c10::DeviceGuard guard(dev);
    return farn_reduce(ptrs.data(), (int)partials.size(), shape[0], shape[1], out.data_ptr(),
                       reinterpret_cast<void *>(stream));
}

// The per-group quant alone: x -> (q, scales).
int64_t quant(const at::Tensor &x, int64_t group_size, const at::Tensor &q, const at::Tensor &scales,
              int64_t stream) {
    const at::Device dev = gpu_of("x", x);
    const at::IntArrayRef shape = x.sizes();
    TORCH_CHECK_VALUE(shape.size() == 2, "x: expected a [T, H] tensor, got ", shape);
    const int64_t T = shape[0], H = shape[1];
    check_tensor("x", x, at::kBFloat16, shape, dev);
    const int64_t G = group_size > 0 ? H / group_size : 0;
    check_buf("q", q, {at::kByte, at::kFloat8_e4m3fn}, T * H, dev);
    check_buf("scales", scales, {at::kFloat}, T * G, dev);
    const c10::DeviceGuard guard(dev);
    return farn_quant_group(x.data_ptr(), T, H, (int)group_size, q.data_ptr(),
                            static_cast<float *>(scales.data_ptr()), reinterpret_cast<void *>(stream));
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m) {
    m.def("fused", &fused, "one fused call (plain, FP8 or MXFP4); returns the farn_status");
    m.def("reduce", &reduce, "the all-reduce alone; returns the farn_status");
    m.def("quant", &quant, "the per-group FP8 quant alone; returns the farn_status");
}
