"""Python binding of libfarn.so: fused reduce + residual-add + RMSNorm (+ per-group FP8
quant) for MI355X (gfx950).

Argument marshalling only: torch tensors supply device memory and the stream; every
step of the op runs in the HIP kernels behind the C ABI (include/farn.h). The tensor
calls go through a small compiled extension (_farn_torch, from csrc/farn_torch.cpp)
that checks every tensor and calls the C ABI's entry points; lib() gives the C ABI
itself through ctypes. Importing this package loads both in-tree libraries and raises
if either has not been built; there is no fallback.

The op is the per-GPU body of the fused tensor-parallel all-reduce + RMSNorm of
"ROCm AITER fused all-reduce + RMSNorm" (vLLM #37646 summary, fused_ar_rms) and of
the per-group FP8 variant in "AMD fused AllReduce-RMSNorm quant kernel" (sglang
#24651 summary, tensor_model_parallel_fused_allreduce_rmsnorm_quant_per_group).
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfarn.so")

OK = 0
STATUS = {0: "FARN_OK", 1: "FARN_ERR_NULL", 2: "FARN_ERR_SHAPE", 3: "FARN_ERR_ALIGN",
          4: "FARN_ERR_ALIAS", 5: "FARN_ERR_EPS", 6: "FARN_ERR_LAUNCH", 7: "FARN_ERR_VARIANT"}
VARIANT_AUTO, VARIANT_WIDE, VARIANT_NARROW = 0, 1, 2
VARIANT_LATENCY, VARIANT_BANDWIDTH = VARIANT_WIDE, VARIANT_NARROW  # older names of the two shapes
SCALES_COL_MAJOR = 0x100
MAX_R, MAX_H, GROUP, MX_BLOCK = 8, 32768, 128, 32
EXPORTS = ("farn_reduce_add_rmsnorm", "farn_reduce_add_rmsnorm_quant_group",
           "farn_reduce_add_rmsnorm_ex", "farn_reduce_add_rmsnorm_quant_group_ex",
           "farn_reduce", "farn_quant_group",
           "farn_reduce_add_rmsnorm_mxfp4", "farn_reduce_add_rmsnorm_mxfp4_ex",
           "farn_select_variant", "farn_status_string", "farn_abi_version")


class FarnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_lib.farn_status_string(status).decode()})")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python tp_all_reduce_amd/build.py` "
                          "(hipcc, gfx950). There is no fallback path.")
    L = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    pp = ctypes.POINTER(ctypes.c_void_p)
    base = [pp, i32, vp, vp, f32, i64, i64]
    L.farn_reduce_add_rmsnorm.argtypes = base + [vp, vp, vp]
    L.farn_reduce_add_rmsnorm_quant_group.argtypes = base + [i32, vp, vp, vp, vp, vp]
    L.farn_reduce_add_rmsnorm_ex.argtypes = base + [vp, vp, vp, i32]
    L.farn_reduce_add_rmsnorm_quant_group_ex.argtypes = base + [i32, vp, vp, vp, vp, vp, i32]
    L.farn_reduce.argtypes = [pp, i32, i64, i64, vp, vp]
    L.farn_quant_group.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    L.farn_reduce_add_rmsnorm_mxfp4.argtypes = base + [vp, vp, vp, vp, vp]
    L.farn_reduce_add_rmsnorm_mxfp4_ex.argtypes = base + [vp, vp, vp, vp, vp, i32]
    for fn in EXPORTS[:8]:
        getattr(L, fn).restype = i32
    L.farn_select_variant.argtypes = [i32, i64, i64, i32]
    L.farn_select_variant.restype = i32
    L.farn_status_string.argtypes = [i32]
    L.farn_status_string.restype = ctypes.c_char_p
    L.farn_abi_version.argtypes = []
    L.farn_abi_version.restype = i32
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def abi_version() -> int:
    return _lib.farn_abi_version()


def select_variant(R: int, T: int, H: int, quant=False) -> int:
    """The launch shape AUTO runs; quant: False for the plain call, True or "fp8" for the FP8
    call, "mxfp4" for the MXFP4 call."""
    kind = 2 if isinstance(quant, str) and quant == "mxfp4" else (1 if quant else 0)
    return _lib.farn_select_variant(R, T, H, kind)


_BF16 = torch.bfloat16
# The current stream's raw handle of a device, read without building a Stream object (the
# public torch.cuda.current_stream costs about 2 us per call, this about 0.1 us).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)

try:
    # tensor checks and pointer marshalling into the C ABI, compiled (csrc/farn_torch.cpp)
    from . import _farn_torch as _ext
except ImportError as e:
    raise ImportError(f"{os.path.dirname(LIB_PATH)}/_farn_torch.so is not built or does not load ({e}); "
                      "run `python tp_all_reduce_amd/build.py`. There is no fallback path.") from e

_PLAIN, _FP8, _MXFP4 = 0, 1, 2


def _device_of(t, name="partials[0]"):
    """The GPU the call runs on: that of its first input. The library takes plain pointers and
    cannot tell host memory from device memory, so host tensors are refused."""
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a tensor on the GPU, got one on {t.device}")
    return t.device


def _stream(device, stream):
    """Raw hipStream_t (an int) of `stream`, or of the current stream of `device`."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _on_stream(stream, made):
    """Outputs a wrapper allocates come from the caching allocator's pool of the current stream.
    When the kernels are launched on another `stream`, mark them as used there, so that their
    memory is not handed out again before that stream's work is done."""
    if stream is not None:
        for t in made:
            if t is not None:
                t.record_stream(stream)


def reduce_add_rmsnorm(partials, residual, gamma, eps: float = 1e-6, *, residual_out=None,
                       out=None, variant: int = VARIANT_AUTO, stream=None):
    """Sum the R partials (list of bf16 [T,H] device tensors) in rank order in fp32, add the
    residual (or None), round to bf16 -> residual_out, then RMSNorm with gamma -> out.
    residual_out may be the residual tensor itself (in place). Returns (residual_out, out)."""
    p0 = partials[0]
    dev = _device_of(p0)
    made = []
    if residual_out is None:
        residual_out = torch.empty_like(p0)
        made.append(residual_out)
    if out is None:
        out = torch.empty_like(p0)
        made.append(out)
    _on_stream(stream, made)
    st = _ext.fused(partials, residual, gamma, eps, residual_out, out, None, None, _PLAIN, 0, variant,
                    _stream(dev, stream))
    if st != OK:
        raise FarnError(st, "farn_reduce_add_rmsnorm")
    return residual_out, out


def reduce_add_rmsnorm_quant_group(partials, residual, gamma, eps: float = 1e-6, *,
                                   group_size: int = GROUP, emit_out: bool = True, residual_out=None,
                                   out=None, q=None, scales=None, variant: int = VARIANT_AUTO,
                                   scales_col_major: bool = False, stream=None):
    """The plain call, then per-128-channel E4M3 quant of the bf16 output. Returns
    (residual_out, out or None, q uint8 [T,H] E4M3 codes, scales float32 [T, H/128], or
    [H/128, T] with scales_col_major)."""
    p0 = partials[0]
    dev = _device_of(p0)
    T, H = p0.shape
    made = []
    if residual_out is None:
        residual_out = torch.empty_like(p0)
        made.append(residual_out)
    if emit_out and out is None:
        out = torch.empty_like(p0)
        made.append(out)
    if not emit_out:
        out = None
    if q is None:
        q = torch.empty((T, H), dtype=torch.uint8, device=dev)
        made.append(q)
    if scales is None:
        G = H // group_size if group_size > 0 else 0
        scales = torch.empty((G, T) if scales_col_major else (T, G), dtype=torch.float32, device=dev)
        made.append(scales)
    _on_stream(stream, made)
    st = _ext.fused(partials, residual, gamma, eps, residual_out, out, q, scales, _FP8, group_size,
                    variant | (SCALES_COL_MAJOR if scales_col_major else 0), _stream(dev, stream))
    if st != OK:
        raise FarnError(st, "farn_reduce_add_rmsnorm_quant_group")
    return residual_out, out, q, scales


def reduce(partials, *, out=None, stream=None):
    """All-reduce alone (first kernel of the unfused compositions): bf16 of the fp32 rank-order
    sum of the partials. Returns out."""
    p0 = partials[0]
    dev = _device_of(p0)
    if out is None:
        out = torch.empty_like(p0)
        _on_stream(stream, [out])
    st = _ext.reduce(partials, out, _stream(dev, stream))
    if st != OK:
        raise FarnError(st, "farn_reduce")
    return out


def quant_group(x, *, group_size: int = GROUP, q=None, scales=None, stream=None):
    """Per-group E4M3 quant alone of a bf16 [T,H] tensor. Returns (q uint8 [T,H], scales fp32 [T,H/128])."""
    dev = _device_of(x, "x")
    T, H = x.shape
    made = []
    if q is None:
        q = torch.empty((T, H), dtype=torch.uint8, device=dev)
        made.append(q)
    if scales is None:
        scales = torch.empty((T, H // group_size if group_size > 0 else 0), dtype=torch.float32, device=dev)
        made.append(scales)
    _on_stream(stream, made)
    st = _ext.quant(x, group_size, q, scales, _stream(dev, stream))
    if st != OK:
        raise FarnError(st, "farn_quant_group")
    return q, scales


def reduce_add_rmsnorm_mxfp4(partials, residual, gamma, eps: float = 1e-6, *, emit_out: bool = True,
                             residual_out=None, out=None, q=None, scales=None,
                             variant: int = VARIANT_AUTO, stream=None):
    """The plain call, then MXFP4 of the bf16 output (OCP MX: 32-channel blocks, E8M0 scales,
    E2M1 codes two per byte). Returns (residual_out, out or None, q uint8 [T, H/2],
    scales uint8 [T, H/32])."""
    p0 = partials[0]
    dev = _device_of(p0)
    T, H = p0.shape
    made = []
    if residual_out is None:
        residual_out = torch.empty_like(p0)
        made.append(residual_out)
    if emit_out and out is None:
        out = torch.empty_like(p0)
        made.append(out)
    if not emit_out:
        out = None
    if q is None:
        q = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
        made.append(q)
    if scales is None:
        scales = torch.empty((T, H // MX_BLOCK), dtype=torch.uint8, device=dev)
        made.append(scales)
    _on_stream(stream, made)
    st = _ext.fused(partials, residual, gamma, eps, residual_out, out, q, scales, _MXFP4, 0, variant,
                    _stream(dev, stream))
    if st != OK:
        raise FarnError(st, "farn_reduce_add_rmsnorm_mxfp4")
    return residual_out, out, q, scales
