"""CPU oracle (plain C, loaded through ctypes) for the fused reduce + residual-add +
RMSNorm (+ per-group FP8 quant) op.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the bench's CPU
baseline leg may import this package; the product path (`tp_all_reduce_amd`)
never does, and the two share no code. The arithmetic lives in
`farn_oracle.c`; this file only marshals numpy arrays into it.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "farn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(force: bool = False) -> str:
    """Compile farn_oracle.c with gcc into oracle/liboracle.so (IEEE single adds, no fast math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
# Thread count the fused-call wrappers use when none is given, and whether they fill their
# outputs with a pattern before the call (so that an element the C code never writes shows
# up as a wrong value rather than as whatever the allocator left there). `threads()` sets
# both for a block of code.
_default_threads = 1
_poison = False
_POISON_BYTE = 0xA5


@contextlib.contextmanager
def threads(n: int, poison: bool = True):
    """Run the fused-call wrappers with `n` threads (rows dealt round-robin to the threads)
    unless a call names its own count, with poisoned outputs. The pins use it to run the
    checks on the threaded row split."""
    global _default_threads, _poison
    saved = (_default_threads, _poison)
    _default_threads, _poison = int(n), bool(poison)
    try:
        yield
    finally:
        _default_threads, _poison = saved


def _nthreads(n):
    return _default_threads if n is None else int(n)


def _out(shape, dtype):
    a = np.empty(shape, dtype)
    if _poison:
        a.view(np.uint8).fill(_POISON_BYTE)
    return a


def _bind(L: ctypes.CDLL) -> ctypes.CDLL:
    u16p = ctypes.POINTER(ctypes.c_uint16)
    L.oracle_reduce_add_rmsnorm.argtypes = [
        ctypes.POINTER(u16p), ctypes.c_int, u16p, u16p, ctypes.c_float, ctypes.c_int64,
        ctypes.c_int64, u16p, u16p, ctypes.c_int]
    L.oracle_reduce_add_rmsnorm.restype = ctypes.c_int
    L.oracle_reduce_add_rmsnorm_quant_group.argtypes = [
        ctypes.POINTER(u16p), ctypes.c_int, u16p, u16p, ctypes.c_float, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int, u16p, u16p, ctypes.POINTER(ctypes.c_uint8),
        ctypes.POINTER(ctypes.c_float), ctypes.c_int]
    L.oracle_reduce_add_rmsnorm_quant_group.restype = ctypes.c_int
    L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    L.oracle_bf16_from_double.restype = ctypes.c_uint16
    L.oracle_e4m3fn_from_double.argtypes = [ctypes.c_double]
    L.oracle_e4m3fn_from_double.restype = ctypes.c_uint8
    dp = ctypes.POINTER(ctypes.c_double)
    L.oracle_bf16_from_double_array.argtypes = [dp, u16p, ctypes.c_int64]
    L.oracle_bf16_from_double_array.restype = None
    L.oracle_e4m3fn_from_double_array.argtypes = [dp, ctypes.POINTER(ctypes.c_uint8), ctypes.c_int64]
    L.oracle_e4m3fn_from_double_array.restype = None
    L.oracle_reduce.argtypes = [ctypes.POINTER(u16p), ctypes.c_int, ctypes.c_int64, ctypes.c_int64, u16p]
    L.oracle_reduce.restype = ctypes.c_int
    L.oracle_quant_group.argtypes = [u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_float)]
    L.oracle_quant_group.restype = ctypes.c_int
    u8p = ctypes.POINTER(ctypes.c_uint8)
    L.oracle_e2m1_from_double.argtypes = [ctypes.c_double]
    L.oracle_e2m1_from_double.restype = ctypes.c_uint8
    L.oracle_e2m1_from_double_array.argtypes = [dp, ctypes.POINTER(ctypes.c_uint8), ctypes.c_int64]
    L.oracle_e2m1_from_double_array.restype = None
    L.oracle_mxfp4.argtypes = [u16p, ctypes.c_int64, ctypes.c_int64, u8p, u8p]
    L.oracle_mxfp4.restype = ctypes.c_int
    L.oracle_reduce_add_rmsnorm_mxfp4.argtypes = [
        ctypes.POINTER(u16p), ctypes.c_int, u16p, u16p, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
        u16p, u16p, u8p, u8p, ctypes.c_int]
    L.oracle_reduce_add_rmsnorm_mxfp4.restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def using(so_path: str):
    """Run the wrappers against another build of the oracle (the pin tests use it to
    check that planted mistakes are caught)."""
    global _lib
    saved = lib()
    _lib = _bind(ctypes.CDLL(so_path))
    try:
        yield
    finally:
        _lib = saved


def _u16(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _partials_list(partials):
    if isinstance(partials, np.ndarray) and partials.ndim == 3:
        return [np.ascontiguousarray(partials[r]) for r in range(partials.shape[0])]
    return [np.ascontiguousarray(p) for p in partials]


def _ptr_array(plist):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    arr = (u16p * len(plist))()
    for i, p in enumerate(plist):
        assert p.dtype == np.uint16
        arr[i] = _u16(p)
    return arr


def reduce_add_rmsnorm(partials, residual, gamma, eps: float = 1e-6, nthreads: int | None = None,
                       in_place: bool = False):
    """Plain call. partials: [R,T,H] (or list of [T,H]) uint16 bf16 bits; residual [T,H]
    uint16 or None; gamma [H] uint16. Returns (residual_out, out) as uint16 arrays.
    With in_place, residual_out is written over a copy of residual passed as both."""
    plist = _partials_list(partials)
    T, H = plist[0].shape
    g = np.ascontiguousarray(gamma, dtype=np.uint16)
    out = _out((T, H), np.uint16)
    if in_place:
        res = np.array(residual, dtype=np.uint16, copy=True)
        res_out = res
    else:
        res = None if residual is None else np.ascontiguousarray(residual, dtype=np.uint16)
        res_out = _out((T, H), np.uint16)
    rc = lib().oracle_reduce_add_rmsnorm(
        _ptr_array(plist), len(plist), None if res is None else _u16(res), _u16(g), eps, T, H,
        _u16(res_out), _u16(out), _nthreads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_reduce_add_rmsnorm failed ({rc})")
    return res_out, out


def reduce_add_rmsnorm_quant_group(partials, residual, gamma, eps: float = 1e-6, group: int = 128,
                                   emit_out: bool = True, nthreads: int | None = None):
    """FP8 call. Returns (residual_out [T,H] u16, out [T,H] u16 or None, q [T,H] u8 e4m3fn codes,
    scales [T, H/group] float32)."""
    plist = _partials_list(partials)
    T, H = plist[0].shape
    g = np.ascontiguousarray(gamma, dtype=np.uint16)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.uint16)
    res_out = _out((T, H), np.uint16)
    out = _out((T, H), np.uint16) if emit_out else None
    q = _out((T, H), np.uint8)
    scales = _out((T, H // group), np.float32)
    rc = lib().oracle_reduce_add_rmsnorm_quant_group(
        _ptr_array(plist), len(plist), None if res is None else _u16(res), _u16(g), eps, T, H, group,
        _u16(res_out), None if out is None else _u16(out),
        q.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
        scales.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _nthreads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_reduce_add_rmsnorm_quant_group failed ({rc})")
    return res_out, out, q, scales


def bf16_from_double(x: float) -> int:
    return int(lib().oracle_bf16_from_double(float(x)))


def e4m3fn_from_double(x: float) -> int:
    return int(lib().oracle_e4m3fn_from_double(float(x)))


def bf16_from_double_array(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_from_double_array(x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), _u16(y), x.size)
    return y


def e4m3fn_from_double_array(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3fn_from_double_array(x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                          y.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), x.size)
    return y


def reduce(partials) -> np.ndarray:
    """All-reduce alone: bf16 of the fp32 rank-order sum of the partials ([R,T,H] or list)."""
    plist = _partials_list(partials)
    T, H = plist[0].shape
    out = np.empty((T, H), np.uint16)
    if lib().oracle_reduce(_ptr_array(plist), len(plist), T, H, _u16(out)) != 0:
        raise RuntimeError("oracle_reduce failed")
    return out


def quant_group(x, group: int = 128):
    """Per-group E4M3 quant alone of a bf16 [T,H] array: returns (q uint8 [T,H], scales [T,H/group])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, H = x.shape
    q = np.empty((T, H), np.uint8)
    scales = np.empty((T, H // group), np.float32)
    rc = lib().oracle_quant_group(_u16(x), T, H, group, q.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                  scales.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    if rc != 0:
        raise RuntimeError("oracle_quant_group failed")
    return q, scales


def e2m1_from_double(x: float) -> int:
    return int(lib().oracle_e2m1_from_double(float(x)))


def e2m1_from_double_array(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, np.uint8)
    lib().oracle_e2m1_from_double_array(x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                        y.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), x.size)
    return y


def mxfp4(x):
    """MXFP4 of a bf16 [T,H] array (H % 32 == 0): (q uint8 [T, H/2] two E2M1 codes per byte,
    element 2i in the low nibble; scales uint8 [T, H/32] E8M0)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, H = x.shape
    q = np.empty((T, H // 2), np.uint8)
    sc = np.empty((T, H // 32), np.uint8)
    u8 = ctypes.POINTER(ctypes.c_uint8)
    if lib().oracle_mxfp4(_u16(x), T, H, q.ctypes.data_as(u8), sc.ctypes.data_as(u8)) != 0:
        raise RuntimeError("oracle_mxfp4 failed")
    return q, sc


def reduce_add_rmsnorm_mxfp4(partials, residual, gamma, eps: float = 1e-6, emit_out: bool = True,
                             nthreads: int | None = None):
    """Fused call with MXFP4 output: (residual_out, out or None, q [T,H/2] u8, scales [T,H/32] u8)."""
    plist = _partials_list(partials)
    T, H = plist[0].shape
    g = np.ascontiguousarray(gamma, dtype=np.uint16)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.uint16)
    res_out = _out((T, H), np.uint16)
    out = _out((T, H), np.uint16) if emit_out else None
    q = _out((T, H // 2), np.uint8)
    sc = _out((T, H // 32), np.uint8)
    u8 = ctypes.POINTER(ctypes.c_uint8)
    rc = lib().oracle_reduce_add_rmsnorm_mxfp4(
        _ptr_array(plist), len(plist), None if res is None else _u16(res), _u16(g), eps, T, H,
        _u16(res_out), None if out is None else _u16(out), q.ctypes.data_as(u8), sc.ctypes.data_as(u8),
        _nthreads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_reduce_add_rmsnorm_mxfp4 failed")
    return res_out, out, q, sc
