"""The GPU conversion instructions the quant paths rely on, checked exhaustively against the
oracle's encoders (which follow the format definitions).

- v_cvt_pk_fp8_f32 (the FP8 call's codes): every fp32 value in (-464, 464), -0 included,
  converts to the round-to-nearest-even OCP E4M3 code, sign of zero included (a negative
  value that rounds to zero gives 0x80). The FP8 path only ever converts
  quotients of magnitude below 464.
- v_cvt_scalef32_pk_fp4_f32 (the MXFP4 call's codes): every non-NaN bf16 value x under every
  E8M0 block exponent s = -127 .. 127 converts to the E2M1 code of x * 2^-s, round to nearest
  even code, saturating at 6.

Test kernels: tests/hw_conversions.hip (built into tests/libhwconv.so by the package build).
"""

from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhwconv.so")


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def hw():
    if not os.path.exists(LIB_PATH):
        pytest.fail("tests/libhwconv.so is not built (python tp_all_reduce_amd/build.py builds it)")
    L = ctypes.CDLL(LIB_PATH)
    L.hwconv_fp8_of_bits.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    L.hwconv_fp4_all_scales.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    L.hwconv_rsq_newton.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    L.hwconv_fp8_scale_inv.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    return L


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("lo,hi", [(0x00000000, 0x43E80000), (0x80000000, 0xC3E80000)],
                         ids=["positive_below_464", "negative_to_-464"])
def test_fp8_conversion_is_rne_e4m3(hw, lo, hi):
    chunk = 1 << 26
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for base in range(lo, hi, chunk):
        n = min(chunk, hi - base) & ~1
        say(f"[gpu] v_cvt_pk_fp8_f32 over fp32 patterns {base:#010x} .. {base + n:#010x}")
        assert hw.hwconv_fp8_of_bits(base, out.data_ptr(), n, _stream()) == 0
        torch.cuda.synchronize()
        got = out[:n].cpu().numpy()
        x = np.arange(base, base + n, dtype=np.uint64).astype(np.uint32).view(np.float32).astype(np.float64)
        want = oracle.e4m3fn_from_double_array(x)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (f"{bad.size} codes differ, first x={x[bad[0]]!r}: "
                               f"conversion {got[bad[0]]:#04x}, RNE E4M3 {want[bad[0]]:#04x}")


def test_fp4_scaled_conversion_is_rne_e2m1(hw):
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = np.ascontiguousarray(x[~np.isnan(x)])
    if x.size % 2:
        x = np.append(x, np.float32(0.0))
    n = x.size
    say(f"[gpu] v_cvt_scalef32_pk_fp4_f32: {n} bf16 values x 255 block exponents")
    xd = torch.from_numpy(x).to("cuda")
    out = torch.empty(n * 255, dtype=torch.uint8, device="cuda")
    assert hw.hwconv_fp4_all_scales(xd.data_ptr(), out.data_ptr(), n, _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(255, n)
    x64 = x.astype(np.float64)
    for k in range(255):
        s = k - 127
        want = oracle.e2m1_from_double_array(np.ldexp(x64, -s))
        bad = np.nonzero(got[k] != want)[0]
        assert bad.size == 0, (f"s={s}: {bad.size} codes differ, first x={x64[bad[0]]!r}: "
                               f"conversion {got[k][bad[0]]:#x}, E2M1 {want[bad[0]]:#x}")


def test_rsq_newton_within_two_units(hw):
    """The fused kernels' rstd: v_rsq_f64 refined by two Newton steps, for m over the whole range
    they use it for (2^-1000 .. 2^1000), is within two fp64 units of 1/sqrt(m) (numpy's, itself
    within one unit of the exact value), and where it differs it is still one of the fp64 values
    next to the exact root (checked in exact rationals). The raw instruction's accuracy is
    reported: one Newton step from it leaves up to ~20 units, hence two."""
    from fractions import Fraction
    rng = np.random.default_rng(3)
    m = np.exp(rng.uniform(np.log(2.0 ** -1000), np.log(2.0 ** 1000), 1 << 20))
    m = np.concatenate([m, rng.uniform(0.5, 2.0, 1 << 18), 2.0 ** np.arange(-1000, 1001, 1.0),
                        [1e-6, 1.0 + 1e-6, 3.0, 7168.0, 1.0 / 7168.0, 1.500721694963552e+237]])
    md = torch.from_numpy(m).to("cuda")
    out = torch.empty(2 * m.size, dtype=torch.float64, device="cuda")
    say(f"[gpu] rsq + Newton over {m.size} values of m")
    assert hw.hwconv_rsq_newton(md.data_ptr(), out.data_ptr(), m.size, _stream()) == 0
    torch.cuda.synchronize()
    both = out.cpu().numpy().reshape(-1, 2)
    raw, got = both[:, 0], both[:, 1]
    ref = 1.0 / np.sqrt(m)
    raw_rel = np.abs(raw / ref - 1.0)
    ulps = np.abs(got.view(np.int64) - ref.view(np.int64))
    say(f"[gpu]   v_rsq_f64 alone: max relative error {raw_rel.max():.2e} (2^{np.log2(raw_rel.max()):.1f}); "
        f"refined: max {int(ulps.max())} unit(s) from 1/sqrt, {int((ulps > 0).sum())} of {m.size} not equal")
    assert ulps.max() <= 2, (m[ulps.argmax()], got[ulps.argmax()], ref[ulps.argmax()])
    for i in np.nonzero(ulps > 0)[0][:200]:
        lo, hi = sorted((got[i], ref[i]))
        lo_n, hi_n = np.nextafter(lo, -np.inf), np.nextafter(hi, np.inf)
        x = Fraction(float(m[i]))
        assert Fraction(float(lo_n)) ** 2 * x < 1 < Fraction(float(hi_n)) ** 2 * x, (m[i], got[i])


def test_fp8_scale_and_reciprocal_exact(hw):
    """The FP8 quant's group scale and its reciprocal, for every 16-bit magnitude pattern a bf16
    group maximum can have (zero, subnormals, normals, inf, every NaN): the FMA-corrected product
    by RN(1/448) equals the IEEE single division amax / 448 bit for bit (a NaN gives a NaN), and
    v_rcp_f32 refined by one Newton step equals the IEEE single division 1 / (scale * k) (k = 2^64
    below 2^-64, else 1; 0 for a zero scale), so the quotients of the quant are those whose codes
    the CPU model checks for every group maximum."""
    bits = (np.arange(0x8000, dtype=np.uint32) << 16)
    dbits = torch.from_numpy(bits.view(np.int32)).to("cuda")
    out = torch.empty(3 * bits.size, dtype=torch.float32, device="cuda")
    say(f"[gpu] FP8 scale and reciprocal over {bits.size} magnitude patterns")
    assert hw.hwconv_fp8_scale_inv(dbits.data_ptr(), out.data_ptr(), bits.size, _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, 3)
    amax = bits.view(np.float32)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        scale = amax / np.float32(448.0)
        k = np.where(scale < np.float32(2.0 ** -64), np.float32(2.0 ** 64), np.float32(1.0)).astype(np.float32)
        sk = (scale * k).astype(np.float32)
        inv = np.where(scale == 0, np.float32(0.0), np.float32(1.0) / sk).astype(np.float32)
    nan = np.isnan(scale)
    assert np.array_equal(np.isnan(got[:, 0]), nan)
    assert np.array_equal(got[~nan, 0].view(np.uint32), scale[~nan].view(np.uint32)), \
        amax[~nan][np.nonzero(got[~nan, 0].view(np.uint32) != scale[~nan].view(np.uint32))[0][:5]]
    assert np.array_equal(got[~nan, 2].view(np.uint32), sk[~nan].view(np.uint32))
    assert np.array_equal(np.isnan(got[:, 1]), nan)
    bad = np.nonzero(got[~nan, 1].view(np.uint32) != inv[~nan].view(np.uint32))[0]
    assert bad.size == 0, [(float(amax[~nan][i]), float(got[~nan, 1][i]), float(inv[~nan][i])) for i in bad[:5]]
