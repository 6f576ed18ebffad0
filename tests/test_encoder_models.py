"""Exhaustive CPU check of the arithmetic the FP8 kernel does before its conversion
instruction: the binary32 quotient o / scale computed without a divide (`fp32_quotient` in
tp_all_reduce_amd/csrc/farn_kernels.hip: q0 = o*inv, the negated remainder nr = q0*scale - o by
FMA, q0 - nr*inv by FMA; with `quant_slots`' per-group scale, 2^64 rescaling of tiny groups and clamped remainder
scale). That quotient can differ from the correctly rounded one by an fp32 unit; this test
shows that its round-to-nearest-even E4M3 code never does, for every finite bf16 value each
group can hold, over ~3,300 group maxima (every bf16 subnormal amax included), signed zeros
included (a -0 value keeps the -0 code 0x80 the division gives). The conversion
instruction's own rounding is checked on the GPU (tests/test_gpu_conversions.py); here it is
the oracle's E4M3 encoder. A model is only as faithful as its transcription: a change to
`fp32_quotient` or to `quant_slots`' per-group arithmetic must be repeated here.

fp32 steps map one to one onto numpy float32 operations (round to nearest even, subnormals
kept); fp32 FMAs are modelled exactly (`_fma32`). The reference is the oracle's encoder of the
binary32 quotient out/scale (numpy's IEEE single division).
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

F32 = np.float32


def _fma32(a, b, c) -> np.ndarray:
    """fp32 FMA a*b + c with one rounding, for arrays of one shape. a*b is exact in binary64
    (24 + 24 bits); the binary64 sum is re-done in exact rationals wherever its result sits on
    an fp32 rounding boundary (the only place rounding it again could differ from one rounding)."""
    a64, b64, c64 = (np.asarray(x, np.float32).astype(np.float64) for x in (a, b, c))
    x = a64 * b64 + c64
    with np.errstate(over="ignore", invalid="ignore"):
        out = x.astype(np.float32)
    edge = np.isfinite(x) & ((x.view(np.uint64) & np.uint64((1 << 29) - 1)) == np.uint64(1 << 28))
    for i in np.nonzero(edge)[0]:
        exact = Fraction(float(a64[i])) * Fraction(float(b64[i])) + Fraction(float(c64[i]))
        y = out[i]
        cands = [np.nextafter(y, F32(-np.inf)), y, np.nextafter(y, F32(np.inf))]
        out[i] = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact), int(np.array(v).view(np.uint32)) & 1))
    return out


def quotient_model(o: np.ndarray, scale_r: np.float32, inv: np.float32) -> np.ndarray:
    """Model of `fp32_quotient(o, scale_r, inv)`."""
    o = np.asarray(o, np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        q0 = (o * F32(inv)).astype(np.float32)
        nr = _fma32(q0, np.full_like(q0, scale_r), -o)
        return _fma32(-nr, np.full_like(q0, inv), q0)


def group_codes_model(o: np.ndarray, amax: np.float32) -> tuple[np.ndarray, np.float32]:
    """Model of `quant_slots`' per-group arithmetic for a group with max magnitude amax:
    scale = amax/448 correctly rounded, the 2^64 rescaling of tiny groups, inv = 1/scale (the
    kernel's FMA-corrected scale and Newton-refined reciprocal equal these two divisions for
    every bf16 amax: test_fast_scale_is_the_division here, and on the GPU
    tests/test_gpu_conversions.py), the
    remainder's scale clamped to the largest finite float; codes are the round-to-nearest-even
    E4M3 codes of the quotients (the conversion instruction; here the oracle's encoder)."""
    scale = F32(np.float64(amax) / 448.0)  # amax/448 is never a tie in fp32, so one rounding
    k = F32(2.0 ** 64) if scale < F32(2.0 ** -64) else F32(1.0)
    sk = F32(scale * k)
    with np.errstate(divide="ignore"):
        inv = F32(0.0) if scale == 0 else F32(1.0) / sk
    sr = F32(min(sk, np.finfo(np.float32).max))
    v = quotient_model((np.asarray(o, np.float32) * k).astype(np.float32), sr, inv)
    return oracle.e4m3fn_from_double_array(v.astype(np.float64)), scale


ALL_BF16 = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
FINITE_BF16 = ALL_BF16[np.isfinite(ALL_BF16)]


def _amax_patterns(n_random: int, seed: int = 0) -> np.ndarray:
    """bf16 magnitude patterns of group maxima: every subnormal, the band where scale crosses
    2^-64, a few landmarks, and n_random random normals."""
    rng = np.random.default_rng(seed)
    fixed = np.concatenate([np.arange(0x0001, 0x0080),                 # bf16 subnormals
                            np.arange(0x1F00, 0x2100, 3),              # scale near 2^-64
                            [0x0080, 0x0400, 0x3C00, 0x3F80, 0x4000, 0x43E0, 0x7F7F]])
    return np.concatenate([fixed, rng.integers(0x0080, 0x7F80, n_random)]).astype(np.uint32)


def _check_groups(amax_patterns: np.ndarray) -> int:
    checked = 0
    for ab in amax_patterns:
        amax = np.array([ab << 16], np.uint32).view(np.float32)[0]
        o = FINITE_BF16[np.abs(FINITE_BF16) <= amax]      # every bf16 value the group can hold
        got, scale = group_codes_model(o, amax)
        with np.errstate(divide="ignore"):
            v32 = (o / scale).astype(np.float32)              # IEEE single division
        want = oracle.e4m3fn_from_double_array(v32.astype(np.float64))
        bad = np.nonzero(got != want)[0]  # bit for bit, signed zeros included
        assert bad.size == 0, (f"amax {amax!r}: o={o[bad[0]]!r} model {got[bad[0]]:#x} "
                               f"binary32 quotient's code {want[bad[0]]:#x} ({bad.size} differ)")
        checked += o.size
    return checked


def test_quotient_codes():
    """Every finite bf16 value each group can hold, for ~3,300 group maxima: about 10^8 pairs."""
    assert _check_groups(_amax_patterns(3000, seed=1)) > 100_000_000


def test_quotient_codes_every_amax():
    """Opt-in (FARN_MODEL_EVERY_AMAX=1, a few minutes): every finite nonzero bf16 magnitude as
    the group maximum, with every bf16 value the group can hold: about 1.07e9 pairs."""
    if not os.environ.get("FARN_MODEL_EVERY_AMAX"):
        pytest.skip("set FARN_MODEL_EVERY_AMAX=1 to check every bf16 group maximum (a few minutes)")
    assert _check_groups(np.arange(0x0001, 0x7F80, dtype=np.uint32)) > 1_000_000_000


def test_quotient_model_specials():
    # -0 keeps its sign through the correction (code 0x80, as -0 / scale gives), +0 stays +0
    codes, _ = group_codes_model(np.array([-0.0, 0.0, -1.0, 1.0], np.float32), F32(1.0))
    assert codes.tolist()[:2] == [0x80, 0x00]
    # an all-zero group: scale 0, inv 0, quotients +-0 (the kernel masks their signs)
    codes, scale = group_codes_model(np.array([0.0, -0.0], np.float32), F32(0.0))
    assert scale == 0 and (codes & 0x7F).tolist() == [0, 0]
    # an inf group (scale inf, inv 0): a finite value's quotient is 0, an infinite one's NaN
    v = quotient_model(np.array([3.0, -2.0, np.inf], np.float32), F32(np.finfo(np.float32).max), F32(0.0))
    assert v[0] == 0 and v[1] == 0 and np.isnan(v[2])
    # 400 is the E4M3 tie between 384 and 416 and goes to 384 (the even code): a group of
    # amax 448 has scale 1, so its quotient is exactly 400
    codes, _ = group_codes_model(np.array([400.0], np.float32), F32(448.0))
    assert codes.tolist() == [0x7C]


def test_uncorrected_product_would_fail():
    """The correction step is needed: the plain product o * (1/scale) lands on the wrong side
    of binary32 ties (a group the sweep found: amax bf16 0x00C4, a subnormal)."""
    amax = np.array([0x00C4 << 16], np.uint32).view(np.float32)[0]
    o = FINITE_BF16[np.abs(FINITE_BF16) <= amax]
    scale = F32(np.float64(amax) / 448.0)
    k = F32(2.0 ** 64)
    sk = F32(scale * k)
    inv = F32(1.0) / sk
    q0 = ((o * k).astype(np.float32) * inv).astype(np.float32)
    v32 = (o / scale).astype(np.float32)
    assert (oracle.e4m3fn_from_double_array(q0.astype(np.float64)) !=
            oracle.e4m3fn_from_double_array(v32.astype(np.float64))).any()


# ----------------------------------------------------------------------------- normalisation
def norm_model(y_bits: np.ndarray, g_bits: np.ndarray, rstd: float):
    """Model of `norm_slot` in tp_all_reduce_amd/csrc/farn_kernels.hip for one row's rstd:
    the fp32 fast path (yg = y*gamma, p = yg * fl32(rstd), bf16 rounding of p), the test that
    sends a value to the fp64 path (yg not a normal number, fl32(rstd) not a positive normal
    number, low 16 bits of p within 0x7FFD .. 0x8003), and the fp64 path ((y*rstd)*gamma
    rounded once, here by the oracle's encoder). Returns (bf16 bits, mask of values that took
    the fp64 path). The kernel takes the fp64 path for a whole wave when any lane needs it;
    the fp64 path gives the one-rounding result for every value, so modelling it per value
    checks the same thing."""
    y = (y_bits.astype(np.uint32) << 16).view(np.float32)
    g = (g_bits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        r32 = np.float32(rstd)
        yg = (y * g).astype(np.float32)
        p = (yg * r32).astype(np.float32)
    normal = lambda x: np.isfinite(x) & (np.abs(x) >= np.float32(2.0 ** -126))
    r_ok = bool(np.isfinite(r32) and r32 >= np.float32(2.0 ** -126))
    near = ((p.view(np.uint32) - np.uint32(0x7FFD)) & np.uint32(0xFFFF)) <= 6
    slow = ~normal(yg) | near | (not r_ok)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        fast_bits = oracle.bf16_from_double_array(p.astype(np.float64))
        exact = (y.astype(np.float64) * rstd) * g.astype(np.float64)
    slow_bits = oracle.bf16_from_double_array(exact)
    return np.where(slow, slow_bits, fast_bits), slow


def _bf16_of(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_norm_fast_path_equals_one_rounding():
    """Wherever the fast path is kept, its bf16 value equals the single rounding of the fp64
    product (y*rstd)*gamma: on random rows, on rows built so that the products land within a
    few fp32 units of bf16 midpoints, and with zero, subnormal, huge, inf and NaN operands."""
    rng = np.random.default_rng(7)
    checked = slow_total = 0
    # random rows: y ~ N(0, 1), gamma ~ U(0.5, 1.5), rstd over many binades
    for _ in range(40):
        y = _bf16_of(rng.standard_normal(1 << 16) * rng.choice([1e-3, 1.0, 30.0]))
        g = _bf16_of(rng.uniform(0.5, 1.5, 1 << 16))
        rstd = float(np.exp(rng.uniform(np.log(2.0 ** -40), np.log(2.0 ** 40))))
        got, slow = norm_model(y, g, rstd)
        want = oracle.bf16_from_double_array((((y.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * rstd)
                                              * (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)))
        assert np.array_equal(got, want)
        checked += y.size
        slow_total += int(slow.sum())
    assert slow_total < 0.001 * checked  # the fp64 path is rare on data like this
    # adversarial: rstd chosen so that y*gamma*rstd sits within +-8 fp32 units of a bf16 midpoint
    n = 1 << 16
    y = _bf16_of(rng.standard_normal(n))
    g = _bf16_of(rng.uniform(0.5, 1.5, n))
    yf = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gf = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    target_bf = _bf16_of(rng.standard_normal(n) * 3)
    mid = ((target_bf.astype(np.uint32) << 16) | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    for k in range(-8, 9):
        for j in range(0, n, 4096):
            sl = slice(j, j + 4096)
            # one rstd per row: take the first element's target, offset by k fp32 units
            y0, g0, m0 = yf[sl][0], gf[sl][0], mid[sl][0]
            if y0 == 0 or m0 == 0 or np.sign(y0 * g0) != np.sign(m0):
                continue
            m_bits = np.array([m0], np.float32).view(np.uint32)[0]
            tgt = np.array([m_bits + np.uint32(k & 0xFFFFFFFF)], np.uint32).view(np.float32)[0]
            rstd = float(tgt) / (y0 * g0)
            got, slow = norm_model(y[sl], g[sl], rstd)
            want = oracle.bf16_from_double_array((yf[sl] * rstd) * gf[sl])
            assert np.array_equal(got, want), (k, j)
            checked += 4096
            if abs(k) <= 2:
                assert slow[0], (k, "a product within 2 units of a midpoint must take the fp64 path")
    # special operands
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0,
                         0x3F80, 0x0100, 0x1000], np.uint16)
    yy, gg = np.meshgrid(specials, specials)
    for rstd in (1.0, 2.0 ** -60, 2.0 ** 60, 2.0 ** -130, 1e300, 0.0, float("inf")):
        got, _ = norm_model(yy.ravel(), gg.ravel(), rstd)
        with np.errstate(all="ignore"):
            want = oracle.bf16_from_double_array(((yy.ravel().astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                                                  * rstd) * (gg.ravel().astype(np.uint32) << 16).view(np.float32)
                                                 .astype(np.float64))
        same = (got == want) | (((got & 0x7FFF) > 0x7F80) & ((want & 0x7FFF) > 0x7F80))
        assert same.all(), (rstd, yy.ravel()[~same][:4], gg.ravel()[~same][:4])
    assert checked > 2_000_000


def fast_scale_model(amax: np.ndarray) -> np.ndarray:
    """Model of the kernel's scale for finite amax: q0 = amax * RN(1/448), then
    q0 + (amax - q0 * 448) * RN(1/448) by two FMAs (`quant_slots`)."""
    c = F32(1.0) / F32(448.0)
    a = np.asarray(amax, np.float32)
    q0 = (a * c).astype(np.float32)
    r = _fma32(-q0, np.full_like(q0, 448.0), a)
    return _fma32(r, np.full_like(q0, c), q0)


def test_fast_scale_is_the_division():
    """For every finite non-negative bf16 amax (zero and subnormals included) the FMA-corrected
    product equals the correctly rounded amax/448; also in exact rationals on a sample."""
    amax = ALL_BF16[:0x7F80]  # the magnitude patterns 0x0000 .. 0x7F7F: every finite amax
    assert np.isfinite(amax).all() and amax.size == 32640
    got = fast_scale_model(amax)
    want = (amax / F32(448.0)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    c = Fraction(float(F32(1.0) / F32(448.0)))
    for a in amax[:: 97]:
        exact = Fraction(float(a)) / 448
        g = Fraction(float(fast_scale_model(np.array([a]))[0]))
        w = float(want[amax == a][0])
        assert g == Fraction(w) and abs(g - exact) <= abs(Fraction(float(np.nextafter(F32(w), F32(np.inf)))) - exact)
    assert c == Fraction(float.fromhex("0x1.24924ap-9"))


def test_uncorrected_scale_would_fail():
    """The product alone (no FMA correction) is not the division for some group maxima, so the
    previous test can tell the two apart."""
    amax = ALL_BF16[:0x7F80]
    q0 = (amax * (F32(1.0) / F32(448.0))).astype(np.float32)
    want = (amax / F32(448.0)).astype(np.float32)
    assert np.count_nonzero(q0.view(np.uint32) != want.view(np.uint32)) > 0
