"""Exhaustive CPU checks of the kernels' two number encoders, as arithmetic models.

The GPU parity tests sample the encoders on realistic data; these tests cover their whole
input space. Each model below repeats, in numpy fp32 and integer arithmetic, the operation
sequence of the corresponding device function in tp_all_reduce_amd/csrc/farn_kernels.hip
(`e4m3_mag` with the tiny-group rescaling of `quant_slot`, and `e2m1_code`), and is compared
with the oracle's encoder of the exact value. A model is only as faithful as its transcription:
a change to either device function must be repeated here.

fp32 steps map one to one onto numpy float32 operations (round to nearest even, subnormals
kept); fp32 FMAs are modelled exactly (`_fma32`). The E4M3 reference is the oracle's encoder of
the binary32 quotient out/scale (numpy's IEEE single division).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

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


def e4m3_mag_model(o: np.ndarray, scale_r: np.float32, inv: np.float32) -> np.ndarray:
    """Model of `e4m3_mag(o, scale_r, inv)`: magnitude code of fl32(|o| / scale)."""
    ao = np.abs(o.astype(np.float32))
    with np.errstate(invalid="ignore", over="ignore"):
        q0 = (ao * F32(inv)).astype(np.float32)
        r = _fma32(-q0, np.full_like(q0, scale_r), ao)
        v = _fma32(r, np.full_like(q0, inv), q0)
        b = v.view(np.uint32).astype(np.uint64)
        cn = (((b + 0x7FFFF + ((b >> 20) & 1)) >> 20) & 0xFFFFFFFF).astype(np.int64) - 960
        cs = np.rint((v * F32(512.0)).astype(np.float32))
        cs = np.where(np.isfinite(cs), cs, 0).astype(np.int64)
    c = np.minimum(np.where(v < F32(2.0 ** -6), cs, cn), 0x7E)
    return np.where(np.isnan(v), 0x7F, c).astype(np.uint8)


def group_codes_model(o: np.ndarray, amax: np.float32) -> tuple[np.ndarray, np.float32]:
    """Model of `quant_slot`'s per-group arithmetic for a group with max magnitude amax:
    scale = amax/448 correctly rounded, the 2^64 rescaling of tiny groups, inv = 1/scale, the
    remainder's scale clamped to the largest finite float."""
    scale = F32(np.float64(amax) / 448.0)  # amax/448 is never a tie in fp32, so one rounding
    k = F32(2.0 ** 64) if scale < F32(2.0 ** -64) else F32(1.0)
    sk = F32(scale * k)
    with np.errstate(divide="ignore"):
        inv = F32(0.0) if scale == 0 else F32(1.0) / sk
    sr = min(sk, np.finfo(np.float32).max)
    return e4m3_mag_model((o.astype(np.float32) * k).astype(np.float32), F32(sr), inv), scale


def e2m1_model(x: np.ndarray) -> np.ndarray:
    """Model of `e2m1_code(x)`: sign bit 3, magnitude code 0..7."""
    x = x.astype(np.float32)
    a = np.abs(x)
    small = a < F32(1.0)
    b = (a + np.where(small, F32(1.0), F32(0.0))).astype(np.float32).view(np.uint32).astype(np.uint64)
    kept = (b + 0x1FFFFF + ((b >> 22) & 1)) >> 22
    c = np.minimum(kept.astype(np.int64) - np.where(small, 254, 252), 7)
    return (((x.view(np.uint32) >> 28) & 8).astype(np.int64) | c).astype(np.uint8)


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


def _check_e4m3_groups(amax_patterns: np.ndarray) -> int:
    checked = 0
    for ab in amax_patterns:
        amax = np.array([ab << 16], np.uint32).view(np.float32)[0]
        o = FINITE_BF16[np.abs(FINITE_BF16) <= amax]      # every bf16 value the group can hold
        got, scale = group_codes_model(o, amax)
        with np.errstate(divide="ignore"):
            v32 = (o / scale).astype(np.float32)              # IEEE single division
        ref = oracle.e4m3fn_from_double_array(v32.astype(np.float64)) & 0x7F
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (f"amax {amax!r}: o={o[bad[0]]!r} model {got[bad[0]]:#x} "
                               f"oracle {ref[bad[0]]:#x} ({bad.size} differ)")
        checked += o.size
    return checked


def test_e4m3_encoder_model():
    """Every finite bf16 value each group can hold, for ~3,300 group maxima (every subnormal
    one included): about 10^8 pairs, some seconds."""
    assert _check_e4m3_groups(_amax_patterns(3000, seed=1)) > 100_000_000


def test_e4m3_encoder_model_specials():
    # NaN -> 0x7F; anything at or above 448 -> 0x7E; zero -> 0; the tie 2^-10 -> 0, 3*2^-10 -> 2
    got = e4m3_mag_model(np.array([np.nan, 448.0, 464.0, 1e30, 0.0, 2.0 ** -10, 3 * 2.0 ** -10], np.float32),
                         F32(1.0), F32(1.0))
    assert got.tolist() == [0x7F, 0x7E, 0x7E, 0x7E, 0, 0, 2]
    # an inf group (scale inf, inv 0): finite values give 0, an infinite one NaN -> 0x7F
    codes, scale = group_codes_model(np.array([3.0, np.inf], np.float32), F32(np.inf))
    assert np.isinf(scale) and codes.tolist() == [0, 0x7F]
    # an all-zero group: scale 0, inv 0, every magnitude code 0
    codes, scale = group_codes_model(np.array([0.0, -0.0], np.float32), F32(0.0))
    assert scale == 0 and codes.tolist() == [0, 0]


def test_e2m1_encoder_model_exhaustive():
    """Every non-NaN bf16 value (each x the kernel encodes is a bf16 value times a power of
    two, so its significand is one of these), and a 2^-10 grid over [0, 8.5] with every tie."""
    x = ALL_BF16[~np.isnan(ALL_BF16)]
    ref = np.array([oracle.e2m1_from_double(float(v)) for v in x], np.uint8)
    assert np.array_equal(e2m1_model(x), ref)
    g = np.arange(0, 8.5, 2.0 ** -10)
    ref = np.array([oracle.e2m1_from_double(float(v)) for v in g], np.uint8)
    assert np.array_equal(e2m1_model(g.astype(np.float32)), ref)
