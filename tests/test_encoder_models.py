"""Exhaustive CPU checks of the kernels' two number encoders, as arithmetic models.

The GPU parity tests sample the encoders on realistic data; these tests cover their whole
input space. Each model below repeats, in numpy fp32 and integer arithmetic, the operation
sequence of the corresponding device function in tp_all_reduce_amd/csrc/farn_kernels.hip
(`e4m3_mag` with the tiny-group rescaling of `quant_slot`, and `e2m1_code`), and is compared
with the oracle's encoder of the exact value. A model is only as faithful as its transcription:
a change to either device function must be repeated here.

fp32 steps map one to one onto numpy float32 operations (round to nearest even, subnormals
kept). The one FMA is modelled by its sign and zero-ness, which is all the encoder reads:
mid*scale is exact in binary64 (24 + 24 bits), so the binary64 difference |o| - mid*scale has
the exact difference's sign and is zero only when it is; the fp32 result is that difference
rounded once (modelled by rounding the binary64 value; the two can differ only for a nonzero
difference within a factor 2 of 2^-150, far below any group scale tested here).
"""

from __future__ import annotations

import numpy as np

import oracle

F32 = np.float32


def e4m3_mag_model(o: np.ndarray, scale: np.float32, inv: np.float32) -> np.ndarray:
    """Model of `e4m3_mag(o, scale, inv)`: magnitude code of |o| / scale."""
    ao = np.abs(o.astype(np.float32))
    with np.errstate(invalid="ignore", over="ignore"):
        a = (ao * F32(inv)).astype(np.float32)
        sub = a < F32(2.0 ** -6)
        off = np.where(sub, F32(2.0 ** -6), F32(0.0)).astype(np.float32)
        xb = (a + off).astype(np.float32).view(np.uint32)
        mid = (((xb & np.uint32(0xFFF00000)) | np.uint32(0x00080000)).view(np.float32) - off).astype(np.float32)
        d = (-mid.astype(np.float64) * np.float64(scale) + ao.astype(np.float64)).astype(np.float32)
    odd = ((xb >> np.uint32(20)) & np.uint32(1)).astype(np.uint64)
    neg = ((d.view(np.uint32).astype(np.uint64) + odd + 0xFFFFFFFF) & 0xFFFFFFFF) >> 31
    c = (xb >> np.uint32(20)).astype(np.int64) - np.where(sub, 967, 959) - neg.astype(np.int64)
    c = np.minimum(c, 0x7E)
    return np.where(np.isnan(a), 0x7F, c).astype(np.uint8)


def group_codes_model(o: np.ndarray, amax: np.float32) -> tuple[np.ndarray, np.float32]:
    """Model of `quant_slot`'s per-group arithmetic for a group with max magnitude amax:
    scale = amax/448 correctly rounded, the 2^64 rescaling of tiny groups, inv = 1/scale."""
    scale = F32(np.float64(amax) / 448.0)  # amax/448 is never a tie in fp32, so one rounding
    k = F32(2.0 ** 64) if scale < F32(2.0 ** -64) else F32(1.0)
    sk = F32(scale * k)
    with np.errstate(divide="ignore"):
        inv = F32(0.0) if scale == 0 else F32(1.0) / sk
    return e4m3_mag_model((o.astype(np.float32) * k).astype(np.float32), sk, inv), scale


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
        ref = oracle.e4m3fn_from_double_array(o.astype(np.float64) / np.float64(scale)) & 0x7F
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (f"amax {amax!r}: o={o[bad[0]]!r} model {got[bad[0]]:#x} "
                               f"oracle {ref[bad[0]]:#x} ({bad.size} differ)")
        checked += o.size
    return checked


def test_e4m3_encoder_model():
    """Every finite bf16 value each group can hold, for ~3,300 group maxima (every subnormal
    one included): about 10^8 pairs, a few seconds."""
    assert _check_e4m3_groups(_amax_patterns(3000, seed=1)) > 100_000_000


def test_e4m3_encoder_model_specials():
    # NaN quotient -> 0x7F; inf and anything at or above 448 -> 0x7E; zero -> 0
    got = e4m3_mag_model(np.array([np.nan, np.inf, 448.0, 464.0, 1e30, 0.0], np.float32), F32(1.0), F32(1.0))
    assert got.tolist() == [0x7F, 0x7E, 0x7E, 0x7E, 0x7E, 0]
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
