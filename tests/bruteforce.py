"""Slow, exact checkers used to pin the CPU oracle (never the GPU path's code).

Everything here works on exact rationals (fractions.Fraction) or 60-digit
decimals, and decodes number formats from their public definitions:
  * bfloat16: upper half of IEEE-754 binary32 (8 exponent bits, bias 127, 7
    mantissa bits, subnormals below 2^-126);
  * E4M3 of the OCP 8-bit floating point specification (OFP8): exponent bias 7,
    3 mantissa bits, subnormals m/8 * 2^-6, S.1111.111 = NaN, no infinities.
Nearest-value rounding is done by search / exact comparison, with ties going to
the code whose last mantissa bit is 0, so it shares no method with the oracle's
frexp/nearbyint encoders.
"""

from __future__ import annotations

import decimal
import math
import struct
from fractions import Fraction

import numpy as np

decimal.getcontext().prec = 60


# ----------------------------------------------------------------------------- bf16
def bf16_bits_to_fraction(b: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]
    assert math.isfinite(f)
    return Fraction(f)


def bf16_bits_to_float(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _floor_log2(q: Fraction) -> int:
    """Exact floor(log2(q)) for q > 0."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def _round_half_even(x: Fraction) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def bf16_nearest(q: Fraction, negative_zero: bool = False) -> int:
    """bf16 bits of the value nearest to the exact rational q (ties to even mantissa)."""
    sign = 0x8000 if (q < 0 or (q == 0 and negative_zero)) else 0
    a = abs(q)
    if a == 0:
        return sign
    e = max(_floor_log2(a), -126)
    quantum = Fraction(2) ** (e - 7)
    m = _round_half_even(a / quantum)
    r = m * quantum
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = struct.unpack("<I", struct.pack("<f", float(r)))[0]
    assert Fraction(struct.unpack("<f", struct.pack("<I", bits))[0]) == r and bits & 0xFFFF == 0
    return sign | (bits >> 16)


# ----------------------------------------------------------------------------- e4m3fn
def e4m3fn_decode(code: int) -> Fraction | None:
    """Value of an OCP E4M3 code, or None for NaN."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return None
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


E4M3_POS = [(c, e4m3fn_decode(c)) for c in range(0x7F)]  # 0x00 .. 0x7E, all finite, ascending


def e4m3fn_decode_array(codes) -> np.ndarray:
    table = np.array([float(e4m3fn_decode(c)) if e4m3fn_decode(c) is not None else np.nan
                      for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_nearest(v: Fraction, negative_zero: bool = False) -> int:
    """Code nearest to v by search over every finite code; ties go to the even code;
    magnitudes above 448 saturate to 448 (satfinite)."""
    sign = 0x80 if (v < 0 or (v == 0 and negative_zero)) else 0
    a = abs(v)
    best = None
    for c, val in E4M3_POS:
        d = abs(a - val)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return sign | best[1]


def e4m3_step(v: float) -> float:
    """Spacing of E4M3 codes around |v|: 2^(max(floor(log2|v|), -6) - 3)."""
    a = abs(v)
    e = -6 if a == 0 else max(math.floor(math.log2(a)), -6)
    return 2.0 ** (e - 3)


# ----------------------------------------------------------------------------- the op, exactly
def exact_row_stats(yb_bits, eps: float) -> decimal.Decimal:
    """rstd = 1/sqrt(mean(y^2) + eps) to 60 digits, for a row of bf16 bits; eps as binary32."""
    H = len(yb_bits)
    ss = sum(bf16_bits_to_fraction(b) ** 2 for b in yb_bits)
    ms = ss / H + Fraction(float(np.float32(eps)))
    d = decimal.Decimal(ms.numerator) / decimal.Decimal(ms.denominator)
    return 1 / d.sqrt()


def exact_out_row(yb_bits, gamma_bits, eps: float) -> list[int]:
    """bf16 out for one row from the exact mean of squares, one rounding."""
    rstd = exact_row_stats(yb_bits, eps)
    res = []
    for y, g in zip(yb_bits, gamma_bits):
        yf, gf = bf16_bits_to_fraction(y), bf16_bits_to_fraction(g)
        prod = decimal.Decimal(yf.numerator) / decimal.Decimal(yf.denominator) * rstd \
            * decimal.Decimal(gf.numerator) / decimal.Decimal(gf.denominator)
        neg0 = (yf == 0 and (y & 0x8000) != (g & 0x8000))
        res.append(bf16_nearest(Fraction(prod), negative_zero=neg0))
    return res
