"""Pins of the CPU oracle against what the number formats, the mathematics and
library routines fix, independent of the oracle's own code.

Each `check_*` function takes no arguments, runs against whatever oracle build is
currently bound (see `oracle.using`), and raises AssertionError on a mismatch.
The pytest tests run them on the real oracle; `test_planted_mistakes_are_caught`
runs them on copies of the oracle with a mistake planted in the C source and
requires every such copy to fail at least one of them.
"""

from __future__ import annotations

import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bruteforce import (bf16_bits_to_float, bf16_bits_to_fraction, bf16_nearest, e4m3_step,
                        e4m3fn_decode, e4m3fn_decode_array, e4m3fn_nearest, exact_out_row)
from gen import CONFIGS, make_inputs
from golden_io import read_value_code_table, read_worked_example

EPS = 1e-6


def f2b(x) -> np.ndarray:
    """float array -> bf16 bits via torch's cast (inputs for tests only)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def ulp_dist_bf16(a, b) -> np.ndarray:
    """Distance in bf16 steps between two bf16 bit arrays (ordered-integer mapping)."""
    def ordered(x):
        x = np.asarray(x, dtype=np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    return np.abs(ordered(a) - ordered(b))


# ============================================================================ encoders
def check_bf16_encoder_vs_torch_cast():
    """binary32 -> bf16 must equal torch's float32 -> bfloat16 cast (RNE) on every class
    of binary32: random bit patterns, subnormals, near-overflow, specials."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    extra = np.array([0, 0x80000000, 0x00000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F7F8000,
                      0x7F7F7FFF, 0x3F808000, 0x3F818000, 0x3F80C000, 0x7F800000, 0xFF800000],
                     dtype=np.uint32)
    bits = np.concatenate([bits, extra, extra | 0x8000, np.arange(0x3F800000, 0x3F820000,
                                                                  dtype=np.uint32)])
    f = bits.view(np.float32)
    fin = ~np.isnan(f)
    ref = torch.from_numpy(f[fin].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_double_array(f[fin].astype(np.float64))
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, f"bf16 mismatch at {bits[fin][bad[:5]]}: torch {ref[bad[:5]]} oracle {got[bad[:5]]}"
    with np.errstate(invalid="ignore"):
        nan_out = oracle.bf16_from_double_array(f[~fin].astype(np.float64))
    assert np.all(np.isnan(bf16_bits_to_float(nan_out)))


def check_bf16_golden_rounding_points():
    for value, code in read_value_code_table("bf16_rounding.txt"):
        got = oracle.bf16_from_double(value)
        assert got == code, f"bf16({value!r}) = {got:04X}, expected {code:04X}"


def check_bf16_encoder_exact_on_doubles():
    """binary64 inputs (one rounding) against exact-rational rounding, incl. near-ties."""
    rng = np.random.default_rng(2)
    base = f2b(rng.standard_normal(2000).astype(np.float32) * 10.0)
    mid = [bf16_bits_to_fraction(b) * (1 + Fraction(1, 256)) for b in base if (b & 0x7F80) != 0x7F80]
    xs = []
    for m in mid[:600]:
        for d in (Fraction(0), Fraction(1, 2 ** 45), -Fraction(1, 2 ** 45)):
            xs.append(float(m * (1 + d)))
    xs += list(rng.standard_normal(2000) * 3.0)
    got = oracle.bf16_from_double_array(np.array(xs))
    for x, g in zip(xs, got):
        want = bf16_nearest(Fraction(x), negative_zero=(x == 0 and np.signbit(x)))
        assert g == want, f"bf16({x!r}) = {g:04X}, exact {want:04X}"


def check_e4m3_encoder_exhaustive_bf16():
    """Every bf16 value -> E4M3: nearest code by search over all finite codes (ties to the
    even code, |v| > 448 saturates), and torch's float8_e4m3fn cast where |v| <= 464."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        f = bf16_bits_to_float(bits).astype(np.float64)
    got = oracle.e4m3fn_from_double_array(f)
    fin = np.isfinite(f)
    assert np.all((got[np.isnan(f)] & 0x7F) == 0x7F)
    assert np.all(got[np.isinf(f)] == np.where(f[np.isinf(f)] > 0, 0x7E, 0xFE))
    # search over the code table, vectorised: distances to all 127 non-negative finite codes
    vals = np.array([float(v) for _, v in __import__("bruteforce").E4M3_POS])
    a = np.minimum(np.abs(f[fin]), 448.0)  # satfinite: beyond the largest code, the largest code
    d = np.abs(a[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & (np.arange(127)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    want = pick.astype(np.uint8) | np.where(np.signbit(f[fin]), 0x80, 0).astype(np.uint8)
    bad = np.nonzero(got[fin] != want)[0]
    assert bad.size == 0, f"e4m3 mismatch at {f[fin][bad[:5]]}: {got[fin][bad[:5]]} vs {want[bad[:5]]}"
    small = fin & (np.abs(f) <= 464)
    ref = torch.from_numpy(f[small].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, got[small])


def check_e4m3_encoder_exact_near_ties():
    """binary64 values just above / below each E4M3 midpoint round away from the tie."""
    vals = [v for _, v in __import__("bruteforce").E4M3_POS]
    xs = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        m = (lo + hi) / 2
        for d in (Fraction(0), Fraction(1, 2 ** 40), -Fraction(1, 2 ** 40)):
            xs.append(float(m * (1 + d)))
    got = oracle.e4m3fn_from_double_array(np.array(xs))
    for x, g in zip(xs, got):
        assert g == e4m3fn_nearest(Fraction(x)), f"e4m3({x!r}) = {g:02X}"


def check_e4m3_golden_codes():
    for value, code in read_value_code_table("e4m3fn_codes.txt"):
        got = oracle.e4m3fn_from_double(value)
        assert got == code, f"e4m3({value!r}) = {got:02X}, expected {code:02X}"
        if code not in (0x7F, 0xFF) and abs(value) <= 448 and e4m3fn_decode(code) == Fraction(value):
            assert float(e4m3fn_decode(code)) == value


# ============================================================================ worked examples
def check_worked_example_plain():
    g = read_worked_example("worked_example_plain.txt")
    ro, out = oracle.reduce_add_rmsnorm(g["partials"], g["residual"], g["gamma"], EPS)
    assert np.array_equal(ro, g["residual_out"]), (ro, g["residual_out"])
    assert np.array_equal(out, g["out"]), ([hex(x) for x in out.ravel()], g["out"])


def check_worked_example_quant():
    g = read_worked_example("worked_example_quant.txt")
    ro, out, q, sc = oracle.reduce_add_rmsnorm_quant_group(g["partials"], None, g["gamma"], EPS, 128)
    assert np.array_equal(ro, g["residual_out"])
    assert np.array_equal(out, g["out"])
    assert np.array_equal(q, g["q"]), q
    num, den = g["scale"].split("/")
    assert sc[0, 0] == np.float32(float(num)) / np.float32(float(den))


# ============================================================================ steps 1-3
def check_integer_sums_exact():
    """Small-integer partials and residual are exact in bf16 and their sums exact in fp32 in
    any order, so residual_out is the integer sum, for every R."""
    rng = np.random.default_rng(3)
    for R in range(1, 9):
        P = rng.integers(-16, 17, size=(R, 5, 16))
        res = rng.integers(-16, 17, size=(5, 16))
        g = f2b(np.ones(16))
        ro, _ = oracle.reduce_add_rmsnorm(f2b(P), f2b(res), g, EPS)
        want = P.sum(axis=0) + res
        assert np.array_equal(bf16_bits_to_float(ro), want.astype(np.float32)), R


def check_fold_order_and_precision():
    """Hand-built rows whose bf16 result depends on the order and precision of the sum.
    P = [1, 2^-8, 2^-24, 2^-24]: a binary32 left fold absorbs each 2^-24 (a tie at 1 + 2^-8,
    kept by ties-to-even), leaving 1 + 2^-8, a bf16 tie that rounds to 1.0 (0x3F80); a reversed
    fold or a binary64 sum keeps 2^-23 and rounds up to 0x3F81.
    P = [2^-24, 1, 2^-8] with residual 2^-24: residual added last gives 0x3F80; the residual
    added first keeps 2^-23 and gives 0x3F81."""
    g = f2b(np.ones(8))
    P = f2b(np.array([1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24])[:, None, None] * np.ones((1, 1, 8)))
    ro, _ = oracle.reduce_add_rmsnorm(P, None, g, EPS)
    assert np.all(ro == 0x3F80), ro
    P = f2b(np.array([2.0 ** -24, 1.0, 2.0 ** -8])[:, None, None] * np.ones((1, 1, 8)))
    ro, _ = oracle.reduce_add_rmsnorm(P, f2b(np.full((1, 8), 2.0 ** -24)), g, EPS)
    assert np.all(ro == 0x3F80), ro


def check_identities():
    """R=1 without residual returns P_0 bit for bit; P_1 = -P_0 returns the residual;
    negating every input negates residual_out and out exactly (RNE is symmetric)."""
    d = make_inputs(CONFIGS["tiny"], seed=11, R=1, T=5, H=64)
    ro, _ = oracle.reduce_add_rmsnorm(d["partials"], None, d["gamma"], EPS)
    assert np.array_equal(ro, d["partials"][0])
    d = make_inputs(CONFIGS["tiny"], seed=12, R=2, T=5, H=64)
    P = d["partials"].copy()
    P[1] = P[0] ^ 0x8000
    ro, _ = oracle.reduce_add_rmsnorm(P, d["residual"], d["gamma"], EPS)
    assert np.array_equal(bf16_bits_to_float(ro), bf16_bits_to_float(d["residual"]))
    d = make_inputs(CONFIGS["tiny"], seed=13, R=5, T=6, H=256)
    ro1, o1, q1, s1 = oracle.reduce_add_rmsnorm_quant_group(d["partials"], d["residual"], d["gamma"], EPS)
    ro2, o2, q2, s2 = oracle.reduce_add_rmsnorm_quant_group(d["partials"] ^ 0x8000, d["residual"] ^ 0x8000,
                                                           d["gamma"], EPS)
    nz = (ro1 & 0x7FFF) != 0
    assert np.array_equal(ro1[nz] ^ 0x8000, ro2[nz])
    nz = (o1 & 0x7FFF) != 0
    assert np.array_equal(o1[nz] ^ 0x8000, o2[nz])
    assert np.array_equal(s1, s2)
    nz = (q1 & 0x7F) != 0
    assert np.array_equal(q1[nz] ^ 0x80, q2[nz])


def check_reduce_vs_exact_sum():
    """residual_out against the bf16 nearest to the exact rational sum: equal except where the
    fp32 fold moved a value across a bf16 rounding boundary, and never more than 1 step off."""
    n_eq = n_all = 0
    for R, T, H, seed in [(2, 4, 256, 0), (1, 5, 16, 1), (3, 5, 16, 2), (8, 5, 16, 3), (6, 3, 64, 4)]:
        d = make_inputs(CONFIGS["tiny"], seed=seed, R=R, T=T, H=H)
        ro, _ = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], EPS)
        for t in range(T):
            for h in range(H):
                s = sum(bf16_bits_to_fraction(d["partials"][r, t, h]) for r in range(R))
                s += bf16_bits_to_fraction(d["residual"][t, h])
                want = bf16_nearest(s)
                n_all += 1
                n_eq += int(want == ro[t, h]) or int((want & 0x7FFF) == 0 and (ro[t, h] & 0x7FFF) == 0)
                assert ulp_dist_bf16([want], [ro[t, h]])[0] <= 1, (R, t, h)
    assert n_eq >= 0.99 * n_all, (n_eq, n_all)


# ============================================================================ steps 4-5
def check_norm_vs_exact():
    """out for tiny shapes equals the bf16 nearest to y*rstd*gamma with rstd from the exact
    mean of squares (60-digit decimal): the oracle's binary64 statistics must not move any
    bf16 result on these inputs."""
    for R, T, H, seed in [(2, 4, 256, 0), (1, 5, 16, 5), (4, 5, 16, 6), (8, 2, 48, 7)]:
        d = make_inputs(CONFIGS["tiny"], seed=seed, R=R, T=T, H=H)
        ro, out = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], EPS)
        for t in range(T):
            want = exact_out_row(list(ro[t]), list(d["gamma"]), EPS)
            assert list(out[t]) == want, (R, T, H, t)


# A row chosen so that its rstd lies within 1.2e-9 (relative) of a bf16 midpoint: R = 1, H = 8,
# y = [1, c, ..., c] with c = 0.9375, gamma = 1, eps the binary32 value 0x3DC917E0. Then
# out[0] = bf16(rstd), and rstd sits just above M = 1 + 2^-8, the midpoint between 1 and
# 1 + 2^-7. (c and eps came from a search over bf16 c and binary32 eps for rows where
# binary32 statistics round out[0] the other way; the pin checks both facts below.)
NEAR_MID_C = 0x3F70
NEAR_MID_EPS_BITS = 0x3DC917E0


def _near_mid_row():
    eps = float(np.array([NEAR_MID_EPS_BITS], np.uint32).view(np.float32)[0])
    y = np.array([[0x3F80] + [NEAR_MID_C] * 7], np.uint16)
    return y[None], np.full(8, 0x3F80, np.uint16), eps


def check_rstd_near_bf16_midpoint():
    """out rounds y*rstd*gamma once with rstd resolved beyond binary32: on the row above, the
    exact mean of squares m = ss/H + eps satisfies m * M^2 < 1 (rationals), so rstd > M and
    out[0] is 1 + 2^-7 (0x3F81); rstd computed in binary32 gives 1 (0x3F80) there. The whole
    row equals the exactly rounded one (60-digit rstd)."""
    partials, gamma, eps = _near_mid_row()
    c = bf16_bits_to_fraction(NEAR_MID_C)
    m = (1 + 7 * c * c) / 8 + Fraction(eps)
    M = 1 + Fraction(1, 256)
    assert m * M * M < 1 and 1 - m * M * M < Fraction(1, 10 ** 8)
    r32 = np.float32(1) / np.sqrt(np.float32(float((1 + 7 * c * c) / 8)) + np.float32(eps), dtype=np.float32)
    assert Fraction(float(r32)) <= M  # binary32 statistics land on the other side of M
    ro, out = oracle.reduce_add_rmsnorm(partials, None, gamma, eps)
    assert list(ro[0]) == list(partials[0, 0])
    assert out[0, 0] == 0x3F81, hex(out[0, 0])
    assert list(out[0]) == exact_out_row(list(ro[0]), list(gamma), eps)


def check_constant_rows():
    """A constant row y = c gives out = bf16(c/sqrt(c^2 + eps) * gamma): eps is added to the mean
    inside the square root. For |c| >> 1e-3 that is gamma * sign(c) bit for bit."""
    H = 256
    gamma = f2b(np.random.default_rng(4).uniform(0.5, 1.5, H))
    for c in (1.0, -2.0, 0.5, 3.0, 2.0 ** -10, 2.0 ** -12, -(2.0 ** -9)):
        P = f2b(np.full((1, 1, H), c))
        ro, out = oracle.reduce_add_rmsnorm(P, None, gamma, EPS)
        cf = Fraction(float(bf16_bits_to_float(P[0, 0, :1])[0]))
        want = exact_out_row([P[0, 0, 0]] * H, list(gamma), EPS)
        assert list(out[0]) == want, c
        if abs(c) >= 0.5:
            assert np.array_equal(out[0], gamma ^ (0x8000 if c < 0 else 0)), c
        # the closed form, checked on the first element in float terms
        exact = float(cf) / np.sqrt(float(cf) ** 2 + float(np.float32(EPS)))
        exact *= float(bf16_bits_to_float(gamma[:1])[0])
        assert abs(float(bf16_bits_to_float(out[0, :1])[0]) - exact) <= 2 ** -8 * abs(exact), c  # half a bf16 step


def check_vs_torch_rms_norm():
    """R = 1 without residual is plain RMSNorm: torch.nn.functional.rms_norm in float64 on the CPU,
    rounded to bf16 by the exact-rational rounding (not through binary32)."""
    for T, H, seed in [(4, 256, 0), (5, 16, 1), (8, 4096, 2), (3, 7168, 3)]:
        d = make_inputs(CONFIGS["tiny"], seed=seed, R=1, T=T, H=H)
        x = torch.from_numpy(bf16_bits_to_float(d["partials"][0]).astype(np.float64))
        w = torch.from_numpy(bf16_bits_to_float(d["gamma"]).astype(np.float64))
        ref = torch.nn.functional.rms_norm(x, (H,), weight=w, eps=float(np.float32(EPS))).numpy()
        want = oracle.bf16_from_double_array(ref)  # pinned above to exact rounding
        _, out = oracle.reduce_add_rmsnorm(d["partials"], None, d["gamma"], EPS)
        dist = ulp_dist_bf16(out, want)
        assert dist.max() <= 1 and (dist == 0).mean() >= 0.999, (T, H, dist.max(), (dist == 0).mean())


def check_constant_gamma_rms():
    """With gamma = c everywhere, RMS(out) = |c| * sqrt(ms / (ms + eps)) up to bf16 rounding."""
    d = make_inputs(CONFIGS["tiny"], seed=21, R=3, T=6, H=1024)
    for c in (1.0, 0.25, -3.0):
        gamma = f2b(np.full(1024, c))
        ro, out = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], gamma, EPS)
        y = bf16_bits_to_float(ro).astype(np.float64)
        ms = (y ** 2).mean(axis=1)
        rms = np.sqrt((bf16_bits_to_float(out).astype(np.float64) ** 2).mean(axis=1))
        want = abs(c) * np.sqrt(ms / (ms + float(np.float32(EPS))))
        assert np.all(np.abs(rms - want) <= 2 ** -8 * abs(c)), (c, rms, want)


def check_scale_invariance():
    """Scaling every partial and the residual by 4 (exact in bf16) scales residual_out by 4 exactly
    and leaves out unchanged but for eps, which may move a rare element by one bf16 step."""
    d = make_inputs(CONFIGS["tiny"], seed=22, R=4, T=8, H=512)
    ro1, o1 = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], EPS)
    up = lambda b: np.where((b & 0x7F80) != 0, b + (2 << 7), b).astype(np.uint16)  # exponent + 2
    ro2, o2 = oracle.reduce_add_rmsnorm(up(d["partials"]), up(d["residual"]), d["gamma"], EPS)
    assert np.array_equal(bf16_bits_to_float(ro2), 4 * bf16_bits_to_float(ro1))
    dist = ulp_dist_bf16(o1, o2)
    assert dist.max() <= 1 and (dist == 0).mean() >= 0.999


# ============================================================================ step 6
def _quant_case(seed, R, T, H, outliers=True):
    cfg = CONFIGS["decode_fp8"] if outliers else CONFIGS["tiny"]
    d = make_inputs(cfg, seed=seed, R=R, T=T, H=H)
    return d, oracle.reduce_add_rmsnorm_quant_group(d["partials"], d["residual"], d["gamma"], EPS, 128)


def check_quant_scale_and_max_code():
    """scale = binary32(amax / 448) recomputed from the group's bf16 out with IEEE single division,
    amax as torch.amax takes it (a NaN in the group makes it NaN), and every group with amax > 0
    holds a code of magnitude 448 (0x7E); a group holding a NaN out (here from one NaN gamma
    channel) has a NaN scale and only NaN codes, the other groups are untouched."""
    cases = [(0, 4, 16, 4096, None), (1, 2, 3, 256, None), (2, 8, 2, 1024, None), (3, 2, 2, 512, 130)]
    for seed, R, T, H, nan_ch in cases:
        d = make_inputs(CONFIGS["decode_fp8"], seed=seed, R=R, T=T, H=H)
        if nan_ch is not None:
            d["gamma"][nan_ch] = 0x7FC0
        ro, out, q, sc = oracle.reduce_add_rmsnorm_quant_group(d["partials"], d["residual"], d["gamma"], EPS, 128)
        o = torch.from_numpy(bf16_bits_to_float(out)).abs().reshape(T, H // 128, 128)
        amax = o.amax(dim=2).numpy().astype(np.float32)
        assert np.array_equal(sc, amax / np.float32(448.0), equal_nan=True)
        qq = q.reshape(T, H // 128, 128) & 0x7F
        nan_grp = np.isnan(amax)
        assert nan_grp.sum() == (0 if nan_ch is None else T)
        assert np.all((qq == 0x7F).all(axis=2)[nan_grp])
        assert np.all(((qq == 0x7E).any(axis=2) | (amax == 0))[~nan_grp])


def _fp32_quotient(bits, s) -> Fraction:
    """out/scale as a binary32 division (numpy's IEEE single division), as an exact rational."""
    return Fraction(float(np.float32(bf16_bits_to_float(np.uint16(bits))) / np.float32(s)))


def check_quant_codes_exact_small():
    """Codes equal the nearest E4M3 (by search over the decoded code table) to the binary32
    quotient out/scale, on tiny shapes."""
    for seed, R, T, H in [(3, 2, 2, 128), (4, 4, 1, 256)]:
        d, (ro, out, q, sc) = _quant_case(seed, R, T, H)
        for t in range(T):
            for h in range(H):
                v = _fp32_quotient(out[t, h], sc[t, h // 128])
                want = e4m3fn_nearest(v, negative_zero=(out[t, h] == 0x8000))
                assert q[t, h] == want, (t, h, q[t, h], want)


def check_quant_fp32_quotient_ties():
    """Where the binary32 quotient out/scale is exactly an E4M3 tie but the rational quotient is
    not, the two readings of out/scale round to different codes: the codes must follow the
    binary32 quotient. Every bf16 value of a few groups (scales not powers of two) is scanned for
    such points with the midpoints of the decoded code table."""
    codes = [c for c in range(0x7F) if e4m3fn_decode(c) is not None]
    vals = sorted(e4m3fn_decode(c) for c in codes)
    mids = np.array([float((a + b) / 2) for a, b in zip(vals, vals[1:])])
    found = 0
    for amax_f in (1.0, 3.0, 0.6875, 1.9375e-3, 37.5):
        amax_b = int(f2b(np.array([amax_f]))[0])
        s = np.float32(bf16_bits_to_float(np.uint16(amax_b))) / np.float32(448.0)
        obits = np.arange(1, amax_b + 1, dtype=np.uint16)                 # every bf16 value in (0, amax]
        of = bf16_bits_to_float(obits).astype(np.float32)
        v32 = (of / s).astype(np.float32)
        hit = np.nonzero(np.isin(v32.astype(np.float64), mids) &
                         (v32.astype(np.float64) != of.astype(np.float64) / np.float64(s)))[0]
        if hit.size == 0:
            continue
        x = np.zeros((len(hit), 128), np.uint16)
        x[:, 0] = amax_b
        x[:, 1] = obits[hit]
        q, sc = oracle.quant_group(x)
        assert np.all(sc[:, 0] == s)
        for i, j in enumerate(hit):
            vq = _fp32_quotient(obits[j], s)
            vr = Fraction(float(of[j])) / Fraction(float(s))
            want = e4m3fn_nearest(vq)
            assert q[i, 1] == want, (amax_f, float(of[j]), q[i, 1], want)
            found += int(want != e4m3fn_nearest(vr))
    assert found >= 5, found


def check_quant_dequant_bound():
    """|decode(q) * scale - out| <= (step(v)/2 + 2^-20 |v|) * scale with v = out/scale."""
    for seed, R, T, H in [(5, 4, 16, 4096), (6, 8, 4, 7168)]:
        d, (ro, out, q, sc) = _quant_case(seed, R, T, H)
        o = bf16_bits_to_float(out).astype(np.float64)
        s = np.repeat(sc.astype(np.float64), 128, axis=1)
        deq = e4m3fn_decode_array(q) * s
        v = o / s
        step = np.vectorize(e4m3_step)(v)
        assert np.all(np.abs(deq - o) <= (step / 2 + 2.0 ** -20 * np.abs(v)) * s)


def check_quant_zero_group_and_consistency():
    """An all-zero group gives scale 0 and codes 0; the FP8 call's residual_out / out equal the
    plain call's; emitting out or not changes nothing else."""
    d = make_inputs(CONFIGS["tiny"], seed=31, R=2, T=3, H=384)
    P = d["partials"].copy()
    res = d["residual"].copy()
    P[1, 1, 128:256] = P[0, 1, 128:256] ^ 0x8000  # cancels exactly
    res[1, 128:256] = 0
    ro, out, q, sc = oracle.reduce_add_rmsnorm_quant_group(P, res, d["gamma"], EPS)
    assert sc[1, 1] == 0 and np.all(q[1, 128:256] == 0)
    assert np.all(sc[[0, 2]] > 0)
    ro2, out2 = oracle.reduce_add_rmsnorm(P, res, d["gamma"], EPS)
    assert np.array_equal(ro, ro2) and np.array_equal(out, out2)
    ro3, none, q3, sc3 = oracle.reduce_add_rmsnorm_quant_group(P, res, d["gamma"], EPS, emit_out=False)
    assert none is None and np.array_equal(ro, ro3) and np.array_equal(q, q3) and np.array_equal(sc, sc3)


def check_in_place_residual():
    d = make_inputs(CONFIGS["tiny"], seed=41, R=3, T=4, H=256)
    ro, out = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], EPS)
    ro2, out2 = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], EPS, in_place=True)
    assert np.array_equal(ro, ro2) and np.array_equal(out, out2)


# ============================================================================ unfused blocks
def check_reduce_alone():
    """All-reduce alone: integer sums exact for every R; R=1 is the identity; the hand-built
    fold-order row; against the bf16 nearest to the exact rational sum."""
    rng = np.random.default_rng(5)
    for R in range(1, 9):
        P = rng.integers(-16, 17, size=(R, 3, 24))
        assert np.array_equal(bf16_bits_to_float(oracle.reduce(f2b(P))), P.sum(axis=0).astype(np.float32))
    d = make_inputs(CONFIGS["tiny"], seed=6, R=1, T=3, H=64)
    assert np.array_equal(oracle.reduce(d["partials"]), d["partials"][0])
    P = f2b(np.array([1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24])[:, None, None] * np.ones((1, 1, 8)))
    assert np.all(oracle.reduce(P) == 0x3F80)
    d = make_inputs(CONFIGS["tiny"], seed=7, R=8, T=3, H=32)
    ar = oracle.reduce(d["partials"])
    eq = 0
    for t in range(3):
        for h in range(32):
            want = bf16_nearest(sum(bf16_bits_to_fraction(d["partials"][r, t, h]) for r in range(8)))
            assert ulp_dist_bf16([want], [ar[t, h]])[0] <= 1
            eq += int(want == ar[t, h])
    assert eq >= 0.95 * 96


def check_quant_alone():
    """Quant alone on bf16 inputs with outliers: scale = IEEE single amax/448, a 448 code in every
    nonzero group, codes = nearest E4M3 of the binary32 quotient, zero groups give zeros."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    x[:, rng.choice(512, 6, replace=False)] *= 20
    x[2, 128:256] = 0.0
    xb = f2b(x)
    q, sc = oracle.quant_group(xb)
    amax = np.abs(bf16_bits_to_float(xb)).reshape(4, 4, 128).max(axis=2).astype(np.float32)
    assert np.array_equal(sc, amax / np.float32(448.0))
    assert sc[2, 1] == 0 and np.all(q[2, 128:256] == 0)
    qq = q.reshape(4, 4, 128) & 0x7F
    assert np.all((qq == 0x7E).any(axis=2) | (amax == 0))
    for t in range(4):
        for h in range(0, 512, 3):
            s = sc[t, h // 128]
            if s == 0:
                continue
            v = _fp32_quotient(xb[t, h], s)
            assert q[t, h] == e4m3fn_nearest(v, negative_zero=(xb[t, h] == 0x8000)), (t, h)
    # a NaN in one group: that group's scale is NaN (torch.amax takes NaN as the maximum) and
    # all its codes are NaN codes; the row's other groups are unchanged
    xn = xb.copy()
    xn[1, 300] = 0x7FC0
    qn, scn = oracle.quant_group(xn)
    amax_n = torch.from_numpy(bf16_bits_to_float(xn)).abs().reshape(4, 4, 128).amax(dim=2).numpy()
    assert np.array_equal(scn, amax_n.astype(np.float32) / np.float32(448.0), equal_nan=True)
    assert np.isnan(scn[1, 2]) and np.all(qn[1, 256:384] & 0x7F == 0x7F)
    keep = np.ones(512, bool)
    keep[256:384] = False
    assert np.array_equal(qn[1, keep], q[1, keep]) and np.array_equal(qn[[0, 2, 3]], q[[0, 2, 3]])


# ============================================================================ MXFP4
E2M1_VALUES = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
               Fraction(4), Fraction(6)]


def e2m1_nearest(v: Fraction) -> int:
    """E2M1 code nearest to v by search over the 8 magnitudes; ties to the even code; > 6 clamps."""
    sign = 0x8 if v < 0 else 0
    a = min(abs(v), Fraction(6))
    best = None
    for c, val in enumerate(E2M1_VALUES):
        d = abs(a - val)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return sign | best[1]


def check_e2m1_encoder():
    """Every finite bf16 value against the nearest-code search, and the OCP MX code table."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        f = bf16_bits_to_float(bits).astype(np.float64)
    for x in f[np.isfinite(f)][::7]:
        got = oracle.e2m1_from_double(float(x))
        want = e2m1_nearest(Fraction(float(x)))
        if x == 0 and np.signbit(x):
            want = 0x8
        assert got == want, (x, got, want)
    for value, code in read_value_code_table("e2m1_codes.txt"):
        assert oracle.e2m1_from_double(value) == code, (value, code)


def _decode_e2m1(c):
    return (-1 if c & 0x8 else 1) * float(E2M1_VALUES[c & 0x7])


def check_mxfp4_blocks():
    """Scales and codes of whole blocks: 2^(s+2) <= amax < 2^(s+3); the block maximum maps to 4 or
    6; dequantised values within half a step (or clamped at 6); zero and NaN blocks; element 2i in
    the low nibble."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 256)).astype(np.float32) * np.float32(3.0)
    x[:, rng.choice(256, 5, replace=False)] *= 20
    x[1, 32:64] = 0.0
    x[2, 64:96] *= np.float32(2.0 ** -100)
    xb = f2b(x)
    xb[3, 100] = 0x7FC0  # NaN in block 3 of row 3
    q, sc = oracle.mxfp4(xb)
    v = bf16_bits_to_float(xb).astype(np.float64)
    for t in range(6):
        for b in range(8):
            blk = v[t, 32 * b:32 * b + 32]
            codes = [(q[t, 16 * b + i // 2] >> (4 * (i % 2))) & 0xF for i in range(32)]
            if np.isnan(blk).any():
                assert sc[t, b] == 0xFF
                continue
            amax = np.abs(blk).max()
            if amax == 0:
                assert sc[t, b] == 0 and all(c == 0 for c in codes)
                continue
            s = int(sc[t, b]) - 127
            assert 2.0 ** (s + 2) <= amax < 2.0 ** (s + 3), (t, b, s, amax)
            X = 2.0 ** s
            top = int(np.argmax(np.abs(blk)))
            assert codes[top] & 0x7 in (6, 7)
            for i in range(32):
                r = blk[i] / X
                step = 0.5 if abs(r) < 2 else (1.0 if abs(r) < 4 else 2.0)
                err = abs(_decode_e2m1(codes[i]) - r)
                assert err <= step / 2 or (abs(r) > 6 and codes[i] & 0x7 == 7), (t, b, i, r, codes[i])
    # a block maximum of 2^-126: floor(log2 amax) - 2 = -128 is clamped to -127 (byte 0x00),
    # so the codes are V / 2^-127: 2^-126 -> 2 (code 4), 3*2^-128 -> 1.5 (code 3), -2^-128 ->
    # -0.5 (code 0x9); without the clamp the byte would wrap to 0xFF, the NaN scale
    z = np.zeros((1, 32), np.uint16)
    z[0, 0] = 0x0080  # 2^-126, the smallest normal bf16
    z[0, 1] = 0x0060  # 3 * 2^-128 = 96 * 2^-133 (subnormal)
    z[0, 2] = 0x8020  # -2^-128 = -32 * 2^-133
    qz, sz = oracle.mxfp4(z)
    assert sz[0, 0] == 0x00 and qz[0, 0] == 0x34 and qz[0, 1] == 0x09 and not qz[0, 2:].any(), (sz, qz)
    # nibble order: a block whose element 0 is the maximum and element 1 zero
    y = np.zeros((1, 32), np.float32)
    y[0, 0] = 4.0
    q1, s1 = oracle.mxfp4(f2b(y))
    assert q1[0, 0] == 0x06 and s1[0, 0] == 127


def check_mxfp4_fused_consistency():
    """The fused MXFP4 call's residual_out / out equal the plain call's, and its codes equal the
    MXFP4 of that out; with out not emitted, the codes are unchanged."""
    d = make_inputs(CONFIGS["decode_fp8"], seed=33, T=5, H=512)
    ro, out, q, sc = oracle.reduce_add_rmsnorm_mxfp4(d["partials"], d["residual"], d["gamma"], EPS)
    ro2, out2 = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], EPS)
    assert np.array_equal(ro, ro2) and np.array_equal(out, out2)
    q2, sc2 = oracle.mxfp4(out)
    assert np.array_equal(q, q2) and np.array_equal(sc, sc2)
    _, none, q3, sc3 = oracle.reduce_add_rmsnorm_mxfp4(d["partials"], d["residual"], d["gamma"], EPS,
                                                      emit_out=False)
    assert none is None and np.array_equal(q, q3) and np.array_equal(sc, sc3)


# ============================================================================ threaded row split
def check_threaded_rows_match_one_thread():
    """The fused calls deal rows round-robin to threads. With 2, 3, 8 and 16 threads, on row
    counts below, at and above the thread count and not multiples of it, every output must
    equal the one-thread result bit for bit (outputs start poisoned, so a row no thread writes,
    or one written twice with another row's values, shows). The one-thread path is what every
    other pin holds to the definition."""
    shapes = [(3, 1, 256), (2, 2, 128), (5, 3, 256), (4, 16, 384), (8, 17, 128), (2, 33, 256), (6, 50, 128)]
    with oracle.threads(1):
        for i, (R, T, H) in enumerate(shapes):
            d = make_inputs(CONFIGS["decode_fp8"], seed=700 + i, R=R, T=T, H=H)
            res = d["residual"] if i % 2 == 0 else None
            ref = (oracle.reduce_add_rmsnorm(d["partials"], res, d["gamma"], EPS),
                   oracle.reduce_add_rmsnorm_quant_group(d["partials"], res, d["gamma"], EPS),
                   oracle.reduce_add_rmsnorm_quant_group(d["partials"], res, d["gamma"], EPS, emit_out=False),
                   oracle.reduce_add_rmsnorm_mxfp4(d["partials"], res, d["gamma"], EPS),
                   oracle.reduce_add_rmsnorm_mxfp4(d["partials"], res, d["gamma"], EPS, emit_out=False))
            for n in (2, 3, 8, 16):
                got = (oracle.reduce_add_rmsnorm(d["partials"], res, d["gamma"], EPS, nthreads=n),
                       oracle.reduce_add_rmsnorm_quant_group(d["partials"], res, d["gamma"], EPS, nthreads=n),
                       oracle.reduce_add_rmsnorm_quant_group(d["partials"], res, d["gamma"], EPS,
                                                             emit_out=False, nthreads=n),
                       oracle.reduce_add_rmsnorm_mxfp4(d["partials"], res, d["gamma"], EPS, nthreads=n),
                       oracle.reduce_add_rmsnorm_mxfp4(d["partials"], res, d["gamma"], EPS, emit_out=False,
                                                       nthreads=n))
                for call, (a, b) in enumerate(zip(ref, got)):
                    for k, (x, y) in enumerate(zip(a, b)):
                        assert (x is None) == (y is None)
                        if x is not None:
                            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
                                f"R={R} T={T} H={H} threads={n}: call {call} output {k} differs"


ALL_CHECKS = [
    check_bf16_encoder_vs_torch_cast, check_bf16_golden_rounding_points, check_bf16_encoder_exact_on_doubles,
    check_e4m3_encoder_exhaustive_bf16, check_e4m3_encoder_exact_near_ties, check_e4m3_golden_codes,
    check_worked_example_plain, check_worked_example_quant,
    check_integer_sums_exact, check_fold_order_and_precision, check_identities, check_reduce_vs_exact_sum,
    check_norm_vs_exact, check_rstd_near_bf16_midpoint, check_constant_rows, check_vs_torch_rms_norm, check_constant_gamma_rms,
    check_scale_invariance,
    check_quant_scale_and_max_code, check_quant_codes_exact_small, check_quant_fp32_quotient_ties,
    check_quant_dequant_bound,
    check_quant_zero_group_and_consistency, check_in_place_residual,
    check_reduce_alone, check_quant_alone,
    check_e2m1_encoder, check_mxfp4_blocks, check_mxfp4_fused_consistency,
    check_threaded_rows_match_one_thread,
]


# Every pin runs on the one-thread oracle and again with its rows dealt to 3 and to 7 threads
# (outputs poisoned before each call): the GPU comparisons and the bench run the oracle
# threaded, so the threaded row split is held to the same pins.
PIN_THREADS = (1, 3, 7)


@pytest.mark.parametrize("nthreads", PIN_THREADS, ids=lambda n: f"threads{n}")
@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__[len("check_"):])
def test_pin(check, nthreads):
    with oracle.threads(nthreads):
        check()


# ============================================================================ planted mistakes
# Each entry: (name, text in farn_oracle.c, replacement[, text, replacement ...]).
# Each mutant must fail at least one pin.
MUTANTS = [
    ("drop_residual", "y32 = acc + bf16_to_float(j->residual[base + h]);", "y32 = acc;"),
    ("drop_rank_1", "for (int r = 1; r < j->R; ++r)", "for (int r = 2; r < j->R; ++r)"),
    ("double_count_rank_0", "float acc = bf16_to_float(j->partials[0][base + h]);",
     "float acc = 2.0f * bf16_to_float(j->partials[0][base + h]);"),
    ("fold_reversed", "for (int r = 1; r < j->R; ++r) acc = acc + bf16_to_float(j->partials[r][base + h]);",
     "acc = bf16_to_float(j->partials[j->R - 1][base + h]); "
     "for (int r = j->R - 2; r >= 0; --r) acc = acc + bf16_to_float(j->partials[r][base + h]);"),
    ("fold_in_double", "        float y32 = acc;\n        if (j->residual) y32 = acc + bf16_to_float(j->residual[base + h]);",
     "        double dacc = 0; for (int r = 0; r < j->R; ++r) dacc += bf16_to_float(j->partials[r][base + h]);\n"
     "        float y32 = (float)dacc;\n        if (j->residual) y32 = (float)(dacc + bf16_to_float(j->residual[base + h]));"),
    ("residual_first", "        float acc = bf16_to_float(j->partials[0][base + h]);",
     "        float acc = bf16_to_float(j->partials[0][base + h]);\n"
     "        if (j->residual) acc = bf16_to_float(j->residual[base + h]) + acc;",
     "if (j->residual) y32 = acc + bf16_to_float(j->residual[base + h]);", ""),
    ("residual_wrong_row", "j->residual[base + h]", "j->residual[h]"),
    ("mean_divisor", "ss / (double)H", "ss / (double)(H - 1)"),
    ("eps_outside_sqrt", "1.0 / sqrt(ss / (double)H + (double)j->eps)",
     "1.0 / (sqrt(ss / (double)H) + (double)j->eps)"),
    ("eps_dropped", "1.0 / sqrt(ss / (double)H + (double)j->eps)", "1.0 / sqrt(ss / (double)H)"),
    ("gamma_reversed", "bf16_to_double(j->gamma[h])", "bf16_to_double(j->gamma[H - 1 - h])"),
    ("no_gamma", "y * rstd * bf16_to_double(j->gamma[h])", "y * rstd"),
    ("scale_240", "amax / 448.0", "amax / 240.0"),
    ("quant_truncates", "double r = nearbyint(a / quantum) * quantum; /* in [0, 448] */",
     "double r = floor(a / quantum) * quantum;"),
    ("bf16_truncates", "double r = nearbyint(a / quantum) * quantum;\n    if (r >= 0x1p128)",
     "double r = trunc(a / quantum) * quantum;\n    if (r >= 0x1p128)"),
    ("bf16_mantissa_6", "double quantum = ldexp(1.0, ex - 7);", "double quantum = ldexp(1.0, ex - 6);"),
    ("e4m3_no_subnormals", "if (ex < -6) ex = -6;", "if (ex < -9) ex = -9;"),
    ("group_offset", "const int64_t h0 = g * j->group;", "const int64_t h0 = g * j->group + (g > 0);"),
    ("scale_transposed", "j->scales[t * G + g] = scale;", "j->scales[g * j->T + t] = scale;"),
    ("abs_dropped", "double v = fabs(bf16_to_double(o[h]));", "double v = bf16_to_double(o[h]);"),
    ("stats_on_gamma_scaled", "ss += y * y;", "ss += y * y * bf16_to_double(j->gamma[h]);"),
    ("reduce_alone_drops_rank_1", "for (int r = 1; r < R; ++r) acc = acc + bf16_to_float(partials[r][i]);",
     "for (int r = 2; r < R; ++r) acc = acc + bf16_to_float(partials[r][i]);"),
    ("quant_alone_scale_240", "float scale = (float)(amax / 448.0);\n            scales[t * G + g] = scale;",
     "float scale = (float)(amax / 240.0);\n            scales[t * G + g] = scale;"),
    ("quant_alone_wrong_group_base", "const uint16_t *o = x + t * H + g * group;", "const uint16_t *o = x + t * H;"),
    ("quotient_in_double", "oracle_e4m3fn_from_double((double)(bf16_to_float(o[h]) / scale))",
     "oracle_e4m3fn_from_double(bf16_to_double(o[h]) / (double)scale)",
     "oracle_e4m3fn_from_double((double)(bf16_to_float(o[h]) / scale))",
     "oracle_e4m3fn_from_double(bf16_to_double(o[h]) / (double)scale)"),
    ("mx_emax_3", "int s = (e2 - 1) - 2;", "int s = (e2 - 1) - 3;"),
    ("mx_nibbles_swapped", "(uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4))", "(uint8_t)(codes[2 * i + 1] | (codes[2 * i] << 4))"),
    ("mx_no_saturation", "if (a >= 6.0) return (uint8_t)(sign | 0x7u);", "if (a >= 1e30) return (uint8_t)(sign | 0x7u);",
     "return (uint8_t)(sign | 0x7u); /* r == 8", "return (uint8_t)(sign | 0x0u); /* r == 8"),
    ("mx_truncates", "double r = nearbyint(a / quantum) * quantum; /* ties to even multiple of the quantum */",
     "double r = floor(a / quantum) * quantum;"),
    ("mx_block_16", "const uint16_t *v = x + t * H + b * 32;", "const uint16_t *v = x + t * H + b * 16;"),
    # rounding ties away from zero instead of to even
    ("bf16_ties_away", "double r = nearbyint(a / quantum) * quantum;\n    if (r >= 0x1p128)",
     "double r = round(a / quantum) * quantum;\n    if (r >= 0x1p128)"),
    ("e4m3_ties_away", "double r = nearbyint(a / quantum) * quantum; /* in [0, 448] */",
     "double r = round(a / quantum) * quantum;"),
    ("mx_ties_away", "double r = nearbyint(a / quantum) * quantum; /* ties to even multiple of the quantum */",
     "double r = round(a / quantum) * quantum;"),
    # normalising the fp32 sum instead of the bf16 residual_out (both statistics and product)
    ("norm_on_fp32_sum",
     "/* One token row: steps 1-6 of the header, in order.",
     "static double fp32_sum(const job_t *j, int64_t i) {\n"
     "    float acc = bf16_to_float(j->partials[0][i]);\n"
     "    for (int r = 1; r < j->R; ++r) acc = acc + bf16_to_float(j->partials[r][i]);\n"
     "    if (j->residual) acc = acc + bf16_to_float(j->residual[i]);\n"
     "    return (double)acc;\n}\n/* One token row: steps 1-6 of the header, in order.",
     "double y = bf16_to_double(j->residual_out[base + h]);", "double y = fp32_sum(j, base + h);",
     "double y = bf16_to_double(j->residual_out[base + h]);", "double y = fp32_sum(j, base + h);"),
    ("group_amax_one_short", "for (int64_t h = h0; h < h0 + j->group; ++h) {\n                double v = fabs",
     "for (int64_t h = h0; h < h0 + j->group - 1; ++h) {\n                double v = fabs"),
    ("zero_group_unguarded", "if (scale == 0.0f)\n                    j->q[base + h] = 0x00u;\n                else\n",
     "if (0)\n                    j->q[base + h] = 0x00u;\n                else\n"),
    ("mx_zero_block_unguarded", "} else if (amax == 0.0) {", "} else if (amax < 0.0) {"),
    ("mx_nan_block_unguarded", "if (isnan(a)) has_nan = 1;", "if (isnan(a)) has_nan = 0;"),
    # the threaded row split: a wrong stride, a wrong first row, a thread never started
    ("thread_row_stride", "for (int64_t t = j->tid; t < j->T; t += j->nthreads)",
     "for (int64_t t = j->tid; t < j->T; t += j->nthreads + (j->tid == 0))"),
    ("thread_first_row", "for (int64_t t = j->tid; t < j->T; t += j->nthreads)",
     "for (int64_t t = j->tid + 1; t < j->T; t += j->nthreads)"),
    ("thread_last_not_started", "for (int k = 1; k < n; ++k) {\n        if (pthread_create",
     "for (int k = 1; k < n - 1; ++k) {\n        if (pthread_create"),
    # signs, special codes and the ends of each format's range
    ("bf16_sign_dropped", "const uint16_t sign = signbit(x) ? 0x8000u : 0u;", "const uint16_t sign = 0u;"),
    ("e4m3_sign_dropped", "const uint8_t sign = signbit(x) ? 0x80u : 0u;", "const uint8_t sign = 0u;"),
    ("e2m1_sign_dropped", "const uint8_t sign = signbit(x) ? 0x8u : 0u;", "const uint8_t sign = 0u;"),
    ("e4m3_nan_as_max", "if (isnan(x)) return (uint8_t)(sign | 0x7Fu);", "if (isnan(x)) return (uint8_t)(sign | 0x7Eu);"),
    ("e4m3_no_saturation", "if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);", "if (a >= 1e30) return (uint8_t)(sign | 0x7Eu);"),
    ("bf16_subnormal_quantum", "if (ex < -126) ex = -126;", "if (ex < -130) ex = -130;"),
    ("e2m1_quantum_1_above_4", "(a < 4.0 ? 1.0 : 2.0)", "(a < 4.0 ? 1.0 : 1.0)"),
    ("mx_scale_bias_126", "scales[t * B + b] = (uint8_t)(s + 127);", "scales[t * B + b] = (uint8_t)(s + 126);"),
    ("mx_scale_clamp_dropped", "if (s < -127) s = -127;", ""),
    # statistics in binary32 instead of binary64
    ("ss_in_float", "    double ss = 0.0;\n    for (int64_t h = 0; h < H; ++h) {\n        double y",
     "    float ss = 0.0f;\n    for (int64_t h = 0; h < H; ++h) {\n        float y"),
    ("rstd_in_float", "double rstd = 1.0 / sqrt(ss / (double)H + (double)j->eps);",
     "double rstd = (double)(1.0f / sqrtf((float)(ss / (double)H) + j->eps));"),
    # the quant taken of residual_out instead of the normalised out
    ("quant_of_residual_out", "double v = fabs(bf16_to_double(o[h]));",
     "double v = fabs(bf16_to_double(j->residual_out[base + h]));",
     "oracle_e4m3fn_from_double((double)(bf16_to_float(o[h]) / scale))",
     "oracle_e4m3fn_from_double((double)(bf16_to_float(j->residual_out[base + h]) / scale))"),
    # NaN and inf: a NaN ignored by the group maximum, NaN rounded to inf, inf to NaN
    ("fp8_amax_ignores_nan", "if (v > amax || isnan(v)) amax = v;\n                if (isnan(amax)) break;\n            }\n            /* amax/448",
     "if (v > amax) amax = v;\n            }\n            /* amax/448"),
    ("bf16_nan_as_inf", "if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);", "if (isnan(x)) return (uint16_t)(sign | 0x7F80u);"),
    ("bf16_inf_as_nan", "if (isinf(x)) return (uint16_t)(sign | 0x7F80u);", "if (isinf(x)) return (uint16_t)(sign | 0x7FC0u);"),
    ("quant_alone_amax_ignores_nan", "if (v > amax || isnan(v)) amax = v;\n                if (isnan(amax)) break;\n            }\n            float scale",
     "if (v > amax) amax = v;\n            }\n            float scale"),
]


@pytest.mark.slow
@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_caught(mutant, tmp_path):
    name, edits = mutant[0], mutant[1:]
    mutated = open(os.path.join(os.path.dirname(oracle.__file__), "farn_oracle.c")).read()
    for old, new in zip(edits[0::2], edits[1::2]):
        assert old in mutated, f"mutation anchor for {name} not found"
        mutated = mutated.replace(old, new, 1)
    c = tmp_path / "mut.c"
    so = tmp_path / "mut.so"
    c.write_text(mutated)
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(so), str(c), "-lm"], check=True)
    caught = []
    with oracle.using(str(so)):
        for n in PIN_THREADS:
            for check in ALL_CHECKS:
                try:
                    with oracle.threads(n):
                        check()
                except AssertionError:
                    caught.append(check.__name__)
                except Exception:  # a crash or bad status also counts as caught
                    caught.append(check.__name__ + "!")
                if caught:
                    break
            if caught:
                break
    assert caught, f"planted mistake {name} passed every pin"
