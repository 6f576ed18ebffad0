"""GPU-vs-oracle comparison at the stated tolerances, shared by the GPU tests, the
smoke check and the bench's parity gate.

Tolerances (the op's statement of parity):
  * bf16 outputs (residual_out, out): |gpu - oracle| <= 2^-7 * |oracle| + 1e-3 per element.
    residual_out is additionally expected bit-exact: both sides do the same fp32 left
    fold and the same round-to-nearest-even.
  * E4M3 codes: at most 0.1% of codes may differ, each by one code (adjacent magnitude,
    same sign).
  * fp32 scales: relative error <= 1e-3.
NaN compares equal to NaN. Signed zeros must match: a +0 against a -0 (bf16 0x0000 / 0x8000,
E4M3 code 0x00 / 0x80, E2M1 code 0x0 / 0x8) counts as a bit or code difference (numerically it
is within every tolerance).
"""

from __future__ import annotations

import numpy as np
import torch

BF16_REL = 2.0 ** -7
BF16_ABS = 1e-3
FP8_MAX_FRAC = 1e-3
SCALE_REL = 1e-3


def bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def compare_bf16(name: str, gpu_bits, ref_bits) -> dict:
    g = bits_to_f32(gpu_bits).astype(np.float64)
    r = bits_to_f32(ref_bits).astype(np.float64)
    both_nan = np.isnan(g) & np.isnan(r)
    with np.errstate(invalid="ignore"):
        err = np.where(both_nan | (g == r), 0.0, np.abs(g - r))  # g == r also covers equal infinities
    with np.errstate(invalid="ignore"):
        tol = BF16_REL * np.abs(r) + BF16_ABS
        bad = ~(err <= tol) & ~both_nan  # a NaN reference has a NaN tolerance
    ne = (gpu_bits != ref_bits) & ~both_nan
    with np.errstate(invalid="ignore"):
        rel = np.where(np.abs(r) > 0, err / np.maximum(np.abs(r), 1e-30), err)
    return {"name": name, "n": int(g.size), "n_bad": int(bad.sum()), "n_bit_diff": int(ne.sum()),
            "max_abs_err": float(err.max()) if err.size else 0.0,
            "max_rel_err": float(rel[~both_nan].max()) if err.size else 0.0,
            "first_bad": None if not bad.any() else tuple(int(i) for i in np.argwhere(bad)[0])}


def _code_rank(c: np.ndarray) -> np.ndarray:
    """E4M3 code -> signed magnitude rank, so adjacent representable values differ by 1."""
    c = c.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def compare_fp8(gpu_q, ref_q, gpu_s, ref_s) -> dict:
    gq, rq = np.asarray(gpu_q, np.uint8), np.asarray(ref_q, np.uint8)
    diff = gq != rq  # 0x00 against 0x80 counts (step 0: the same value)
    step = np.abs(_code_rank(gq) - _code_rank(rq))
    gs, rs = np.asarray(gpu_s, np.float64), np.asarray(ref_s, np.float64)
    s_nan = np.isnan(gs) & np.isnan(rs)
    s_err = np.where(s_nan, 0.0, np.abs(gs - rs) / np.where(rs != 0, np.abs(rs), 1.0))
    s_err = np.where((rs == 0) & (gs == 0), 0.0, s_err)
    return {"n": int(gq.size), "n_code_diff": int(diff.sum()),
            "frac_code_diff": float(diff.mean()) if gq.size else 0.0,
            "max_code_step": int(step.max()) if step.size else 0,
            "n_scales": int(gs.size), "max_scale_rel_err": float(s_err.max()) if s_err.size else 0.0}


def within_tolerance(rep_ro: dict, rep_out: dict | None, rep_fp8: dict | None,
                     require_ro_exact: bool = True) -> tuple[bool, str]:
    msgs = []
    if rep_ro["n_bad"]:
        msgs.append(f"residual_out: {rep_ro['n_bad']} elements beyond tolerance, first at {rep_ro['first_bad']}")
    if require_ro_exact and rep_ro["n_bit_diff"]:
        msgs.append(f"residual_out: {rep_ro['n_bit_diff']} elements not bit-exact")
    if rep_out is not None and rep_out["n_bad"]:
        msgs.append(f"out: {rep_out['n_bad']} elements beyond tolerance, first at {rep_out['first_bad']}")
    if rep_fp8 is not None:
        if rep_fp8["frac_code_diff"] > FP8_MAX_FRAC:
            msgs.append(f"q: {rep_fp8['frac_code_diff']:.2e} of codes differ (> {FP8_MAX_FRAC})")
        if rep_fp8["max_code_step"] > 1:
            msgs.append(f"q: a code differs by {rep_fp8['max_code_step']} steps")
        if rep_fp8["max_scale_rel_err"] > SCALE_REL:
            msgs.append(f"scales: rel err {rep_fp8['max_scale_rel_err']:.2e}")
    return (not msgs), "; ".join(msgs)


def compare_mxfp4(gpu_q, ref_q, gpu_s, ref_s) -> dict:
    """MXFP4 codes (two per byte) and E8M0 scale bytes. Tolerance, by the same reading as the
    E4M3 codes: at most 0.1% of codes differ, each by one step of the E2M1 grid; scale bytes
    differ on at most 0.1% of blocks, by one exponent."""
    gq, rq = np.asarray(gpu_q, np.uint8), np.asarray(ref_q, np.uint8)
    g = np.stack([gq & 0xF, gq >> 4], axis=-1).reshape(-1).astype(np.int32)
    r = np.stack([rq & 0xF, rq >> 4], axis=-1).reshape(-1).astype(np.int32)
    rank = lambda c: np.where(c & 0x8, -(c & 0x7), c & 0x7)
    diff = g != r  # 0x0 against 0x8 counts (step 0: the same value)
    step = np.abs(rank(g) - rank(r))
    gs, rs = np.asarray(gpu_s, np.int32), np.asarray(ref_s, np.int32)
    sdiff = gs != rs
    return {"n": int(g.size), "n_code_diff": int(diff.sum()), "frac_code_diff": float(diff.mean()) if g.size else 0.0,
            "max_code_step": int(step.max()) if step.size else 0, "n_scales": int(gs.size),
            "n_scale_diff": int(sdiff.sum()), "max_scale_step": int(np.abs(gs - rs).max()) if gs.size else 0}


def mxfp4_within_tolerance(rep: dict) -> tuple[bool, str]:
    msgs = []
    if rep["frac_code_diff"] > FP8_MAX_FRAC or rep["max_code_step"] > 1:
        msgs.append(f"mxfp4 codes: {rep['n_code_diff']} differ, max step {rep['max_code_step']}")
    if rep["n_scale_diff"] > FP8_MAX_FRAC * max(1, rep["n_scales"]) or rep["max_scale_step"] > 1:
        msgs.append(f"mxfp4 scales: {rep['n_scale_diff']} differ, max step {rep['max_scale_step']}")
    return (not msgs), "; ".join(msgs)
