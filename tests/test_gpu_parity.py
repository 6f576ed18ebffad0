"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element,
on the same seeded bf16 inputs, at the tolerances stated in tests/parity.py.

Every configuration is compared whole, every row and every element: the full-size prefill
chunk (R=8, T=8192, H=7168) in the launch configuration the bench times, with and without
FP8 and with MXFP4 output, and every point of the message-size sweep (R=8, H=8192,
T=2..4096). The oracle runs threaded (rows dealt to the host's cores); its threaded row
split is pinned on the CPU like the rest of it.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle
import tp_all_reduce_amd as F
from gen import CONFIGS, SWEEP_T, make_inputs, sweep_config
from parity import (bits_to_f32, compare_bf16, compare_fp8, compare_mxfp4, from_dev_bf16,
                    mxfp4_within_tolerance, to_dev_bf16, within_tolerance)

pytestmark = pytest.mark.gpu
EPS = 1e-6
VARIANTS = {"auto": F.VARIANT_AUTO, "wide": F.VARIANT_WIDE, "narrow": F.VARIANT_NARROW}
# oracle threads: the host cores this process may run on, at most 16
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    return torch.device("cuda:0")


class Uploaded:
    def __init__(self, d, dev, residual=True):
        self.d = d
        self.R, self.T, self.H = d["R"], d["T"], d["H"]
        self.P = [to_dev_bf16(d["partials"][r], dev) for r in range(self.R)]
        self.res = to_dev_bf16(d["residual"], dev) if residual else None
        self.g = to_dev_bf16(d["gamma"], dev)

    def oracle_rows(self, rows, quant, emit_out=True, residual=True):
        d = self.d
        every = len(rows) == self.T and np.array_equal(rows, np.arange(self.T))
        P = d["partials"] if every else d["partials"][:, rows, :]
        res = (d["residual"] if every else d["residual"][rows]) if (residual and self.res is not None) else None
        if quant:
            return oracle.reduce_add_rmsnorm_quant_group(P, res, d["gamma"], EPS, 128, emit_out,
                                                         nthreads=ORACLE_THREADS)
        return oracle.reduce_add_rmsnorm(P, res, d["gamma"], EPS, nthreads=ORACLE_THREADS)


def run_and_compare(u: Uploaded, quant: bool, variant: str = "auto",
                    emit_out: bool = True, rows=None, label: str = "", ref=None):
    say(f"[gpu] {label} R={u.R} T={u.T} H={u.H} quant={quant} variant={variant} "
        f"emit={emit_out} residual={u.res is not None}")
    if quant:
        ro, out, q, sc = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS, emit_out=emit_out,
                                                          variant=VARIANTS[variant])
    else:
        ro, out = F.reduce_add_rmsnorm(u.P, u.res, u.g, EPS, variant=VARIANTS[variant])
    torch.cuda.synchronize()
    rows = np.arange(u.T) if rows is None else np.asarray(rows)
    g_ro = from_dev_bf16(ro)[rows]
    g_out = from_dev_bf16(out)[rows] if out is not None else None
    if ref is None:
        ref = u.oracle_rows(rows, quant, emit_out)
    rep_ro = compare_bf16("residual_out", g_ro, ref[0])
    rep_out = compare_bf16("out", g_out, ref[1]) if g_out is not None else None
    rep_fp8 = None
    if quant:
        rep_fp8 = compare_fp8(q.cpu().numpy()[rows], ref[2], sc.cpu().numpy()[rows], ref[3])
    ok, why = within_tolerance(rep_ro, rep_out, rep_fp8)
    assert ok, f"{label}: {why} | {rep_ro} {rep_out} {rep_fp8}"
    return rep_ro, rep_out, rep_fp8


# ------------------------------------------------------------------ the configurations
SMALL = ["tiny", "decode_ds", "decode_fp8"]


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", SMALL)
def test_configs_small(dev, name, variant):
    cfg = CONFIGS[name]
    u = Uploaded(make_inputs(cfg), dev)
    for quant in cfg.quant:
        run_and_compare(u, quant, variant, label=name)
    if cfg.H % 128 == 0 and True not in cfg.quant:
        run_and_compare(u, True, variant, label=name + "+fp8")


@pytest.fixture(scope="module")
def prefill(dev):
    say("[gpu] generating prefill chunk R=8 T=8192 H=7168")
    u = Uploaded(make_inputs(CONFIGS["prefill"]), dev)
    u.refs = {}  # the oracle's outputs over every row, per call kind, computed once
    return u


def _prefill_ref(u, kind):
    if kind not in u.refs:
        say(f"[gpu] oracle over all {u.T} rows ({kind}, {ORACLE_THREADS} threads)")
        d = u.d
        if kind == "mxfp4":
            u.refs[kind] = oracle.reduce_add_rmsnorm_mxfp4(d["partials"], d["residual"], d["gamma"], EPS,
                                                           nthreads=ORACLE_THREADS)
        else:
            u.refs[kind] = u.oracle_rows(np.arange(u.T), kind == "fp8")
    return u.refs[kind]


@pytest.mark.parametrize("quant", [False, True])
@pytest.mark.parametrize("variant", ["auto", "wide", "narrow"])
def test_prefill_full_size_all_rows(prefill, quant, variant):
    rep = run_and_compare(prefill, quant, variant, label="prefill, every row",
                          ref=_prefill_ref(prefill, "fp8" if quant else "plain"))
    say(f"[gpu]   {rep}")


def test_prefill_full_size_properties(prefill):
    """Whole-tensor checks at full size: the wide and narrow launch shapes agree bit for
    bit on every row (their fp64 sums of squares differ only in addition order), and every
    output is finite."""
    say("[gpu] prefill whole-tensor variant identity")
    a = F.reduce_add_rmsnorm_quant_group(prefill.P, prefill.res, prefill.g, EPS, variant=F.VARIANT_WIDE)
    b = F.reduce_add_rmsnorm_quant_group(prefill.P, prefill.res, prefill.g, EPS, variant=F.VARIANT_NARROW)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    assert torch.isfinite(a[0].float()).all() and torch.isfinite(a[1].float()).all()
    assert torch.isfinite(a[3]).all() and (a[3] > 0).all()
    assert ((a[2] & 0x7F) == 0x7E).view(prefill.T, -1, 128).any(dim=2).all()  # a 448 code per group


@pytest.mark.parametrize("R,H", [(6, 7168), (4, 6656), (7, 8192), (8, 6656)])
def test_two_workgroups_per_cu_launch(dev, R, H):
    """The plain call's narrow shape at H = 6152..8192 with R = 4..7 from T = 2048 is launched
    with LDS reserved so that at most two workgroups share a compute unit (with R = 8 its
    registers already allow no more): its outputs match the oracle on every row, and the wide
    shape (launched without the reservation) bit for bit on every row."""
    T = 2048
    u = Uploaded(make_inputs(CONFIGS["prefill"], seed=40 + R, R=R, T=T, H=H), dev)
    assert F.select_variant(R, T, H, False) == F.VARIANT_NARROW
    run_and_compare(u, False, "auto", label="two-per-CU")
    a = F.reduce_add_rmsnorm(u.P, u.res, u.g, EPS, variant=F.VARIANT_NARROW)
    b = F.reduce_add_rmsnorm(u.P, u.res, u.g, EPS, variant=F.VARIANT_WIDE)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("T", list(SWEEP_T))
def test_sweep_points(dev, T):
    """Every row of every message-size sweep point, in every launch shape."""
    cfg = sweep_config(T)
    u = Uploaded(make_inputs(cfg), dev)
    ref = u.oracle_rows(np.arange(T), False)
    for variant in VARIANTS:
        run_and_compare(u, False, variant, label=cfg.name, ref=ref)


# ------------------------------------------------------------------ edge shapes
@pytest.mark.parametrize("T", [1, 5, 80, 81])
def test_edge_T(dev, T):
    u = Uploaded(make_inputs(CONFIGS["decode_ds"], seed=100 + T, T=T), dev)
    for variant in VARIANTS:
        run_and_compare(u, False, variant, label=f"T{T}")
        run_and_compare(u, True, variant, label=f"T{T}")


@pytest.mark.parametrize("H", [8, 16, 64, 264, 512, 1024, 2048, 4096, 7168, 8192, 8200, 16384, 24576, 32768])
def test_edge_H(dev, H):
    u = Uploaded(make_inputs(CONFIGS["tiny"], seed=H, R=3, T=6, H=H), dev)
    for variant in VARIANTS:
        run_and_compare(u, False, variant, label=f"H{H}")
        if H % 128 == 0:
            run_and_compare(u, True, variant, label=f"H{H}")


@pytest.mark.parametrize("R", list(range(1, 9)))
def test_edge_R(dev, R):
    u = Uploaded(make_inputs(CONFIGS["tiny"], seed=R, R=R, T=7, H=1024), dev)
    for variant in ("wide", "narrow"):
        run_and_compare(u, False, variant, label=f"R{R}")
        run_and_compare(u, True, variant, label=f"R{R}")


def test_no_residual(dev):
    d = make_inputs(CONFIGS["decode_fp8"], seed=7)
    u = Uploaded(d, dev, residual=False)
    for variant in VARIANTS:
        run_and_compare(u, False, variant, label="nores")
        run_and_compare(u, True, variant, label="nores")
    # R=1 without residual: residual_out is P_0 bit for bit
    u1 = Uploaded(make_inputs(CONFIGS["tiny"], seed=8, R=1, T=9, H=2048), dev, residual=False)
    ro, _ = F.reduce_add_rmsnorm(u1.P, None, u1.g, EPS)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(ro), u1.d["partials"][0])


def test_quant_without_bf16_out(dev):
    u = Uploaded(make_inputs(CONFIGS["decode_fp8"], seed=9), dev)
    for variant in VARIANTS:
        run_and_compare(u, True, variant, emit_out=False, label="no-out")


@pytest.mark.parametrize("T,H", [(33, 7168), (600, 7168), (9, 20480)])
def test_in_place_residual(dev, T, H):
    """residual_out written over the residual: decode and many rows, two and four vector slots."""
    d = make_inputs(CONFIGS["decode_ds"], seed=10, T=T, H=H)
    ref_ro, ref_out = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], EPS, nthreads=8)
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        say(f"[gpu] in-place residual variant={variant}")
        u = Uploaded(d, dev)
        ro, out = F.reduce_add_rmsnorm(u.P, u.res, u.g, EPS, residual_out=u.res, variant=variant)
        torch.cuda.synchronize()
        assert ro.data_ptr() == u.res.data_ptr()
        assert np.array_equal(from_dev_bf16(ro), ref_ro)
        ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro), ref_ro),
                                   compare_bf16("out", from_dev_bf16(out), ref_out), None)
        assert ok, why


@pytest.mark.parametrize("T,H", [(21, 7168), (600, 7168), (9, 20480)])
def test_in_place_residual_quant(dev, T, H):
    """In place with the FP8 and MXFP4 calls too (their kernels store residual_out at a
    different point of the row than the plain two-slot kernel): the small-call schedule, the
    streaming one (each slot's residual_out stored right after its fold, T = 600) and four
    vector slots per lane."""
    d = make_inputs(CONFIGS["decode_ds"], seed=11, T=T, H=H)
    ref = oracle.reduce_add_rmsnorm_quant_group(d["partials"], d["residual"], d["gamma"], EPS, nthreads=8)
    ref_mx = oracle.reduce_add_rmsnorm_mxfp4(d["partials"], d["residual"], d["gamma"], EPS, nthreads=8)
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        say(f"[gpu] in-place residual, FP8 and MXFP4, variant={variant}")
        u = Uploaded(d, dev)
        ro, out, q, sc = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS, residual_out=u.res, variant=variant)
        torch.cuda.synchronize()
        assert ro.data_ptr() == u.res.data_ptr() and np.array_equal(from_dev_bf16(ro), ref[0])
        ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro), ref[0]),
                                   compare_bf16("out", from_dev_bf16(out), ref[1]),
                                   compare_fp8(q.cpu().numpy(), ref[2], sc.cpu().numpy(), ref[3]))
        assert ok, why
        u = Uploaded(d, dev)
        ro, out, q, sc = F.reduce_add_rmsnorm_mxfp4(u.P, u.res, u.g, EPS, residual_out=u.res, variant=variant)
        torch.cuda.synchronize()
        assert ro.data_ptr() == u.res.data_ptr() and np.array_equal(from_dev_bf16(ro), ref_mx[0])
        ok, why = mxfp4_within_tolerance(compare_mxfp4(q.cpu().numpy(), ref_mx[2], sc.cpu().numpy(), ref_mx[3]))
        assert ok, why


def test_empty_T(dev):
    say("[gpu] T = 0")
    p = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    g = torch.ones(256, dtype=torch.bfloat16, device=dev)
    ro, out = F.reduce_add_rmsnorm([p, p], p, g, EPS)
    ro, out, q, s = F.reduce_add_rmsnorm_quant_group([p], None, g, EPS)
    torch.cuda.synchronize()
    assert ro.numel() == 0 and q.numel() == 0


# ------------------------------------------------------------------ state, order, determinism
def test_back_to_back_calls_do_not_leak(dev):
    """Alternate two shapes on one stream without synchronising and check every result."""
    say("[gpu] back-to-back alternating calls")
    ua = Uploaded(make_inputs(CONFIGS["decode_ds"], seed=30), dev)
    ub = Uploaded(make_inputs(CONFIGS["decode_fp8"], seed=31), dev)
    outs = []
    for i in range(6):
        if i % 2 == 0:
            outs.append(("a", F.reduce_add_rmsnorm(ua.P, ua.res, ua.g, EPS, variant=i % 3)))
        else:
            outs.append(("b", F.reduce_add_rmsnorm_quant_group(ub.P, ub.res, ub.g, EPS, variant=i % 3)))
    torch.cuda.synchronize()
    ref_a = ua.oracle_rows(np.arange(ua.T), False)
    ref_b = ub.oracle_rows(np.arange(ub.T), True)
    for tag, res in outs:
        if tag == "a":
            ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(res[0]), ref_a[0]),
                                       compare_bf16("out", from_dev_bf16(res[1]), ref_a[1]), None)
        else:
            ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(res[0]), ref_b[0]),
                                       compare_bf16("out", from_dev_bf16(res[1]), ref_b[1]),
                                       compare_fp8(res[2].cpu().numpy(), ref_b[2], res[3].cpu().numpy(), ref_b[3]))
        assert ok, why


def test_deterministic_and_variants_identical(dev):
    u = Uploaded(make_inputs(CONFIGS["decode_ds"], seed=40, T=200), dev)
    say("[gpu] determinism")
    runs = [F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS, variant=v) for v in (1, 1, 2, 2, 0)]
    torch.cuda.synchronize()
    for other in runs[1:]:
        for x, y in zip(runs[0], other):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


# ------------------------------------------------------------------ special values
def test_subnormal_and_tiny_values(dev):
    """Sums in the bf16 subnormal range: residual_out must round exactly like the oracle
    (no flush to zero)."""
    d = make_inputs(CONFIGS["tiny"], seed=50, R=4, T=4, H=512)
    P = d["partials"].astype(np.uint32)
    # move every exponent down so that values sit around 2^-128 .. 2^-120
    exp = (P >> 7) & 0xFF
    newexp = np.clip(exp.astype(np.int32) - 122, 0, 255).astype(np.uint32)
    P = np.where(exp > 0, (P & 0x807F) | (newexp << 7), P).astype(np.uint16)
    d["partials"] = P
    d["residual"] = np.zeros_like(d["residual"])
    u = Uploaded(d, dev)
    for variant in ("wide", "narrow"):
        run_and_compare(u, False, variant, label="subnormal")
        run_and_compare(u, True, variant, label="subnormal")


def _with_group_exponents(x, exps, rng):
    """bf16 array x [.., H]: channel group g (128 channels) gets biased exponent exps[g]
    (0 = subnormal, with a nonzero mantissa), random sign and mantissa."""
    x = x.astype(np.uint32).copy()
    for gi, e in enumerate(exps):
        sl = (..., slice(gi * 128, (gi + 1) * 128))
        mant = rng.integers(1 if e == 0 else 0, 128, size=x[sl].shape, dtype=np.uint32)
        sign = rng.integers(0, 2, size=x[sl].shape, dtype=np.uint32) << 15
        x[sl] = sign | (np.uint32(e) << 7) | mant
    return x.astype(np.uint16)


# per-group exponents of gamma (or x): a normal group; groups whose scale lands on either
# side of 2^-64; groups whose scale is an fp32 subnormal (1/scale overflows fp32); bf16
# subnormal values
TINY_GROUP_EXPONENTS = [127, 70, 69, 27, 4, 1, 0, 0]


def test_tiny_scale_groups(dev):
    """FP8 groups whose amax lies far below the fp32 normal range: codes and scales must be
    bit-exact with the oracle (the quotient, 1/scale and the rounding remainder must not
    overflow or underflow), in the fused call and in the quant alone."""
    rng = np.random.default_rng(71)
    d = make_inputs(CONFIGS["tiny"], seed=71, R=2, T=8, H=1024)
    d["gamma"] = _with_group_exponents(d["gamma"][None, :], TINY_GROUP_EXPONENTS, rng)[0]
    u = Uploaded(d, dev)
    for variant in ("wide", "narrow"):
        _, _, rep = run_and_compare(u, True, variant, label="tiny-scale groups")
        assert rep["n_code_diff"] == 0 and rep["max_scale_rel_err"] == 0.0, rep
    x = _with_group_exponents(make_inputs(CONFIGS["tiny"], seed=72, R=1, T=16, H=1024)["residual"],
                              TINY_GROUP_EXPONENTS, rng)
    say("[gpu] quant alone, tiny-scale groups T=16 H=1024")
    q, sc = F.quant_group(to_dev_bf16(x, dev))
    torch.cuda.synchronize()
    rq, rs = oracle.quant_group(x)
    rep = compare_fp8(q.cpu().numpy(), rq, sc.cpu().numpy(), rs)
    assert rep["n_code_diff"] == 0 and rep["max_scale_rel_err"] == 0.0, rep


def test_nan_row(dev):
    d = make_inputs(CONFIGS["tiny"], seed=60, R=2, T=4, H=256)
    d["partials"][1, 2, 5] = 0x7FC0
    u = Uploaded(d, dev)
    say("[gpu] NaN row")
    ro, out, q, s = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS)
    torch.cuda.synchronize()
    rof = ro.float().cpu().numpy()
    outf = out.float().cpu().numpy()
    assert np.isnan(rof[2, 5]) and np.isfinite(np.delete(rof[2], 5)).all()
    assert np.isnan(outf[2]).all() and np.isfinite(outf[[0, 1, 3]]).all()
    qq = q.cpu().numpy()
    assert ((qq[2] & 0x7F) == 0x7F).all() and np.isnan(s.cpu().numpy()[2]).all()
    ref = u.oracle_rows(np.array([0, 1, 3]), True)
    ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro)[[0, 1, 3]], ref[0]),
                               compare_bf16("out", from_dev_bf16(out)[[0, 1, 3]], ref[1]),
                               compare_fp8(qq[[0, 1, 3]], ref[2], s.cpu().numpy()[[0, 1, 3]], ref[3]))
    assert ok, why


def test_signed_zeros_bit_exact(dev):
    """Elements whose sum is -0 (every partial and the residual -0) give residual_out = out =
    -0 and the -0 codes (E4M3 0x80, E2M1 0x8), as the oracle's division and encoders give;
    tiny negative values beside a large group maximum round to the -0 code too. Every output
    must equal the oracle bit for bit, in both launch shapes."""
    d = make_inputs(CONFIGS["tiny"], seed=61, R=3, T=5, H=1024)
    P, res = d["partials"], d["residual"]
    for t in range(5):
        cols = np.arange(t, 1024, 7 + t)
        P[:, t, cols] = 0x8000
        res[t, cols] = 0x8000
    # row 4: one large value per group, the rest tiny negatives (quotients far below 2^-10)
    P[:, 4, :] = 0x8000
    res[4, :] = 0xB000            # -4.7e-10
    res[4, ::128] = 0x4300        # 128.0
    u = Uploaded(d, dev)
    ref = u.oracle_rows(np.arange(5), True)
    ref_mx = oracle.reduce_add_rmsnorm_mxfp4(P, res, d["gamma"], EPS, nthreads=4)
    assert (ref[1] == 0x8000).sum() >= 400 and (ref[2][4] == 0x80).sum() >= 1000
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        say(f"[gpu] signed zeros, variant={variant}")
        ro, out, q, sc = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS, variant=variant)
        mro, mout, mq, msc = F.reduce_add_rmsnorm_mxfp4(u.P, u.res, u.g, EPS, variant=variant)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_bf16(ro), ref[0]) and np.array_equal(from_dev_bf16(out), ref[1])
        assert np.array_equal(q.cpu().numpy(), ref[2]), "E4M3 codes differ (signed zeros included)"
        assert np.array_equal(sc.cpu().numpy(), ref[3])
        assert np.array_equal(from_dev_bf16(mout), ref_mx[1])
        assert np.array_equal(mq.cpu().numpy(), ref_mx[2]), "E2M1 codes differ (signed zeros included)"
        assert np.array_equal(msc.cpu().numpy(), ref_mx[3])


# ------------------------------------------------------------------ graph capture
@pytest.mark.parametrize("R,T,H", [(1, 5, 1024), (3, 5, 1024), (3, 520, 1024), (2, 3, 20480)])
def test_signed_zeros_no_residual(dev, R, T, H):
    """With no residual, elements whose partials are all -0 sum to -0 (nothing is added to them:
    a +0 would turn the sum into +0), so residual_out, out and the codes are the -0 ones, bit for
    bit as the oracle gives. The shapes reach every form of the kernels' fold: both launch
    shapes, the FP8 / MXFP4 small-call schedule (T <= 512) and streaming schedule (T = 520),
    four vectors per lane (H = 20480), and the standalone all-reduce."""
    d = make_inputs(CONFIGS["tiny"], seed=62, R=R, T=T, H=H)
    P = d["partials"]
    for t in range(T):
        P[:, t, np.arange(t % 7, H, 5 + t % 7)] = 0x8000
    u = Uploaded(d, dev, residual=False)
    rows = np.arange(T)
    ref_q = u.oracle_rows(rows, True)
    ref_p = u.oracle_rows(rows, False)
    ref_mx = oracle.reduce_add_rmsnorm_mxfp4(P, None, d["gamma"], EPS, nthreads=ORACLE_THREADS)
    assert (ref_p[0] == 0x8000).sum() >= T * H // 12 and (ref_p[1] == 0x8000).sum() >= T * H // 12
    assert (ref_q[2] == 0x80).sum() >= T * H // 12
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        say(f"[gpu] signed zeros without residual, R={R} T={T} H={H} variant={variant}")
        ro, out = F.reduce_add_rmsnorm(u.P, None, u.g, EPS, variant=variant)
        qro, qout, q, sc = F.reduce_add_rmsnorm_quant_group(u.P, None, u.g, EPS, variant=variant)
        mro, mout, mq, msc = F.reduce_add_rmsnorm_mxfp4(u.P, None, u.g, EPS, variant=variant)
        torch.cuda.synchronize()
        for name, got, want in (("residual_out", ro, ref_p[0]), ("out", out, ref_p[1]),
                                ("FP8 residual_out", qro, ref_q[0]), ("FP8 out", qout, ref_q[1]),
                                ("MXFP4 residual_out", mro, ref_mx[0]), ("MXFP4 out", mout, ref_mx[1])):
            assert np.array_equal(from_dev_bf16(got), want), f"{name} differs, variant {variant}"
        assert np.array_equal(q.cpu().numpy(), ref_q[2]) and np.array_equal(sc.cpu().numpy(), ref_q[3])
        assert np.array_equal(mq.cpu().numpy(), ref_mx[2]) and np.array_equal(msc.cpu().numpy(), ref_mx[3])
    red = F.reduce(u.P)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(red), oracle.reduce(P)), "all-reduce differs"


def _bf16_of(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _extreme_inputs():
    """Rows of ordinary, huge (2^60), tiny (2^-100), zero and subnormal (2^-131) magnitude, and a
    gamma holding zeros of both signs, negatives, subnormals, the largest finite values, infinities,
    a NaN, and blocks of tiny (2^-100) and huge (2^100) values."""
    R, T, H = 2, 6, 1024
    rng = np.random.default_rng(71)
    scale = np.array([1.0, 2.0 ** 60, 2.0 ** -100, 1.0, 0.0, 2.0 ** -131], np.float32)
    P = _bf16_of(rng.standard_normal((R, T, H)).astype(np.float32) * scale[None, :, None])
    g = _bf16_of(rng.uniform(0.5, 1.5, H).astype(np.float32))
    for i, v in enumerate([0x0000, 0x8000, 0xBF80, 0x0001, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0,
                           0x0010, 0x1F80, 0x6F80]):
        g[i * 7] = v
    g[700:760] = _bf16_of(np.float32(2.0 ** -100) * rng.uniform(1, 2, 60).astype(np.float32))
    g[800:860] = _bf16_of(np.float32(2.0 ** 100) * rng.uniform(1, 2, 60).astype(np.float32))
    return P, g


def _same_codes(gq, rq, gs, rs, nan_code):
    """Codes and scales equal bit for bit, NaN codes and NaN scales compared as NaN."""
    gq, rq = np.asarray(gq), np.asarray(rq)
    nr, ng = nan_code(rq), nan_code(gq)
    assert np.array_equal(nr, ng) and np.array_equal(gq[~nr], rq[~nr]), "codes differ"
    gs, rs = np.asarray(gs), np.asarray(rs)
    if gs.dtype == np.float32:
        assert np.array_equal(np.isnan(gs), np.isnan(rs))
        assert np.array_equal(gs[~np.isnan(rs)].view(np.uint32), rs[~np.isnan(rs)].view(np.uint32)), "scales differ"
    else:
        assert np.array_equal(gs, rs), "scale bytes differ"


@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_gamma_and_rstd_extremes(dev, eps):
    """Where the normalisation's fp32 fast path cannot be trusted it must hand over to fp64: y*gamma
    overflowing fp32 while the output is finite (rows of 2^60 with huge gamma), y*gamma subnormal
    or underflowing to zero while the output is not (tiny rows and gamma), an fp32 rstd that is
    infinite or above the fp32 range (eps = 0 with a zero or subnormal row), zero, negative,
    infinite and NaN gamma. Every output equals the oracle bit for bit (NaN as NaN), plain, FP8
    and MXFP4, in both launch shapes."""
    P, g = _extreme_inputs()
    R, T, H = P.shape
    ref_p = oracle.reduce_add_rmsnorm(P, None, g, eps, nthreads=ORACLE_THREADS)
    ref_q = oracle.reduce_add_rmsnorm_quant_group(P, None, g, eps, 128, True, nthreads=ORACLE_THREADS)
    ref_m = oracle.reduce_add_rmsnorm_mxfp4(P, None, g, eps, nthreads=ORACLE_THREADS)
    # the hazards are present: overflowing and underflowing fp32 products with finite, nonzero outputs
    y, gf = bits_to_f32(ref_p[0]), bits_to_f32(g)
    outf = bits_to_f32(ref_p[1])
    with np.errstate(all="ignore"):
        yg = y * gf[None, :]
    over = np.isinf(yg) & np.isfinite(y) & np.isfinite(gf)[None, :]
    under = (np.abs(yg) < 2.0 ** -126) & (y != 0) & (gf != 0)[None, :]
    assert np.isfinite(outf[over]).sum() >= 32 and (outf[under] != 0).sum() >= 500
    Pd = [to_dev_bf16(P[r], dev) for r in range(R)]
    gd = to_dev_bf16(g, dev)
    fp8_nan = lambda c: (c & 0x7F) == 0x7F
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        say(f"[gpu] gamma and rstd extremes, eps={eps} variant={variant}")
        ro, out = F.reduce_add_rmsnorm(Pd, None, gd, eps, variant=variant)
        qro, qout, q, sc = F.reduce_add_rmsnorm_quant_group(Pd, None, gd, eps, variant=variant)
        mro, mout, mq, msc = F.reduce_add_rmsnorm_mxfp4(Pd, None, gd, eps, variant=variant)
        torch.cuda.synchronize()
        for name, got, want in (("residual_out", ro, ref_p[0]), ("out", out, ref_p[1]),
                                ("FP8 out", qout, ref_q[1]), ("MXFP4 out", mout, ref_m[1])):
            rep = compare_bf16(name, from_dev_bf16(got), want)
            assert rep["n_bit_diff"] == 0, rep
        _same_codes(q.cpu().numpy(), ref_q[2], sc.cpu().numpy(), ref_q[3], fp8_nan)
        _same_codes(mq.cpu().numpy(), ref_m[2], msc.cpu().numpy(), ref_m[3], lambda c: np.zeros(c.shape, bool))


@pytest.mark.parametrize("eps", [1.0, 1e30, float(np.finfo(np.float32).max)])
def test_large_eps_and_aliased_partials(dev, eps):
    """Any finite eps >= 0 is accepted: with eps = 1, 1e30 and the largest binary32 value rstd
    falls to 1e-15 .. 5e-20 (the outputs tiny, FP8 scales below 2^-64 at the largest), and the
    partials are four pointers to two buffers (aliasing each other, as the calls allow). Every
    output equals the oracle's bit for bit, plain, FP8 and MXFP4, in both launch shapes."""
    d = make_inputs(CONFIGS["decode_fp8"], seed=91, R=2, T=33, H=4096)
    P = np.stack([d["partials"][0], d["partials"][1], d["partials"][0], d["partials"][1]])
    res, g = d["residual"], d["gamma"]
    ref_p = oracle.reduce_add_rmsnorm(P, res, g, eps, nthreads=ORACLE_THREADS)
    ref_q = oracle.reduce_add_rmsnorm_quant_group(P, res, g, eps, 128, True, nthreads=ORACLE_THREADS)
    ref_m = oracle.reduce_add_rmsnorm_mxfp4(P, res, g, eps, nthreads=ORACLE_THREADS)
    if eps > 1e38:
        assert (ref_q[3] < 2.0 ** -64).all() and (ref_q[3] > 0).all()
    p0, p1 = to_dev_bf16(d["partials"][0], dev), to_dev_bf16(d["partials"][1], dev)
    Pd = [p0, p1, p0, p1]
    rd, gd = to_dev_bf16(res, dev), to_dev_bf16(g, dev)
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        say(f"[gpu] eps={eps} aliased partials variant={variant}")
        ro, out = F.reduce_add_rmsnorm(Pd, rd, gd, eps, variant=variant)
        qro, qout, q, sc = F.reduce_add_rmsnorm_quant_group(Pd, rd, gd, eps, variant=variant)
        mro, mout, mq, msc = F.reduce_add_rmsnorm_mxfp4(Pd, rd, gd, eps, variant=variant)
        torch.cuda.synchronize()
        for name, got, want in (("residual_out", ro, ref_p[0]), ("out", out, ref_p[1]),
                                ("FP8 out", qout, ref_q[1]), ("MXFP4 out", mout, ref_m[1])):
            rep = compare_bf16(name, from_dev_bf16(got), want)
            assert rep["n_bit_diff"] == 0, rep
        assert np.array_equal(q.cpu().numpy(), ref_q[2]) and np.array_equal(sc.cpu().numpy(), ref_q[3])
        assert np.array_equal(mq.cpu().numpy(), ref_m[2]) and np.array_equal(msc.cpu().numpy(), ref_m[3])


# Rows whose rstd lies within 1.2e-9 (relative) above the bf16 midpoint 1 + 2^-8: the pattern
# y = [1, c x 7] (c = 0.9375) repeated along H, gamma = 1, eps the binary32 value 0x3DC917E0, so
# the mean of squares is the same at every H; the exact result of each 1 is 1 + 2^-7 (0x3F81),
# and an rstd rounded to binary32 gives 1 (0x3F80). The same row pins the oracle.
NEAR_MID_EPS = float(np.array([0x3DC917E0], np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("R,T,H", [(1, 3, 8), (8, 40, 128), (2, 70, 7168), (8, 9, 20480)])
def test_rstd_near_bf16_midpoint(dev, R, T, H):
    """The fp32 normalisation fast path must hand an element whose product lies this close to a
    bf16 midpoint over to fp64, and the row's rstd must resolve it: every output equals the
    oracle's bit for bit (plain, FP8 and MXFP4 where H allows), in both launch shapes."""
    y = np.tile(np.array([0x3F80] + [0x3F70] * 7, np.uint16), (T, H // 8))
    P = np.zeros((R, T, H), np.uint16)
    P[0] = y
    g = np.full(H, 0x3F80, np.uint16)
    eps = NEAR_MID_EPS
    ref_p = oracle.reduce_add_rmsnorm(P, None, g, eps, nthreads=ORACLE_THREADS)
    assert (ref_p[1][:, 0::8] == 0x3F81).all()
    ref_q = oracle.reduce_add_rmsnorm_quant_group(P, None, g, eps, 128, True, nthreads=ORACLE_THREADS) \
        if H % 128 == 0 else None
    ref_m = oracle.reduce_add_rmsnorm_mxfp4(P, None, g, eps, nthreads=ORACLE_THREADS) if H % 32 == 0 else None
    Pd = [to_dev_bf16(P[r], dev) for r in range(R)]
    gd = to_dev_bf16(g, dev)
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        say(f"[gpu] rstd near a bf16 midpoint R={R} T={T} H={H} variant={variant}")
        ro, out = F.reduce_add_rmsnorm(Pd, None, gd, eps, variant=variant)
        torch.cuda.synchronize()
        for name, got, want in (("residual_out", ro, ref_p[0]), ("out", out, ref_p[1])):
            rep = compare_bf16(name, from_dev_bf16(got), want)
            assert rep["n_bit_diff"] == 0, rep
        if ref_q is not None:
            qro, qout, q, sc = F.reduce_add_rmsnorm_quant_group(Pd, None, gd, eps, variant=variant)
            torch.cuda.synchronize()
            assert compare_bf16("FP8 out", from_dev_bf16(qout), ref_q[1])["n_bit_diff"] == 0
            assert np.array_equal(q.cpu().numpy(), ref_q[2]) and np.array_equal(sc.cpu().numpy(), ref_q[3])
        if ref_m is not None:
            mro, mout, mq, msc = F.reduce_add_rmsnorm_mxfp4(Pd, None, gd, eps, variant=variant)
            torch.cuda.synchronize()
            assert compare_bf16("MXFP4 out", from_dev_bf16(mout), ref_m[1])["n_bit_diff"] == 0
            assert np.array_equal(mq.cpu().numpy(), ref_m[2]) and np.array_equal(msc.cpu().numpy(), ref_m[3])


def test_graph_capture_replays_match_eager(dev):
    """The calls allocate nothing and never synchronise, so a serving loop can capture them in a
    HIP graph. Replay several times with the program's own eager work and synchronisations
    between the replays; every replay must equal the eager result bit for bit."""
    say("[gpu] graph capture")
    ua = Uploaded(make_inputs(CONFIGS["decode_ds"], seed=70), dev)
    ub = Uploaded(make_inputs(CONFIGS["decode_fp8"], seed=71), dev)
    # a plain call large enough to take the launch with LDS reserved (two workgroups per CU)
    uc = Uploaded(make_inputs(CONFIGS["prefill"], seed=72, R=6, T=2048, H=6152), dev)
    ea = F.reduce_add_rmsnorm(ua.P, ua.res, ua.g, EPS)
    eb = F.reduce_add_rmsnorm_quant_group(ub.P, ub.res, ub.g, EPS)
    ec = F.reduce_add_rmsnorm(uc.P, uc.res, uc.g, EPS)
    torch.cuda.synchronize()
    # the eager results themselves against the oracle
    ra, rb = ua.oracle_rows(np.arange(ua.T), False), ub.oracle_rows(np.arange(ub.T), True)
    rows_c = np.arange(uc.T)
    rc = uc.oracle_rows(rows_c, False)
    for (ro, out), r, rows in ((ea, ra, slice(None)), (eb[:2], rb, slice(None)), (ec, rc, rows_c)):
        ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro)[rows], r[0]),
                                   compare_bf16("out", from_dev_bf16(out)[rows], r[1]),
                                   compare_fp8(eb[2].cpu().numpy(), rb[2], eb[3].cpu().numpy(), rb[3]) if r is rb else None)
        assert ok, why
    ga = (torch.empty_like(ea[0]), torch.empty_like(ea[1]))
    gb = tuple(torch.empty_like(x) for x in eb)
    gc = (torch.empty_like(ec[0]), torch.empty_like(ec[1]))
    # warm up on a side stream, as graph capture requires
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        F.reduce_add_rmsnorm(ua.P, ua.res, ua.g, EPS, residual_out=ga[0], out=ga[1])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        F.reduce_add_rmsnorm(ua.P, ua.res, ua.g, EPS, residual_out=ga[0], out=ga[1])
        F.reduce_add_rmsnorm_quant_group(ub.P, ub.res, ub.g, EPS, residual_out=gb[0], out=gb[1],
                                         q=gb[2], scales=gb[3])
        F.reduce_add_rmsnorm(uc.P, uc.res, uc.g, EPS, residual_out=gc[0], out=gc[1])
    for rep in range(4):
        for t in ga + gb + gc:
            t.view(torch.uint8).fill_(0xA5)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(ea + eb + ec, ga + gb + gc):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"replay {rep}"


# ------------------------------------------------------------------ unfused building blocks
@pytest.mark.parametrize("name", ["decode_ds", "decode_fp8", "tiny"])
def test_unfused_blocks_and_compositions(dev, name):
    """The all-reduce alone and the quant alone match their oracle blocks bit for bit; the
    2-kernel composition (fused AR+RMSNorm, then quant) equals the fused FP8 call; the 3-kernel
    composition (AR, then add+RMSNorm with the AR output as one partial, then quant) matches the
    oracle's composition of the same blocks."""
    cfg = CONFIGS[name]
    d = make_inputs(cfg, seed=80)
    u = Uploaded(d, dev)
    say(f"[gpu] unfused blocks {name}")
    ar = F.reduce(u.P)
    torch.cuda.synchronize()
    ref_ar = oracle.reduce(d["partials"])
    assert np.array_equal(from_dev_bf16(ar), ref_ar)
    if cfg.H % 128:
        return
    # 2-kernel: fused plain call, then quant alone
    ro2, out2 = F.reduce_add_rmsnorm(u.P, u.res, u.g, EPS)
    q2, s2 = F.quant_group(out2)
    fused = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS)
    torch.cuda.synchronize()
    for x, y in zip((ro2, out2, q2, s2), fused):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    rq, rs = oracle.quant_group(from_dev_bf16(out2))
    ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro2), from_dev_bf16(ro2)), None,
                               compare_fp8(q2.cpu().numpy(), rq, s2.cpu().numpy(), rs))
    assert ok and np.array_equal(q2.cpu().numpy(), rq), why
    # 3-kernel: AR alone, add + RMSNorm on it, quant alone
    ro3, out3 = F.reduce_add_rmsnorm([ar], u.res, u.g, EPS)
    q3, s3 = F.quant_group(out3)
    torch.cuda.synchronize()
    r_ro3, r_out3 = oracle.reduce_add_rmsnorm(ref_ar[None], d["residual"], d["gamma"], EPS)
    r_q3, r_s3 = oracle.quant_group(r_out3)
    ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro3), r_ro3),
                               compare_bf16("out", from_dev_bf16(out3), r_out3),
                               compare_fp8(q3.cpu().numpy(), r_q3, s3.cpu().numpy(), r_s3))
    assert ok, why


@pytest.mark.parametrize("H", [128, 4096, 7168, 10240, 16384, 20480, 32768])
def test_reduce_alone_shapes(dev, H):
    """The all-reduce alone at every launch shape (one vector per lane; two or four per lane
    above H = 8192 on as few lanes as cover the row: 640 lanes at H = 10240 and 20480, 1024 at
    16384 and 32768), bit for bit against the oracle's block."""
    d = make_inputs(CONFIGS["decode_ds"], seed=H, R=8, T=7, H=H)
    u = Uploaded(d, dev)
    say(f"[gpu] reduce alone H={H}")
    ar = F.reduce(u.P)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(ar), oracle.reduce(d["partials"]))


@pytest.mark.parametrize("H", [128, 4096, 7168, 10240, 16384, 20480, 32768])
def test_quant_alone_shapes(dev, H):
    rng = np.random.default_rng(H)
    x = rng.standard_normal((5, H)).astype(np.float32)
    x[:, rng.choice(H, max(1, H // 100), replace=False)] *= 20
    x[3, :128] = 0
    import torch as _t
    xb = _t.from_numpy(x).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16)
    say(f"[gpu] quant alone H={H}")
    q, s = F.quant_group(to_dev_bf16(xb, dev))
    torch.cuda.synchronize()
    rq, rs = oracle.quant_group(xb)
    assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs)



def test_quant_every_group_max(dev):
    """One 128-channel group for each of the 32,768 bf16 magnitude patterns as its maximum (zero,
    subnormals, normals, inf, every NaN), its other channels random below it with random signs:
    the quant alone gives scales bit-identical to the oracle's (IEEE single divisions) for every
    one of them, and codes bit-identical wherever the quotient is a number. A NaN group's
    quotients are NaN, whose sign IEEE 754 leaves open (the oracle's division keeps the NaN
    operand's sign, the kernel's correction step may flip it): there both codes must be NaN
    codes (0x7F / 0xFF)."""
    rng = np.random.default_rng(91)
    T, H = 512, 8192
    ng = H // 128
    p = np.arange(0x8000, dtype=np.uint32).reshape(T, ng)
    mag = rng.integers(0, 1 << 16, size=(T, ng, 128), dtype=np.uint32) % (p[..., None] + 1)
    mag[np.arange(T)[:, None], np.arange(ng)[None, :], rng.integers(0, 128, size=(T, ng))] = p
    sign = rng.integers(0, 2, size=mag.shape, dtype=np.uint32) << 15
    xb = (mag | sign).astype(np.uint16).reshape(T, H)
    say(f"[gpu] quant alone, every group maximum T={T} H={H}")
    q, s = F.quant_group(to_dev_bf16(xb, dev))
    torch.cuda.synchronize()
    rq, rs = oracle.quant_group(xb)
    gs, gq = s.cpu().numpy(), q.cpu().numpy()
    nan = np.isnan(rs)
    assert nan.sum() == 0x8000 - 0x7F81 and np.array_equal(np.isnan(gs), nan)
    assert np.array_equal(gs[~nan].view(np.uint32), rs[~nan].view(np.uint32))
    ref_nan = (rq & 0x7F) == 0x7F  # every code of a NaN group, and inf / inf in the inf group
    assert ref_nan[np.repeat(nan, 128, axis=1)].all()
    bad = np.nonzero((gq != rq) & ~ref_nan)
    assert bad[0].size == 0, [(int(p[r, c // 128]), int(xb[r, c]), int(gq[r, c]), int(rq[r, c]))
                              for r, c in zip(*(b[:5] for b in bad))]
    assert ((gq[ref_nan] & 0x7F) == 0x7F).all()


def test_mxfp4_every_block_max(dev):
    """One 32-channel MXFP4 block for each of the 32,768 bf16 magnitude patterns as its maximum
    (zero, subnormals, normals, inf, every NaN), its other channels random below it with random
    signs. With every partial 1.0, no residual and eps = 0 a row's mean square is exactly 1, so
    rstd = 1 and the normalised output is gamma itself: gamma sets the blocks, 1,024 per call of
    H = 32768. Codes and scale bytes equal the oracle's bit for bit, and so do the FP8 codes and
    scales of the same outputs (groups of four such blocks)."""
    rng = np.random.default_rng(92)
    H = 32768
    nb = H // 32
    P1 = np.full((1, 1, H), 0x3F80, np.uint16)
    Pd = [to_dev_bf16(P1[0], dev)]
    say(f"[gpu] MXFP4 every block maximum, {0x8000 // nb} calls of H={H}")
    for c in range(0x8000 // nb):
        p = np.arange(c * nb, (c + 1) * nb, dtype=np.uint32)
        mag = rng.integers(0, 1 << 16, size=(nb, 32), dtype=np.uint32) % (p[:, None] + 1)
        mag[np.arange(nb), rng.integers(0, 32, size=nb)] = p
        sign = rng.integers(0, 2, size=mag.shape, dtype=np.uint32) << 15
        g = (mag | sign).astype(np.uint16).reshape(H)
        gd = to_dev_bf16(g, dev)
        _, mout, mq, msc = F.reduce_add_rmsnorm_mxfp4(Pd, None, gd, 0.0)
        _, qout, q, sc = F.reduce_add_rmsnorm_quant_group(Pd, None, gd, 0.0)
        torch.cuda.synchronize()
        ref_m = oracle.reduce_add_rmsnorm_mxfp4(P1, None, g, 0.0, nthreads=ORACLE_THREADS)
        ref_q = oracle.reduce_add_rmsnorm_quant_group(P1, None, g, 0.0, 128, True, nthreads=ORACLE_THREADS)
        gnan = (g & 0x7FFF) > 0x7F80
        assert np.array_equal(ref_m[1][0][~gnan], g[~gnan])  # out is gamma
        for name, got in (("MXFP4 out", mout), ("FP8 out", qout)):
            rep = compare_bf16(name, from_dev_bf16(got), ref_m[1])
            assert rep["n_bit_diff"] == 0, (c, rep)
        _same_codes(mq.cpu().numpy(), ref_m[2], msc.cpu().numpy(), ref_m[3], lambda x: np.zeros(x.shape, bool))
        _same_codes(q.cpu().numpy(), ref_q[2], sc.cpu().numpy(), ref_q[3], lambda x: (x & 0x7F) == 0x7F)


def test_fp8_every_group_max_fused_one_slot(dev):
    """Each of the 32,768 bf16 magnitude patterns (zero, subnormals, normals, inf, every NaN) as
    the maximum of one 128-channel group through the fused FP8 call in the one-slot kernel (wide
    shape, H = 8192, 64 groups a call), so both the quotient path without the 2^64 rescaling and
    the rescaled one run on every group maximum. As above, all partials 1.0, no residual and
    eps = 0 make the output gamma. Codes and scales equal the oracle's bit for bit (NaN codes as
    NaN codes)."""
    rng = np.random.default_rng(93)
    H = 8192
    ng = H // 128
    P1 = np.full((1, 1, H), 0x3F80, np.uint16)
    Pd = [to_dev_bf16(P1[0], dev)]
    say(f"[gpu] FP8 every group maximum through the one-slot fused kernel, {0x8000 // ng} calls of H={H}")
    gs, qs = [], []
    for c in range(0x8000 // ng):
        p = np.arange(c * ng, (c + 1) * ng, dtype=np.uint32)
        mag = rng.integers(0, 1 << 16, size=(ng, 128), dtype=np.uint32) % (p[:, None] + 1)
        mag[np.arange(ng), rng.integers(0, 128, size=ng)] = p
        sign = rng.integers(0, 2, size=mag.shape, dtype=np.uint32) << 15
        g = (mag | sign).astype(np.uint16).reshape(H)
        _, out, q, sc = F.reduce_add_rmsnorm_quant_group(Pd, None, to_dev_bf16(g, dev), 0.0,
                                                         variant=F.VARIANT_WIDE)
        gs.append(g)
        qs.append((out, q, sc))
    torch.cuda.synchronize()
    for c, (g, (out, q, sc)) in enumerate(zip(gs, qs)):
        ref = oracle.reduce_add_rmsnorm_quant_group(P1, None, g, 0.0, 128, True, nthreads=ORACLE_THREADS)
        rep = compare_bf16("out", from_dev_bf16(out), ref[1])
        assert rep["n_bit_diff"] == 0, (c, rep)
        _same_codes(q.cpu().numpy(), ref[2], sc.cpu().numpy(), ref[3], lambda x: (x & 0x7F) == 0x7F)


# ------------------------------------------------------------------ MXFP4 output
def run_mxfp4(u: Uploaded, variant="auto", emit_out=True, rows=None, label="", ref=None):
    say(f"[gpu] mxfp4 {label} R={u.R} T={u.T} H={u.H} variant={variant} emit={emit_out}")
    ro, out, q, sc = F.reduce_add_rmsnorm_mxfp4(u.P, u.res, u.g, EPS, emit_out=emit_out, variant=VARIANTS[variant])
    torch.cuda.synchronize()
    rows = np.arange(u.T) if rows is None else np.asarray(rows)
    d = u.d
    if ref is None:
        ref = oracle.reduce_add_rmsnorm_mxfp4(d["partials"][:, rows, :],
                                              None if u.res is None else d["residual"][rows], d["gamma"], EPS,
                                              emit_out, nthreads=ORACLE_THREADS)
    ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro)[rows], ref[0]),
                               None if out is None else compare_bf16("out", from_dev_bf16(out)[rows], ref[1]), None)
    assert ok, f"{label}: {why}"
    rep = compare_mxfp4(q.cpu().numpy()[rows], ref[2], sc.cpu().numpy()[rows], ref[3])
    ok, why = mxfp4_within_tolerance(rep)
    assert ok, f"{label}: {why} {rep}"
    return rep


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["tiny", "decode_ds", "decode_fp8"])
def test_mxfp4_configs(dev, name, variant):
    u = Uploaded(make_inputs(CONFIGS[name], seed=90), dev)
    rep = run_mxfp4(u, variant, label=name)
    assert rep["n_code_diff"] == 0 and rep["n_scale_diff"] == 0  # bit-exact in practice


@pytest.mark.parametrize("variant", ["auto", "wide", "narrow"])
def test_mxfp4_prefill_all_rows(prefill, variant):
    rep = run_mxfp4(prefill, variant, label="prefill, every row", ref=_prefill_ref(prefill, "mxfp4"))
    say(f"[gpu]   {rep}")


@pytest.mark.parametrize("H", [32, 96, 160, 1024, 8224, 16384, 32768])
def test_mxfp4_edge_H(dev, H):
    u = Uploaded(make_inputs(CONFIGS["decode_fp8"], seed=H, R=3, T=5, H=H), dev)
    for variant in VARIANTS:
        run_mxfp4(u, variant, label=f"H{H}")


def test_mxfp4_no_residual_no_out_and_special_blocks(dev):
    d = make_inputs(CONFIGS["tiny"], seed=91, R=2, T=4, H=256)
    d["partials"][1, 1, 32:64] = d["partials"][0, 1, 32:64] ^ 0x8000   # row 1 block 1 cancels ...
    d["partials"][1, 2, 70] = 0x7FC0                                     # row 2 has a NaN
    u = Uploaded(d, dev, residual=False)                                 # ... with no residual: zero block
    for variant in VARIANTS:
        run_mxfp4(u, variant, emit_out=False, label="special")
    ro, out, q, sc = F.reduce_add_rmsnorm_mxfp4(u.P, None, u.g, EPS)
    torch.cuda.synchronize()
    scn = sc.cpu().numpy()
    assert scn[1, 1] == 0 and np.all(q.cpu().numpy()[1, 16:32] == 0)
    assert np.all(scn[2] == 0xFF)  # the NaN makes the whole row's out NaN


@pytest.mark.parametrize("name,shape", [("decode_ds", None), ("decode_fp8", None),
                                        ("decode_ds", (8, 1100, 7168)), ("decode_ds", (3, 40, 20480))])
def test_fp8_scales_column_major(dev, name, shape):
    """Column-major scales ([H/128, T]) hold the same values as the row-major ones, transposed;
    codes and bf16 outputs are unchanged. The decode shapes, a call of many rows (the streaming
    two-slot kernel with LDS reserved) and four vector slots per lane (H = 20480)."""
    extra = {} if shape is None else dict(R=shape[0], T=shape[1], H=shape[2])
    u = Uploaded(make_inputs(CONFIGS[name], seed=95, **extra), dev)
    say(f"[gpu] column-major scales {name}")
    r_ro, r_out, r_q, r_s = u.oracle_rows(np.arange(u.T), True)
    for variant in (F.VARIANT_WIDE, F.VARIANT_NARROW):
        a = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS, variant=variant)
        b = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS, variant=variant, scales_col_major=True)
        torch.cuda.synchronize()
        for x, y in zip(a[:3], b[:3]):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
        assert b[3].shape == (u.H // 128, u.T) and torch.equal(a[3].t().contiguous(), b[3])
        # against the oracle directly: its row-major scales, transposed
        rep = compare_fp8(b[2].cpu().numpy(), r_q, b[3].cpu().numpy().T, r_s)
        ok, why = within_tolerance(compare_bf16("residual_out", from_dev_bf16(b[0]), r_ro),
                                   compare_bf16("out", from_dev_bf16(b[1]), r_out), rep)
        assert ok, why


def test_random_shapes(dev):
    """Seeded random shapes through every entry point and both launch shapes."""
    rng = np.random.default_rng(2024)
    for i in range(24):
        R = int(rng.integers(1, 9))
        T = int(rng.integers(1, 300))
        H = int(rng.integers(1, 129)) * 128 if i % 3 else int(rng.integers(1, 2049)) * 8
        d = make_inputs(CONFIGS["decode_fp8"], seed=1000 + i, R=R, T=T, H=H)
        u = Uploaded(d, dev, residual=bool(i % 4))
        variant = ["auto", "wide", "narrow"][i % 3]
        run_and_compare(u, False, variant, label=f"rand{i}")
        if H % 128 == 0:
            run_and_compare(u, True, variant, emit_out=bool(i % 2), label=f"rand{i}")
        if H % 32 == 0:
            run_mxfp4(u, variant, emit_out=bool(i % 2), label=f"rand{i}")


def test_random_shapes_many_rows_bit_exact(dev):
    """Seeded random calls of many rows (T log-uniform over 300 .. 4000, H a multiple of 128 up
    to 32768, R = 1 .. 8, with and without residual; the automatic shape and both forced ones):
    the streaming two-slot kernels, the reserved-LDS launches and the four-slot kernels, every
    output bit for bit equal to the oracle's (plain, FP8 with and without the bf16 output,
    MXFP4). FARN_MANY_SHAPES=N runs N such calls instead of 18 (same seeds for the first 18),
    printing one line per call."""
    rng = np.random.default_rng(2025)
    n_calls = int(os.environ.get("FARN_MANY_SHAPES", "18"))
    for i in range(n_calls):
        R = int(rng.integers(1, 9))
        T = int(np.exp(rng.uniform(np.log(300), np.log(4000))))
        H = int(rng.integers(1, 65)) * 128 if i % 6 else int(rng.integers(129, 257)) * 128
        T = min(T, (24 << 20) // H)  # at most 24 M elements per array
        d = make_inputs(CONFIGS["decode_fp8"], seed=5000 + i, R=R, T=T, H=H)
        u = Uploaded(d, dev, residual=bool(i % 4))
        variant = ["auto", "wide", "narrow"][i % 3]
        emit = bool(i % 2)
        rows = np.arange(T)
        rep_ro, rep_out, _ = run_and_compare(u, False, variant, label=f"many{i}")
        assert rep_ro["n_bit_diff"] == 0 and rep_out["n_bit_diff"] == 0, (i, R, T, H)
        _, rep_out, rep_fp8 = run_and_compare(u, True, variant, emit_out=emit, label=f"many{i}")
        assert rep_fp8["n_code_diff"] == 0 and rep_fp8["max_scale_rel_err"] == 0.0, (i, R, T, H, rep_fp8)
        assert rep_out is None or rep_out["n_bit_diff"] == 0, (i, R, T, H)
        ro, out, q, sc = F.reduce_add_rmsnorm_mxfp4(u.P, u.res, u.g, EPS, emit_out=emit, variant=VARIANTS[variant])
        torch.cuda.synchronize()
        ref = oracle.reduce_add_rmsnorm_mxfp4(d["partials"], d["residual"] if u.res is not None else None,
                                              d["gamma"], EPS, emit, nthreads=ORACLE_THREADS)
        assert np.array_equal(from_dev_bf16(ro), ref[0]), (i, "MXFP4 residual_out")
        assert out is None or np.array_equal(from_dev_bf16(out), ref[1]), (i, "MXFP4 out")
        assert np.array_equal(q.cpu().numpy(), ref[2]) and np.array_equal(sc.cpu().numpy(), ref[3]), (i, "MXFP4 codes")
        if n_calls > 18:
            print(f"many{i}: R={R} T={T} H={H} {variant} residual={u.res is not None} emit={emit}: bit-exact",
                  flush=True)
        del u, d


# one point inside every band of the automatic shape rule (and the reserved-LDS launches), and
# points just outside them: (R, T, H)
RULE_BAND_POINTS = [
    (8, 64, 6272), (8, 600, 7168), (6, 2100, 7168), (4, 2048, 6656), (8, 4096, 8192), (8, 3000, 8192),
    (8, 1024, 5120), (2, 1500, 4736), (8, 2048, 5120), (4, 600, 2304), (2, 1500, 3072), (4, 1024, 4096),
    (3, 700, 6144), (8, 4096, 2048), (8, 4200, 1664), (8, 4096, 1536), (5, 520, 7168), (1, 513, 8192),
    (8, 800, 4736), (6, 300, 3328), (8, 100, 2560), (7, 400, 5504), (4, 700, 4096), (2, 1300, 4096),
    (8, 767, 3712),
]


@pytest.mark.parametrize("R,T,H", RULE_BAND_POINTS)
def test_rule_bands(dev, R, T, H):
    """Every band of the automatic launch-shape rule, with the LDS reservation where it applies,
    against the oracle on every row, through the plain, FP8 and MXFP4 calls."""
    d = make_inputs(CONFIGS["decode_fp8"], seed=3000 + R * 7 + T + H, R=R, T=T, H=H)
    u = Uploaded(d, dev, residual=bool((T + H) % 3))
    ref = u.oracle_rows(np.arange(T), False)
    rep_ro, rep_out, _ = run_and_compare(u, False, "auto", label="band", ref=ref)
    assert rep_ro["n_bit_diff"] == 0 and rep_out["n_bit_diff"] == 0
    if H % 128 == 0:
        _, rep_out, rep_fp8 = run_and_compare(u, True, "auto", label="band")
        assert rep_out["n_bit_diff"] == 0 and rep_fp8["n_code_diff"] == 0 and rep_fp8["max_scale_rel_err"] == 0.0
    if H % 32 == 0:
        rep = run_mxfp4(u, "auto", label="band")
        assert rep["n_code_diff"] == 0 and rep["n_scale_diff"] == 0


def test_two_streams_at_once(dev):
    """The library keeps no state: calls enqueued on two streams at the same time, on different
    inputs (one FP8, one plain, one MXFP4 per stream, back to back), each match the oracle."""
    cases = []
    for i, (T, H) in enumerate([(96, 7168), (40, 4096)]):
        d = make_inputs(CONFIGS["tiny"], seed=80 + i, R=4 + 4 * i, T=T, H=H)
        cases.append((d, Uploaded(d, dev)))
    torch.cuda.synchronize()  # inputs were uploaded on the default stream
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    say("[gpu] two streams at once")
    outs = []
    for (d, u), st in zip(cases, streams):
        with torch.cuda.stream(st):
            fp8 = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS)
            plain = F.reduce_add_rmsnorm(u.P, u.res, u.g, EPS)
            mx = F.reduce_add_rmsnorm_mxfp4(u.P, u.res, u.g, EPS)
        outs.append((fp8, plain, mx))
    torch.cuda.synchronize()
    for (d, u), (fp8, plain, mx) in zip(cases, outs):
        rows = np.arange(u.T)
        r_ro, r_out, r_q, r_s = u.oracle_rows(rows, True)
        assert np.array_equal(from_dev_bf16(fp8[0]), r_ro) and np.array_equal(from_dev_bf16(fp8[1]), r_out)
        rep = compare_fp8(fp8[2].cpu().numpy(), r_q, fp8[3].cpu().numpy(), r_s)
        assert rep["n_code_diff"] == 0 and rep["max_scale_rel_err"] == 0.0, rep
        assert np.array_equal(from_dev_bf16(plain[0]), r_ro) and np.array_equal(from_dev_bf16(plain[1]), r_out)
        m_ro, m_out, m_q, m_s = oracle.reduce_add_rmsnorm_mxfp4(d["partials"], d["residual"], d["gamma"], EPS,
                                                              True, nthreads=8)
        assert np.array_equal(mx[2].cpu().numpy(), m_q) and np.array_equal(mx[3].cpu().numpy(), m_s)


def test_plain_c_client():
    """tests/c_abi_client.c: a C program with no Python and no torch calls the ABI on
    hipMalloc'd memory and checks closed-form results (exit status 0 = all hold)."""
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_client")
    if not os.path.exists(exe):
        pytest.fail("tests/c_abi_client is not built (python tp_all_reduce_amd/build.py builds it)")
    print("case: plain C client", flush=True)
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert "0 mismatches" in proc.stdout


# ------------------------------------------------------------------ row schedules
@pytest.mark.parametrize("quant", ["fp8", "mxfp4"])
def test_small_and_streaming_schedules_agree(dev, quant):
    """The two-slot quant kernels store in a different order for few rows (T <= 512) than for
    many; results must not depend on it. The same 512 rows run as a 512-row call (small-call
    schedule) and inside a 520-row call (streaming schedule), narrow shape, and every output
    byte of those rows must agree; the small call is also checked against the oracle."""
    d = make_inputs(CONFIGS["decode_ds"], seed=77, T=520)
    u = Uploaded(d, dev)
    P512 = [p[:512] for p in u.P]
    call = F.reduce_add_rmsnorm_quant_group if quant == "fp8" else F.reduce_add_rmsnorm_mxfp4
    say(f"[gpu] schedules agree ({quant}): T=512 vs T=520")
    big = call(u.P, u.res, u.g, EPS, variant=F.VARIANT_NARROW)
    small = call(P512, u.res[:512], u.g, EPS, variant=F.VARIANT_NARROW)
    torch.cuda.synchronize()
    for a, b in zip(small, big):
        assert torch.equal(a.view(torch.uint8), b[:512].contiguous().view(torch.uint8))
    if quant == "fp8":
        r = oracle.reduce_add_rmsnorm_quant_group(d["partials"][:, :512], d["residual"][:512], d["gamma"], EPS,
                                                  nthreads=8)
        ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(small[0]), r[0]),
                                   compare_bf16("out", from_dev_bf16(small[1]), r[1]),
                                   compare_fp8(small[2].cpu().numpy(), r[2], small[3].cpu().numpy(), r[3]))
    else:
        r = oracle.reduce_add_rmsnorm_mxfp4(d["partials"][:, :512], d["residual"][:512], d["gamma"], EPS, nthreads=8)
        ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(small[0]), r[0]),
                                   compare_bf16("out", from_dev_bf16(small[1]), r[1]), None)
        ok2, why2 = mxfp4_within_tolerance(compare_mxfp4(small[2].cpu().numpy(), r[2], small[3].cpu().numpy(), r[3]))
        ok, why = ok and ok2, f"{why} {why2}"
    assert ok, why


# ------------------------------------------------------------------ binding checks
def test_binding_stream_handle(dev):
    """The binding launches on the stream torch reports as current: its raw handle lookup agrees
    with torch.cuda.current_stream on the default stream and inside a side-stream context."""
    assert F._stream(dev, None) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert F._stream(dev, None) == torch.cuda.current_stream(dev).cuda_stream == s.cuda_stream
    assert F._stream(dev, s) == s.cuda_stream


def test_explicit_stream_outputs(dev):
    """A call given stream= (not the current stream) launches there with outputs the wrapper
    allocates and marks as used on that stream; after that stream finishes they hold the
    oracle's results."""
    d = make_inputs(CONFIGS["decode_ds"], seed=12, T=40)
    u = Uploaded(d, dev)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    say("[gpu] explicit stream, wrapper-allocated outputs")
    ro, out, q, sc = F.reduce_add_rmsnorm_quant_group(u.P, u.res, u.g, EPS, stream=s)
    s.synchronize()
    ref = u.oracle_rows(np.arange(u.T), True)
    ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(ro), ref[0]),
                               compare_bf16("out", from_dev_bf16(out), ref[1]),
                               compare_fp8(q.cpu().numpy(), ref[2], sc.cpu().numpy(), ref[3]))
    assert ok, why


def test_binding_rejects_bad_output_buffers(dev):
    """Output buffers of the wrong shape, dtype or device are refused by the binding before
    the library is called (the library only sees pointers)."""
    T, H = 4, 256
    P = [torch.zeros(T, H, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    g = torch.ones(H, dtype=torch.bfloat16, device=dev)
    small = torch.empty(T - 1, H, dtype=torch.bfloat16, device=dev)
    host = torch.empty(T, H, dtype=torch.bfloat16)
    bad = [
        lambda: F.reduce_add_rmsnorm(P, None, g, residual_out=small),
        lambda: F.reduce_add_rmsnorm(P, None, g, out=host),
        lambda: F.reduce_add_rmsnorm_quant_group(P, None, g, residual_out=small),
        lambda: F.reduce_add_rmsnorm_quant_group(P, None, g, out=host),
        lambda: F.reduce_add_rmsnorm_quant_group(P, None, g, q=torch.empty(T, H, dtype=torch.uint8)),
        lambda: F.reduce_add_rmsnorm_quant_group(P, None, g, scales=torch.empty(T, dtype=torch.float32, device=dev)),
        lambda: F.reduce_add_rmsnorm_quant_group(P, None, g, q=torch.empty(T, H, dtype=torch.int32, device=dev)),
        lambda: F.reduce_add_rmsnorm_mxfp4(P, None, g, residual_out=small),
        lambda: F.reduce_add_rmsnorm_mxfp4(P, None, g, q=torch.empty(T, H, dtype=torch.uint8, device=dev)),
        lambda: F.reduce_add_rmsnorm_mxfp4(P, None, g, scales=torch.empty(T, H // 32, dtype=torch.uint8)),
        lambda: F.reduce(P, out=small),
        lambda: F.quant_group(P[0], q=torch.empty(T, H - 128, dtype=torch.uint8, device=dev)),
        lambda: F.quant_group(P[0], scales=torch.empty(T, H // 128, dtype=torch.float32)),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
            pytest.fail(f"case {i} was accepted")
    torch.cuda.synchronize()
