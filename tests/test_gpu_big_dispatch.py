"""GPU test of calls taller than one dispatch (about 161 GiB of device memory). It runs before
the other GPU test files: freeing that much memory leaves the next process's calls about 1 %
slower for a few seconds, which is kept away from whatever runs after the suite."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import tp_all_reduce_amd as F
from gen import CONFIGS, make_inputs
from parity import compare_bf16, compare_fp8, from_dev_bf16, to_dev_bf16, within_tolerance

pytestmark = pytest.mark.gpu
EPS = 1e-6


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    return torch.device("cuda:0")


def test_rows_beyond_one_dispatch(dev):
    """One workgroup per row, and a dispatch holds at most 2^32 - 1 work-items: at H = 8192 on
    the one-vector-per-lane shape (1024 lanes) that is 4,194,303 rows, so T = 4,194,308 goes
    out as two launches. The all-reduce alone, the quant alone and the fused FP8 call (no
    residual, no bf16 out, column-major scales) are compared with the oracle on the rows
    around the boundary and the last row; every output starts as all-ones bytes, so a row left
    unwritten shows. Needs about 161 GiB of device memory."""
    H, lanes = 8192, 1024
    per = (2 ** 32 - 1) // lanes
    T = per + 5
    G = H // 128
    need = T * H * (2 + 2 + 1) + T * G * 4
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(dev)
    if free < need + (4 << 30):
        pytest.skip(f"needs {need / 2 ** 30:.0f} GiB of free device memory, {free / 2 ** 30:.0f} GiB free")
    blk_rows = 64  # a seeded block of distinct rows, repeated down the array
    d = make_inputs(CONFIGS["decode_ds"], seed=91, R=1, T=blk_rows, H=H)
    rows = np.array([0, 1, per - 2, per - 1, per, per + 1, T - 1])
    src = d["partials"][0][rows % blk_rows]
    say(f"[gpu] rows beyond one dispatch: T={T} H={H} ({need / 2 ** 30:.0f} GiB)")
    A = B = Q = S = None
    try:
        blk = to_dev_bf16(d["partials"][0], dev)
        A = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        n = T // blk_rows
        A[: n * blk_rows].view(n, blk_rows, H).copy_(blk.unsqueeze(0).expand(n, blk_rows, H))
        A[n * blk_rows:].copy_(blk[: T - n * blk_rows])
        B = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        Q = torch.empty((T, H), dtype=torch.uint8, device=dev)
        S = torch.empty((G, T), dtype=torch.float32, device=dev)
        idx = torch.from_numpy(rows).to(dev)
        g = to_dev_bf16(d["gamma"], dev)

        say("[gpu]   all-reduce alone")
        B.view(torch.int16).fill_(-1)
        F.reduce([A], out=B)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_bf16(B[idx]), oracle.reduce(src[None]))

        say("[gpu]   quant alone")
        Q.fill_(0xFF)
        S.fill_(float("nan"))
        F.quant_group(B, q=Q, scales=S.view(T, G))
        torch.cuda.synchronize()
        rq, rs = oracle.quant_group(src)
        assert np.array_equal(Q[idx].cpu().numpy(), rq)
        assert np.array_equal(S.view(T, G)[idx].cpu().numpy(), rs)

        say("[gpu]   fused FP8, wide shape, column-major scales")
        B.view(torch.int16).fill_(-1)
        Q.fill_(0xFF)
        S.fill_(float("nan"))
        F.reduce_add_rmsnorm_quant_group([A], None, g, EPS, emit_out=False, residual_out=B, q=Q,
                                         scales=S, variant=F.VARIANT_WIDE, scales_col_major=True)
        torch.cuda.synchronize()
        r_ro, _, r_q, r_s = oracle.reduce_add_rmsnorm_quant_group(src[None], None, d["gamma"], EPS,
                                                                  emit_out=False)
        ok, why = within_tolerance(compare_bf16("ro", from_dev_bf16(B[idx]), r_ro), None,
                                   compare_fp8(Q[idx].cpu().numpy(), r_q, S[:, idx].T.cpu().numpy(), r_s))
        assert ok, why
    finally:
        del A, B, Q, S
        torch.cuda.empty_cache()
