"""Seeded input generator: rank partials, residual and gamma as raw bf16 bits.

Workload shapes follow the serving shapes the pages discuss:
  * H = 7168 is the DeepSeek hidden size the one-stage fused kernel was extended
    to ("ROCm AITER fused all-reduce + RMSNorm" summary, review notes on
    DeepSeek support and hidden_dim 7168); 4096 and 8192 sit in / next to the
    supported hidden set of the same page's `_rocm_aiter_fused_allreduce_rmsnorm_impl`.
  * R = 8 is the largest TP degree the pages run ("[AMD] Support
    --enable-aiter-allreduce-fusion on AMD GPUs", Commands Used, `--tp 8`).
  * T = 64 is a decode batch, T = 8192 a prefill chunk, and the sweep covers the
    32K..64M per-rank message sizes of the TP=8 all-reduce table in
    "[AMD] Add AITER Custom All-Reduce" (Benchmarking and Profiling).
  * group 128 FP8 quant with outlier channels exercises the per-1x128 quant of
    "AMD fused AllReduce-RMSNorm quant kernel" (sglang #24651 summary, layernorm.py
    snippet).

Distributions (all drawn in float32 from numpy's PCG64, then rounded to bf16 by
torch's float32 -> bfloat16 cast):
  partials P_r ~ N(0, 1/R) (so the rank sum is ~N(0, 1)), residual ~ N(0, 1),
  gamma ~ U(0.5, 1.5). With outliers, round(frac * H) distinct channels (drawn
  without replacement, shared by every rank) of every partial are scaled x20
  before rounding. Each array has its own stream: `SeedSequence(seed).spawn(R + 3)`
  gives children 0..R-1 for P_0..P_{R-1} (each [T, H] row-major), R for the
  residual, R+1 for gamma and R+2 for the outlier channel set, so the arrays can
  be drawn in parallel threads and still come out the same.

Random numbers are the only thing this module computes: no step of the op.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    R: int
    T: int
    H: int
    quant: tuple  # which quant modes the workload is run with (False = plain call, True = FP8 call)
    outlier_frac: float = 0.0
    seed: int = 0
    what: str = ""

    @property
    def nbytes_plain(self) -> int:
        """Algorithmic bytes of one plain call: (R+1) inputs read, residual_out and out written."""
        th = self.T * self.H
        return self.R * th * 2 + th * 2 + 2 * th * 2

    def nbytes_quant(self, emit_out: bool = True) -> int:
        """Algorithmic bytes of one FP8 call: plain bytes, + codes and fp32 group scales,
        minus the bf16 `out` when it is not emitted."""
        th = self.T * self.H
        b = self.nbytes_plain + th + self.T * (self.H // 128) * 4
        if not emit_out:
            b -= th * 2
        return b


CONFIGS = {
    "tiny": Config("tiny", R=2, T=4, H=256, quant=(False,), what="tiny parity case"),
    "decode_ds": Config("decode_ds", R=8, T=64, H=7168, quant=(False,),
                        what="decode, DeepSeek-like hidden size"),
    "decode_fp8": Config("decode_fp8", R=4, T=16, H=4096, quant=(True,), outlier_frac=0.01,
                         what="decode with per-group FP8 quant and 1% outlier channels"),
    "prefill": Config("prefill", R=8, T=8192, H=7168, quant=(False, True),
                      what="prefill chunk, with and without FP8 quant"),
}


def sweep_config(T: int) -> Config:
    """Message-size sweep point: R=8, H=8192, T tokens (T*H*2 bytes per rank buffer)."""
    return Config(f"sweep_T{T}", R=8, T=T, H=8192, quant=(False,), what="message-size sweep")


SWEEP_T = tuple(2 ** k for k in range(1, 13))  # 2 .. 4096


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via torch's cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_inputs(cfg: Config, seed: int | None = None, T: int | None = None,
                R: int | None = None, H: int | None = None) -> dict:
    """Draw one batch for `cfg` (shape overrides allowed for edge-case tests).

    Returns a dict of numpy arrays:
      partials [R, T, H] uint16 (bf16 bits), residual [T, H] uint16,
      gamma [H] uint16, outliers int64 channel indices (possibly empty).
    """
    R = cfg.R if R is None else R
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    seed = cfg.seed if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(R + 3)
    std = np.float32(1.0 / np.sqrt(R))
    n_out = int(round(cfg.outlier_frac * H)) if cfg.outlier_frac else 0
    outliers = np.zeros(0, dtype=np.int64)
    if n_out:
        pick = np.random.default_rng(kids[R + 2])
        outliers = np.sort(pick.choice(H, size=n_out, replace=False)).astype(np.int64)

    partials = np.empty((R, T, H), dtype=np.uint16)

    def draw_partial(r: int) -> None:
        x = np.random.default_rng(kids[r]).standard_normal((T, H), dtype=np.float32)
        x *= std
        if n_out:
            x[:, outliers] *= np.float32(20.0)
        partials[r] = _to_bf16_bits(x)

    workers = max(1, min(8, len(os.sched_getaffinity(0)), R))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(draw_partial, range(R)))
    residual = _to_bf16_bits(np.random.default_rng(kids[R]).standard_normal((T, H), dtype=np.float32))
    gamma = _to_bf16_bits(np.random.default_rng(kids[R + 1]).uniform(0.5, 1.5, size=H).astype(np.float32))
    return {"partials": partials, "residual": residual, "gamma": gamma, "outliers": outliers,
            "R": R, "T": T, "H": H}
