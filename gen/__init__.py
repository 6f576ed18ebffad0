"""Seeded synthetic inputs for the fused reduce + residual-add + RMSNorm (+ FP8 quant) op.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
bench. It draws random numbers and rounds them to bf16 with torch's own cast;
it holds none of the op's arithmetic.
"""

from .inputs import CONFIGS, SWEEP_T, Config, make_inputs, sweep_config  # noqa: F401
