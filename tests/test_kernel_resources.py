"""Register and private-memory use of every kernel in the built library (CPU only).

The gfx950 code object is taken out of libfarn.so's offload bundle and its AMDGPU
metadata read with llvm-readelf. Every kernel must keep all its state in registers and
LDS: no private (scratch) segment and no spilled VGPRs or SGPRs. A kernel of 1024 lanes
has at most 128 VGPRs per lane (the register file holds 512 per SIMD lane and such a
workgroup puts four waves on each SIMD); the four-slot kernels for rows beyond 16384
channels are the ones closest to that limit, and they spilled before each slot's gamma
was loaded only when it is normalised.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tp_all_reduce_amd", "libfarn.so")
LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
BUNDLER = os.path.join(LLVM, "clang-offload-bundler")
READELF = os.path.join(LLVM, "llvm-readelf")
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _kernel_metadata(tmp_path):
    """One dict per kernel: the scalar fields of its metadata map (name, counts, sizes)."""
    if not os.path.exists(LIB):
        pytest.skip("libfarn.so is not built")
    objcopy = shutil.which("objcopy")
    if objcopy is None or not os.path.exists(BUNDLER) or not os.path.exists(READELF):
        pytest.skip("objcopy, clang-offload-bundler or llvm-readelf not found")
    fat = tmp_path / "fat.bin"
    code = tmp_path / "gfx950.co"
    subprocess.run([objcopy, "-O", "binary", "--only-section=.hip_fatbin", LIB, str(fat)], check=True)
    listed = subprocess.run([BUNDLER, "--list", "--type=o", f"--input={fat}"], check=True,
                            capture_output=True, text=True).stdout.split()
    assert TARGET in listed, listed
    subprocess.run([BUNDLER, "--unbundle", "--type=o", f"--input={fat}", f"--targets={TARGET}",
                    f"--output={code}"], check=True)
    notes = subprocess.run([READELF, "--notes", str(code)], check=True, capture_output=True,
                           text=True).stdout
    kernels, cur = [], None
    for line in notes.splitlines():
        m = re.match(r"^  - \.(\w+):\s*(\S*)", line)  # first key of a kernel's map
        if m:
            cur = {m.group(1): m.group(2)}
            kernels.append(cur)
            continue
        m = re.match(r"^    \.(\w+):\s*(\S+)", line)  # the kernel map's own keys, not its args'
        if m and cur is not None:
            cur[m.group(1)] = m.group(2)
    return [k for k in kernels if ".kd" in k.get("symbol", "")]


def test_no_kernel_uses_private_memory(tmp_path):
    kernels = _kernel_metadata(tmp_path)
    names = [k["name"] for k in kernels]
    # the fused kernel of every rank count, slot count and output kind, and the unfused blocks
    assert sum("farn_rows" in n for n in names) >= 8 * 3 * 3, len(names)
    assert any("farn_reduce_rows" in n for n in names) and any("farn_quant_rows" in n for n in names)
    bad = [(k["name"], k["private_segment_fixed_size"], k["vgpr_spill_count"], k["sgpr_spill_count"])
           for k in kernels
           if (k["private_segment_fixed_size"], k["vgpr_spill_count"], k["sgpr_spill_count"]) != ("0", "0", "0")]
    assert not bad, bad
    for k in kernels:
        assert k["uses_dynamic_stack"] == "false", k["name"]
        assert k["wavefront_size"] == "64", k["name"]


def test_register_budget_of_1024_lane_kernels(tmp_path):
    kernels = _kernel_metadata(tmp_path)
    wide = [k for k in kernels if int(k["max_flat_workgroup_size"]) == 1024]
    assert wide
    for k in wide:
        assert int(k["vgpr_count"]) + int(k.get("agpr_count", "0")) <= 128, (k["name"], k["vgpr_count"])
