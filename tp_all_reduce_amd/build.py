"""Build libfarn.so (gfx950) in-tree with hipcc.

    python tp_all_reduce_amd/build.py

(Run it by path: importing the package loads the built library.)

The C-ABI layer (csrc/farn_api.cpp) makes no HIP call and is compiled by g++; the
kernels (csrc/farn_kernels.hip) by hipcc for gfx950; hipcc links the two.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfarn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are kept out of every kernel: the compiler is asked not to
# form them from ordinary float code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; nothing else is expected
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    lines = [ln for ln in proc.stdout.splitlines() if ln.strip() and not any(n in ln for n in noise)]
    if proc.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return lines


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    api_o = os.path.join(BUILD_DIR, "farn_api.o")
    ker_o = os.path.join(BUILD_DIR, "farn_kernels.o")
    out = []
    out += _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "farn_api.cpp"), "-o", api_o])
    out += _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "farn_kernels.hip"), "-o", ker_o])
    tmp = LIB + f".tmp{os.getpid()}"
    out += _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, api_o, ker_o])
    os.replace(tmp, LIB)
    if verbose:
        for ln in out:
            print(ln)
    return LIB


if __name__ == "__main__":
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        sys.exit(f"hipcc not found at {HIPCC}")
    print(build(verbose=True))
