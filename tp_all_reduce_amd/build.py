"""Build libfarn.so (gfx950) in-tree with hipcc.

    python tp_all_reduce_amd/build.py

(Run it by path: importing the package loads the built library.)

The C-ABI layer (csrc/farn_api.cpp) makes no HIP call and is compiled by g++; the
kernels (csrc/farn_kernels.hip) by hipcc for gfx950; hipcc links the two. The tensor-level
Python binding (csrc/farn_torch.cpp -> _farn_torch.so) is compiled by g++ against torch's
headers and links libfarn.so. The plain C
client of the ABI that the GPU tests run (tests/c_abi_client.c) is compiled by gcc
against include/farn.h and the built library, and the test kernels of the conversion
instructions (tests/hw_conversions.hip) by hipcc.
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
TORCH_BINDING = os.path.join(HERE, "_farn_torch.so")
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_abi_client")
HWCONV_SRC = os.path.join(ROOT, "tests", "hw_conversions.hip")
HWCONV = os.path.join(ROOT, "tests", "libhwconv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
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
    out += build_torch_binding()
    out += build_c_client()
    out += build_hwconv()
    if verbose:
        for ln in out:
            print(ln)
    return LIB


def build_c_client() -> list:
    """gcc, no HIP compiler: the client sees only the C header, the HIP runtime API and
    libfarn.so (found next to the package through the rpath)."""
    tmp = C_CLIENT + f".tmp{os.getpid()}"
    out = _run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                f"-I{ROCM}/include", C_CLIENT_SRC, "-o", tmp, f"-L{HERE}", "-lfarn",
                f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/../tp_all_reduce_amd",
                f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, C_CLIENT)
    return out


def build_torch_binding() -> list:
    """The tensor-level Python binding (csrc/farn_torch.cpp): a torch C++ extension compiled
    by g++ against torch's headers, linked to libfarn.so (found next to it through the
    rpath) and to the torch libraries the importing process has already loaded."""
    import sysconfig

    import torch
    from torch.utils import cpp_extension

    tmp = TORCH_BINDING + f".tmp{os.getpid()}"
    abi = int(torch._C._GLIBCXX_USE_CXX11_ABI)
    cmd = ["g++", *CXX_FLAGS, "-shared", f"-D_GLIBCXX_USE_CXX11_ABI={abi}",
           "-DTORCH_EXTENSION_NAME=_farn_torch", "-DTORCH_API_INCLUDE_EXTENSION_H",
           *[f"-I{p}" for p in cpp_extension.include_paths()], f"-I{sysconfig.get_paths()['include']}",
           os.path.join(CSRC, "farn_torch.cpp"), "-o", tmp,
           *[f"-L{p}" for p in cpp_extension.library_paths()], "-lc10", "-ltorch", "-ltorch_cpu",
           "-ltorch_python", f"-L{HERE}", "-lfarn", "-Wl,-rpath,$ORIGIN"]
    # torch's own headers trip -Wextra's unused-parameter warning; the binding's code does not
    cmd.append("-Wno-unused-parameter")
    out = _run(cmd)
    os.replace(tmp, TORCH_BINDING)
    return out


def build_hwconv() -> list:
    """The test kernels of the conversion instructions the quant paths use."""
    tmp = HWCONV + f".tmp{os.getpid()}"
    out = _run([HIPCC, *HIP_FLAGS, "-shared", "-o", tmp, HWCONV_SRC])
    os.replace(tmp, HWCONV)
    return out


if __name__ == "__main__":
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        sys.exit(f"hipcc not found at {HIPCC}")
    print(build(verbose=True))
