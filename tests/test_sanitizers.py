"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (CPU only): the
C-ABI validation layer, with the kernel launcher replaced by a recording stub, and the CPU
oracle. Each is built by g++/gcc into an executable that exercises every entry point
(tests/sanitize_abi_driver.cpp, tests/sanitize_oracle_driver.c) and must exit cleanly with
no sanitizer report."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "ERROR: AddressSanitizer" not in p.stderr and "runtime error" not in p.stderr, p.stderr
    return p.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", *SAN,
                    os.path.join(ROOT, "tp_all_reduce_amd", "csrc", "farn_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize_abi_driver.cpp"), "-o", exe], check=True)
    out = _run(exe)
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-pthread", *SAN,
                    os.path.join(ROOT, "oracle", "farn_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize_oracle_driver.c"), "-o", exe, "-lm"], check=True)
    out = _run(exe)
    assert "0 failures" in out
