"""Host-side tests of the C ABI (no GPU): the library loads, exports every function
include/farn.h declares, and rejects every malformed call with the documented status
before touching the GPU. Pointers here are fake, aligned host addresses: the checks
never dereference them, and every call below is rejected before any HIP call."""

from __future__ import annotations

import ctypes
import json
import os
import re
import subprocess

import pytest

import tp_all_reduce_amd as F

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "farn.h")
L = F.lib()

OK, NULL, SHAPE, ALIGN, ALIAS, EPS, LAUNCH, VARIANT = range(8)
MiB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(farn_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    declared = declared_functions()
    assert set(declared) == set(F.EXPORTS), declared
    nm = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r"\bT (farn_[a-z0-9_]+)$", nm, flags=re.M))
    assert exported == set(declared), (exported, declared)
    for name in declared:
        assert hasattr(L, name)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (FARN_[A-Z_]+) (\d+)", text))
    assert int(consts["FARN_MAX_R"]) == F.MAX_R
    assert int(consts["FARN_MAX_H"]) == F.MAX_H
    assert int(consts["FARN_GROUP"]) == F.GROUP
    assert int(consts["FARN_MX_BLOCK"]) == F.MX_BLOCK
    assert int(consts["FARN_ABI_VERSION"]) == F.abi_version()
    names = re.findall(r"(FARN_(?:OK|ERR_[A-Z]+)) = (\d+)", text)
    assert {int(v): k for k, v in names} == F.STATUS


def test_status_strings_and_select():
    for s in range(8):
        assert L.farn_status_string(s)
    assert L.farn_status_string(99) == b"unknown status"
    for T in (1, 2, 64, 512, 4096, 8192, 1 << 20):
        for H in (256, 7168, 8192):
            assert F.select_variant(8, T, H, False) in (F.VARIANT_WIDE, F.VARIANT_NARROW)
    assert (F.VARIANT_LATENCY, F.VARIANT_BANDWIDTH) == (F.VARIANT_WIDE, F.VARIANT_NARROW)


W, N = F.VARIANT_WIDE, F.VARIANT_NARROW
# Every band of the AUTO rule as include/farn.h states it, at its edges: (R, T, H, quant, shape)
HEADER_RULE_POINTS = [
    # 6144 < H <= 8192, except the plain call with H > 7168 from T = 4096
    (8, 1, 6152, False, N), (8, 64, 7168, False, N), (8, 8192, 7168, False, N), (8, 8192, 7168, True, N),
    (2, 8192, 7168, False, N), (8, 64, 8192, False, N), (8, 4095, 8192, False, N), (8, 4096, 8192, False, W),
    (8, 8192, 8192, False, W), (2, 4096, 8192, False, W), (8, 8192, 8192, True, N), (8, 4096, 7176, False, W),
    (8, 4096, 7168, False, N), (8, 64, 6144, False, W), (8, 8192, 8192, "mxfp4", N), (8, 64, 7168, "mxfp4", N),
    # 4608 < H <= 5120 with 768 <= T < 2048
    (8, 768, 5120, False, N), (8, 2047, 4616, True, N), (8, 767, 5120, False, W), (8, 2048, 5120, False, W),
    (8, 1024, 4608, False, W), (8, 1024, 5128, False, W), (6, 1000, 4736, "mxfp4", N), (8, 767, 5120, True, W),
    # the FP8 call with 2048 < H <= 6144 and T < 768, when H <= 3712 from T = 80 or 256 <= T < 512
    (8, 80, 2560, True, N), (8, 79, 2560, True, W), (8, 16, 2560, True, W), (2, 1, 3712, True, W),
    (8, 80, 2560, False, W), (8, 80, 2560, "mxfp4", W), (8, 767, 3712, True, N),
    (8, 768, 3712, True, W), (8, 100, 3720, True, W), (8, 256, 6144, True, N), (8, 511, 4096, True, N),
    (8, 512, 4096, True, W), (8, 255, 4096, True, W), (8, 300, 2048, True, W), (8, 300, 2056, True, N),
    (1, 80, 2056, True, N), (1, 1, 2056, True, W), (6, 300, 4096, "fp8", N), (6, 300, 4096, "mxfp4", W),
    # R <= 4 and 2048 < H <= 6144 with 512 <= T < 768 (R <= 2: T < 1536)
    (4, 512, 2056, False, N), (4, 767, 6144, False, N), (4, 768, 4096, False, W), (4, 511, 3072, False, W),
    (2, 1535, 4096, False, N), (2, 1536, 3072, False, W), (1, 512, 4096, False, N), (5, 512, 3072, False, W),
    (4, 512, 2048, False, W), (3, 600, 6144, "mxfp4", N), (2, 1024, 4096, "mxfp4", N), (4, 700, 6144, True, N),
    # everything else: wide (H = 1544 .. 2048 from T = 4096 included)
    (8, 4096, 2048, False, W), (8, 8192, 1544, True, W), (8, 64, 4096, False, W), (8, 8192, 4096, True, W),
    (8, 8192, 6144, False, W), (8, 1024, 2048, False, W), (4, 16, 4096, True, W), (8, 4, 256, False, W),
    (2, 8192, 32768, False, W), (2, 8192, 32768, "mxfp4", W),
]


@pytest.mark.parametrize("R,T,H,quant,shape", HEADER_RULE_POINTS)
def test_select_matches_header(R, T, H, quant, shape):
    """farn_select_variant implements the rule include/farn.h documents, at every band edge."""
    assert F.select_variant(R, T, H, quant) == shape


def test_header_states_the_rule():
    text = open(HEADER).read()
    for phrase in ("6144 < H <= 8192, except the plain call with H > 7168 from T = 4096",
                   "4608 < H <= 5120 with 768 <= T < 2048",
                   "the FP8 call with 2048 < H <= 6144 and T < 768, when H <= 3712 from T = 80 or 256 <= T < 512",
                   "R <= 4 and 2048 < H <= 6144 with 512 <= T < 768 (R <= 2: T < 1536)",
                   "and WIDE everywhere else", "quant: 0 for the plain call, 1 for the FP8 call, 2 for the MXFP4 call"):
        assert phrase in " ".join(text.replace("*", " ").split()), phrase


class FakeCall:
    """A well-formed plain / FP8 call over fake, disjoint, 4 KiB-aligned host addresses."""

    def __init__(self, R=2, T=4, H=256, quant=False):
        self.R, self.T, self.H, self.quant = R, T, H, quant
        base = 0x10_0000_0000
        self.partials = [base + i * 16 * MiB for i in range(R)]
        self.residual = base + 100 * 16 * MiB
        self.gamma = base + 101 * 16 * MiB
        self.residual_out = base + 102 * 16 * MiB
        self.out = base + 103 * 16 * MiB
        self.q = base + 104 * 16 * MiB
        self.scales = base + 105 * 16 * MiB
        self.eps = 1e-6
        self.group = 128
        self.variant = 0

    def call(self):
        arr = (ctypes.c_void_p * max(1, len(self.partials)))(*self.partials) if self.partials is not None else None
        if self.quant:
            return L.farn_reduce_add_rmsnorm_quant_group_ex(
                arr, self.R, self.residual, self.gamma, self.eps, self.T, self.H, self.group,
                self.residual_out, self.out, self.q, self.scales, None, self.variant)
        return L.farn_reduce_add_rmsnorm_ex(arr, self.R, self.residual, self.gamma, self.eps, self.T,
                                            self.H, self.residual_out, self.out, None, self.variant)


def mk(**kw):
    quant = kw.pop("quant", False)
    dims = {k: kw.pop(k) for k in ("R", "T", "H") if k in kw}
    c = FakeCall(quant=quant, **dims)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


REJECTIONS = [
    # (description, FakeCall overrides, expected status)
    ("partials NULL", dict(partials=None), NULL),
    ("a partial NULL", dict(partials=[0x10_0000_0000, 0]), NULL),
    ("gamma NULL", dict(gamma=None), NULL),
    ("residual_out NULL", dict(residual_out=None), NULL),
    ("plain out NULL", dict(out=None), NULL),
    ("quant q NULL", dict(quant=True, q=None), NULL),
    ("quant scales NULL", dict(quant=True, scales=None), NULL),
    ("R = 0", dict(R=0, partials=[1 << 36]), SHAPE),
    ("R = 9", dict(R=9), SHAPE),
    ("T < 0", dict(T=-1), SHAPE),
    ("T huge", dict(T=1 << 41), SHAPE),
    ("H = 0", dict(H=0), SHAPE),
    ("H % 8", dict(H=260), SHAPE),
    ("H > max", dict(H=F.MAX_H + 8), SHAPE),
    ("quant group 64", dict(quant=True, group=64), SHAPE),
    ("quant H % 128", dict(quant=True, H=264), SHAPE),
    ("eps NaN", dict(eps=float("nan")), EPS),
    ("eps inf", dict(eps=float("inf")), EPS),
    ("eps < 0", dict(eps=-1e-6), EPS),
    ("partial misaligned", dict(partials=[0x10_0000_0000, 0x10_0000_0008 + 16 * MiB]), ALIGN),
    ("residual misaligned", dict(residual=0x20_0000_0004), ALIGN),
    ("gamma misaligned", dict(gamma=0x20_0000_0002), ALIGN),
    ("out misaligned", dict(out=0x20_0000_0008), ALIGN),
    ("q misaligned", dict(quant=True, q=0x20_0000_0008), ALIGN),
    ("scales misaligned", dict(quant=True, scales=0x20_0000_0002), ALIGN),
    ("out overlaps a partial", dict(out=0x10_0000_0000 + 16 * MiB + 256), ALIAS),
    ("residual_out overlaps gamma", dict(gamma=0x10_0000_0000 + 102 * 16 * MiB + 64), ALIAS),
    ("out overlaps residual_out", dict(out=0x10_0000_0000 + 102 * 16 * MiB + 1024), ALIAS),
    ("out == residual (not in place)", dict(out=0x10_0000_0000 + 100 * 16 * MiB), ALIAS),
    ("residual_out shifted into residual", dict(residual_out=0x10_0000_0000 + 100 * 16 * MiB + 16), ALIAS),
    ("q overlaps scales", dict(quant=True, scales=0x10_0000_0000 + 104 * 16 * MiB + 512), ALIAS),
    ("q overlaps a partial", dict(quant=True, q=0x10_0000_0000 + 16), ALIAS),
    ("variant 3", dict(variant=3), VARIANT),
    ("variant -1", dict(variant=-1), VARIANT),
]


@pytest.mark.parametrize("what,kw,want", REJECTIONS, ids=[r[0] for r in REJECTIONS])
def test_rejections(what, kw, want):
    assert mk(**kw).call() == want, what


def test_empty_call_enqueues_nothing():
    # T == 0 passes every check and returns OK without a launch (no GPU needed)
    assert mk(T=0).call() == OK
    assert mk(T=0, quant=True).call() == OK
    assert mk(T=0, residual=None).call() == OK


def test_quant_out_may_be_null_and_residual_may_be_null():
    # these are valid; with T == 0 they are accepted without a launch
    assert mk(T=0, quant=True, out=None).call() == OK
    assert mk(T=0, quant=True, residual=None).call() == OK


def test_validation_unit_is_hip_free():
    """The C-ABI layer compiles with plain g++ and no HIP headers."""
    src = os.path.join(os.path.dirname(F.LIB_PATH), "csrc", "farn_api.cpp")
    text = open(src).read()
    assert "hip/" not in text and "hip" not in re.findall(r"#include\s*[<\"]([^>\"]+)", text)
    subprocess.run(["g++", "-std=c++17", "-fsyntax-only", "-Wall", "-Wextra", "-Werror", src], check=True)


def reduce_call(partials=(0x10_0000_0000, 0x10_1000_0000), R=None, T=4, H=256, out=0x10_2000_0000):
    R = len(partials) if R is None else R
    arr = (ctypes.c_void_p * max(1, len(partials)))(*partials) if partials is not None else None
    return L.farn_reduce(arr, R, T, H, out, None)


def quant_call(x=0x10_0000_0000, T=4, H=256, group=128, q=0x10_1000_0000, scales=0x10_2000_0000):
    return L.farn_quant_group(x, T, H, group, q, scales, None)


UNFUSED_REJECTIONS = [
    ("reduce partials NULL", lambda: reduce_call(partials=None, R=2), NULL),
    ("reduce a partial NULL", lambda: reduce_call(partials=(0x10_0000_0000, 0)), NULL),
    ("reduce out NULL", lambda: reduce_call(out=0), NULL),
    ("reduce R = 9", lambda: reduce_call(R=9), SHAPE),
    ("reduce H % 8", lambda: reduce_call(H=12), SHAPE),
    ("reduce T < 0", lambda: reduce_call(T=-2), SHAPE),
    ("reduce misaligned out", lambda: reduce_call(out=0x10_2000_0008), ALIGN),
    ("reduce out overlaps a partial", lambda: reduce_call(out=0x10_1000_0000 + 512), ALIAS),
    ("quant x NULL", lambda: quant_call(x=0), NULL),
    ("quant q NULL", lambda: quant_call(q=0), NULL),
    ("quant scales NULL", lambda: quant_call(scales=0), NULL),
    ("quant group 64", lambda: quant_call(group=64), SHAPE),
    ("quant H % 128", lambda: quant_call(H=200), SHAPE),
    ("quant misaligned q", lambda: quant_call(q=0x10_1000_0004), ALIGN),
    ("quant misaligned scales", lambda: quant_call(scales=0x10_2000_0002), ALIGN),
    ("quant q overlaps x", lambda: quant_call(q=0x10_0000_0000 + 64), ALIAS),
    ("quant scales overlap q", lambda: quant_call(scales=0x10_1000_0000 + 64), ALIAS),
]


@pytest.mark.parametrize("what,fn,want", UNFUSED_REJECTIONS, ids=[r[0] for r in UNFUSED_REJECTIONS])
def test_unfused_rejections(what, fn, want):
    assert fn() == want, what


def test_unfused_empty():
    assert reduce_call(T=0, out=0) == OK
    assert quant_call(T=0, x=0, q=0, scales=0) == OK


def mx_call(H=256, q=0x10_3000_0000, scales=0x10_4000_0000, out=0x10_5000_0000, T=4):
    c = FakeCall(T=T, H=H)
    arr = (ctypes.c_void_p * 2)(*c.partials)
    return L.farn_reduce_add_rmsnorm_mxfp4_ex(arr, 2, c.residual, c.gamma, 1e-6, T, H, c.residual_out, out,
                                              q, scales, None, 0)


MX_REJECTIONS = [
    ("mxfp4 H % 32", lambda: mx_call(H=264), SHAPE),
    ("mxfp4 q NULL", lambda: mx_call(q=0), NULL),
    ("mxfp4 scales NULL", lambda: mx_call(scales=0), NULL),
    ("mxfp4 q misaligned", lambda: mx_call(q=0x10_3000_0008), ALIGN),
    ("mxfp4 q overlaps scales", lambda: mx_call(scales=0x10_3000_0000 + 100), ALIAS),
    ("mxfp4 scales overlap out", lambda: mx_call(scales=0x10_5000_0000 + 7), ALIAS),
]


@pytest.mark.parametrize("what,fn,want", MX_REJECTIONS, ids=[r[0] for r in MX_REJECTIONS])
def test_mxfp4_rejections(what, fn, want):
    assert fn() == want, what


def test_mxfp4_accepts_byte_aligned_scales_and_null_out():
    assert mx_call(T=0, scales=0x10_4000_0001, out=0) == OK


def test_option_bits():
    c = FakeCall(quant=True)
    c.variant = 0x100 | 1
    c.T = 0
    assert c.call() == OK
    c.variant = 0x200
    assert c.call() == VARIANT
    p = FakeCall()
    p.variant = 0x100  # column-major scales asked of the plain call
    assert p.call() == VARIANT


def test_column_major_scales_limit():
    """Column-major FP8 scales are addressed through one 32-bit range: T * H/128 * 4 bytes
    must stay below 2^31. At H = 32768 that is T < 2^21. Arrays are spaced 2^40 bytes apart,
    so the ranges do not overlap."""
    def tall(T):
        c = FakeCall(R=1, T=T, H=32768, quant=True)
        c.partials = [1 << 41]
        c.residual, c.gamma, c.residual_out = 2 << 41, 3 << 41, 4 << 41
        c.out, c.q, c.scales = 5 << 41, 6 << 41, 7 << 41
        c.variant = 0x100
        return c
    # (a call that passed every check would launch on these fake addresses: none is made)
    assert tall(1 << 21).call() == SHAPE
    assert tall(1 << 62).call() == SHAPE  # rejected by the T range check, no overflow


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU; asked for more it exits with a message before touching a GPU."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([os.sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=300)
    assert proc.returncode == 2 and "one GPU" in proc.stderr


def _bench_module():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(root, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_kernel_hash_ignores_comments_only(tmp_path, monkeypatch):
    """The hash that ties recorded HBM counters to the kernels changes with the code and not
    with its comments, blank lines or trailing blanks."""
    B = _bench_module()
    copies = []
    for src in B.KERNEL_SRCS:
        dst = tmp_path / os.path.basename(src)
        dst.write_text(open(src).read())
        copies.append(str(dst))
    monkeypatch.setattr(B, "KERNEL_SRCS", copies)
    base = B.kernel_hash()
    assert base == _bench_module().kernel_hash()  # the copies hash as the sources do
    text = open(copies[0]).read()
    commented = text.replace("constexpr int kMaxWaves = 16;",
                             "// a comment line\n\nconstexpr int kMaxWaves = 16;   /* and a block\n comment */  ")
    assert commented != text
    open(copies[0], "w").write(commented)
    assert B.kernel_hash() == base
    open(copies[0], "w").write(text.replace("constexpr int kMaxWaves = 16;", "constexpr int kMaxWaves = 32;"))
    assert B.kernel_hash() != base
    open(copies[0], "w").write(text)
    header = open(copies[1]).read()
    open(copies[1], "w").write(header.replace("0x1.24924ap-9f", "0x1.24924cp-9f"))
    assert B.kernel_hash() != base  # the device-math header is part of the kernels' code


def test_recorded_traffic_only_for_the_kernels_it_was_taken_on(tmp_path, monkeypatch):
    """roofline.traffic comes from counters recorded under a kernel hash; for any other hash
    (the kernels changed since) the bench reports none."""
    B = _bench_module()
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(B, "TRAFFIC_FILE", str(path))
    assert B.recorded_traffic("prefill_fp8") is None  # no file
    path.write_text(json.dumps({"prefill_fp8": {"kernel_sha": B.kernel_hash(), "bytes_per_launch": 123}}))
    assert B.recorded_traffic("prefill_fp8") == 123
    assert B.recorded_traffic("prefill") is None  # no record for that workload
    path.write_text(json.dumps({"prefill_fp8": {"kernel_sha": "0" * 16, "bytes_per_launch": 123}}))
    assert B.recorded_traffic("prefill_fp8") is None
    path.write_text("{not json")
    assert B.recorded_traffic("prefill_fp8") is None


def test_c_client_builds_against_header_alone(tmp_path):
    """A C program (not C++) that includes only include/farn.h and the HIP runtime API
    compiles warning-free with gcc and links against libfarn.so: the header is valid C."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "client")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic-errors",
                    "-Wno-error=pedantic", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
                    os.path.join(root, "tests", "c_abi_client.c"), "-o", exe,
                    f"-L{os.path.dirname(F.LIB_PATH)}", "-lfarn", f"-L{rocm}/lib", "-lamdhip64"],
                   check=True)
    assert os.path.getsize(exe) > 0


def test_binding_refuses_host_tensors():
    """The library takes plain pointers and cannot tell host memory from device memory: the
    binding refuses host tensors before calling it."""
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    g = torch.ones(256, dtype=torch.bfloat16)
    calls = [lambda: F.reduce_add_rmsnorm([x], None, g), lambda: F.reduce_add_rmsnorm_quant_group([x], None, g),
             lambda: F.reduce_add_rmsnorm_mxfp4([x], None, g), lambda: F.reduce([x]), lambda: F.quant_group(x)]
    for call in calls:
        with pytest.raises(ValueError, match="on the GPU"):
            call()


def test_package_refuses_to_load_without_its_library(tmp_path):
    """There is no fallback path: a copy of the package without libfarn.so raises on import."""
    import shutil
    pkg = os.path.dirname(F.__file__)
    dst = tmp_path / "tp_all_reduce_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    proc = subprocess.run(["python", "-c", "import tp_all_reduce_amd"], cwd=tmp_path,
                          capture_output=True, text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert proc.returncode != 0
    assert "ImportError" in proc.stderr and "no fallback" in proc.stderr, proc.stderr[-500:]


def test_product_never_uses_the_oracle():
    """The oracle is test infrastructure: nothing in the package (binding, host layer, kernels)
    imports, links or names it."""
    pkg = os.path.dirname(F.__file__)
    for root, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(root, name)).read()
                assert not re.search(r"oracle", text, re.I), name
