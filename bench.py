"""Bench of the fused reduce + residual-add + RMSNorm (+ FP8 group-128 quant) op on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--variant V]
                    [--kernels 1|2|3] [--cpu-budget S] [--no-secondary] [--no-sweep]

A step is one call of the FP8 entry point (reduce, residual add, bf16 round,
RMSNorm, per-group E4M3 quant, size-based dispatch) over one batch already resident
in HBM (with --kernels 2 or 3, the same step as the two- or three-kernel composition
the fused call replaces). The default workload is the prefill chunk R=8, T=8192, H=7168 with the bf16
output emitted: 1,352,400,896 algorithmic bytes per call, well beyond the 256 MB
Infinity Cache, so every call streams from HBM.

Prints ONE JSON line: value = algorithmic bytes per step / time per step (GB/s), with
the roofline of the kernel (HBM bound, 8 TB/s peak), the CPU oracle timed on host
cores on the same workload (its last pass also checks every output of the timed GPU
call: the parity field), the message-size sweep (R=8, H=8192, T=2..4096: us/call and
GB/s, cache-hot and streaming from HBM), and secondary figures for the decode shapes
(us/call).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tp_all_reduce_amd as F  # noqa: E402  (raises if the HIP library is not built)
from gen import CONFIGS, SWEEP_T, Config, make_inputs, sweep_config  # noqa: E402

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak, AMD's published figure
METRIC = "effective HBM GB/s (% of MI355X peak) and µs/call of fused reduce+RMSNorm"
KERNEL_SRCS = [os.path.join(ROOT, "tp_all_reduce_amd", "csrc", f) for f in ("farn_kernels.hip", "farn_device_math.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

WORKLOADS = {
    # name: (config, quant, emit_out)
    "prefill_fp8": (CONFIGS["prefill"], True, True),
    "prefill": (CONFIGS["prefill"], False, True),
    "decode_ds": (CONFIGS["decode_ds"], False, True),
    "decode_fp8": (CONFIGS["decode_fp8"], True, True),
    "tiny": (CONFIGS["tiny"], False, True),
    "prefill_mxfp4": (CONFIGS["prefill"], "mxfp4", True),
    "decode_ds_mxfp4": (CONFIGS["decode_ds"], "mxfp4", True),
    # the FP8 call with the bf16 output off (emit_bf16 false): its own, smaller byte count
    "decode_fp8_noout": (CONFIGS["decode_fp8"], True, False),
    "prefill_fp8_noout": (CONFIGS["prefill"], True, False),
}
for _T in SWEEP_T:
    WORKLOADS[f"sweep_T{_T}"] = (sweep_config(_T), False, True)

VARIANT_NAMES = {"auto": F.VARIANT_AUTO, "wide": F.VARIANT_WIDE, "narrow": F.VARIANT_NARROW,
                 "latency": F.VARIANT_WIDE, "bandwidth": F.VARIANT_NARROW}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """sha256[:16] of the kernels' source code (the kernel file and its device-math header):
    comments, blank lines and trailing blanks removed, so that recorded counters stay tied to
    the code they were taken on and not to its comments."""
    import re
    text = "".join(open(p).read() for p in KERNEL_SRCS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def describe(cfg, quant, emit_out):
    kind = ", MXFP4 (32-channel E8M0 blocks)" if quant == "mxfp4" else ", FP8 group-128 quant"
    q = kind + (" + bf16 out" if emit_out else ", bf16 out not written") if quant else ""
    return f"{cfg.what}: R={cfg.R} T={cfg.T} H={cfg.H}{q}"


class Bufs:
    """One set of device inputs and outputs for a workload."""

    def __init__(self, d, dev, quant, emit_out):
        from tests.parity import to_dev_bf16
        self.R, self.T, self.H = d["R"], d["T"], d["H"]
        self.P = [to_dev_bf16(d["partials"][r], dev) for r in range(self.R)]
        self.res = to_dev_bf16(d["residual"], dev)
        self.g = to_dev_bf16(d["gamma"], dev)
        self.quant, self.emit_out = quant, emit_out
        self.kernels = 1  # 2 or 3: call() runs the unfused composition of the FP8 step
        self.alloc_outputs(dev)

    def alloc_outputs(self, dev):
        T, H = self.T, self.H
        self.ro = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if (self.emit_out or not self.quant) else None
        if self.quant == "mxfp4":
            self.q = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
            self.s = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        else:
            self.q = torch.empty((T, H), dtype=torch.uint8, device=dev) if self.quant else None
            self.s = torch.empty((T, H // 128), dtype=torch.float32, device=dev) if self.quant else None

    def clone(self, dev):
        c = object.__new__(Bufs)
        c.R, c.T, c.H, c.quant, c.emit_out = self.R, self.T, self.H, self.quant, self.emit_out
        c.kernels = self.kernels
        c.P = [p.clone() for p in self.P]
        c.res, c.g = self.res.clone(), self.g.clone()
        c.alloc_outputs(dev)
        return c

    def call_2kernel(self, variant=0):
        """Fused AR + RMSNorm, then the quant alone (the pages' two-kernel fallback)."""
        F.reduce_add_rmsnorm(self.P, self.res, self.g, 1e-6, residual_out=self.ro, out=self.out,
                             variant=variant)
        F.quant_group(self.out, q=self.q, scales=self.s)

    def call_3kernel(self, variant=0):
        """All-reduce alone, add + RMSNorm, then the quant alone (three kernels)."""
        if not hasattr(self, "ar"):
            self.ar = torch.empty_like(self.ro)
        F.reduce(self.P, out=self.ar)
        F.reduce_add_rmsnorm([self.ar], self.res, self.g, 1e-6, residual_out=self.ro, out=self.out,
                             variant=variant)
        F.quant_group(self.out, q=self.q, scales=self.s)

    def call(self, variant):
        if self.kernels == 2:
            return self.call_2kernel(variant)
        if self.kernels == 3:
            return self.call_3kernel(variant)
        if self.quant == "mxfp4":
            F.reduce_add_rmsnorm_mxfp4(self.P, self.res, self.g, 1e-6, emit_out=self.emit_out,
                                       residual_out=self.ro, out=self.out, q=self.q, scales=self.s,
                                       variant=variant)
        elif self.quant:
            F.reduce_add_rmsnorm_quant_group(self.P, self.res, self.g, 1e-6, emit_out=self.emit_out,
                                             residual_out=self.ro, out=self.out, q=self.q, scales=self.s,
                                             variant=variant)
        else:
            F.reduce_add_rmsnorm(self.P, self.res, self.g, 1e-6, residual_out=self.ro, out=self.out,
                                 variant=variant)


def nbytes(cfg, quant, emit_out):
    if quant == "mxfp4":
        th = cfg.T * cfg.H
        return cfg.nbytes_plain + th // 2 + th // 32 - (0 if emit_out else th * 2)
    return cfg.nbytes_quant(emit_out) if quant else cfg.nbytes_plain


def time_calls(sets, variant, steps, warmup, method="call"):
    """Average ms per call over `steps` back-to-back calls, rotating over `sets`, timed with
    events on the stream the kernels are launched on (torch's current stream)."""
    for i in range(warmup):
        getattr(sets[i % len(sets)], method)(variant)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        getattr(sets[i % len(sets)], method)(variant)
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return start.elapsed_time(end) / steps, wall / steps


def time_graph(sets, variant, calls, replays, method="call"):
    """Average ms per call with the launches captured in a HIP graph (the way a serving loop
    issues decode steps), so host launch overhead is out of the measurement. One graph holds
    `calls` back-to-back calls rotating over `sets`; it is replayed `replays` times."""
    for b in sets:
        getattr(b, method)(variant)  # warm the code objects before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            getattr(sets[i % len(sets)], method)(variant)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (replays * calls)
    del g
    return ms


def median_graph(sets, variant, calls, replays, method="call", runs=3):
    """Median of `runs` time_graph measurements: decode calls are bound by instruction
    issue and memory latency on a few compute units and move with the shader clock from one
    measurement to the next, by up to 15 %."""
    return statistics.median(time_graph(sets, variant, calls, replays, method) for _ in range(runs))


def parity_report(ref, bufs, quant, emit_out):
    """GPU outputs of the timed call against reference outputs `ref` = (residual_out, out,
    q, scales) as the oracle returns them, over every row."""
    from tests.parity import compare_bf16, compare_fp8, from_dev_bf16, within_tolerance
    r_ro, r_out = ref[0], ref[1]
    mx = fp8 = None
    if quant == "mxfp4":
        from tests.parity import compare_mxfp4, mxfp4_within_tolerance
        mx = compare_mxfp4(bufs.q.cpu().numpy(), ref[2], bufs.s.cpu().numpy(), ref[3])
    elif quant:
        fp8 = compare_fp8(bufs.q.cpu().numpy(), ref[2], bufs.s.cpu().numpy(), ref[3])
    rep_ro = compare_bf16("residual_out", from_dev_bf16(bufs.ro), r_ro)
    rep_out = compare_bf16("out", from_dev_bf16(bufs.out), r_out) if bufs.out is not None else None
    ok, why = within_tolerance(rep_ro, rep_out, fp8)
    if mx is not None:
        ok2, why2 = mxfp4_within_tolerance(mx)
        ok, why = ok and ok2, "; ".join(w for w in (why, why2) if w)
    return {"ok": ok, "why": why, "rows_checked": int(bufs.T), "against": "oracle, all rows",
            "residual_out_bit_diffs": rep_ro["n_bit_diff"],
            "out_max_rel_err": None if rep_out is None else rep_out["max_rel_err"],
            "out_bit_diffs": None if rep_out is None else rep_out["n_bit_diff"],
            "fp8_code_diffs": None if fp8 is None else fp8["n_code_diff"],
            "scale_max_rel_err": None if fp8 is None else fp8["max_scale_rel_err"]}


def cpu_baseline(d, cfg, quant, emit_out, budget_s, bufs=None):
    """The oracle as it stands, on the host cores, over whole passes of the workload until
    about budget_s seconds have been spent. With `bufs` (the timed GPU call's buffers), the
    last pass's outputs are also compared with the GPU's over every row: returns
    (baseline, parity report or None)."""
    import oracle
    threads, affinity, share = oracle_threads()
    passes, spent, ref = 0, 0.0, None
    while spent < budget_s:
        t0 = time.perf_counter()
        if quant == "mxfp4":
            ref = oracle.reduce_add_rmsnorm_mxfp4(d["partials"], d["residual"], d["gamma"], 1e-6, emit_out,
                                                  nthreads=threads)
        elif quant:
            ref = oracle.reduce_add_rmsnorm_quant_group(d["partials"], d["residual"], d["gamma"], 1e-6, 128,
                                                        emit_out, nthreads=threads)
        else:
            ref = oracle.reduce_add_rmsnorm(d["partials"], d["residual"], d["gamma"], 1e-6, nthreads=threads)
        spent += time.perf_counter() - t0
        passes += 1
    gbps = nbytes(cfg, quant, emit_out) * passes / spent / 1e9
    # one thread on a sample of rows, for the per-core figure
    rows = min(cfg.T, 256)
    P1, r1 = d["partials"][:, :rows], d["residual"][:rows]
    t0 = time.perf_counter()
    if quant == "mxfp4":
        oracle.reduce_add_rmsnorm_mxfp4(P1, r1, d["gamma"], 1e-6, emit_out, nthreads=1)
    elif quant:
        oracle.reduce_add_rmsnorm_quant_group(P1, r1, d["gamma"], 1e-6, 128, emit_out, nthreads=1)
    else:
        oracle.reduce_add_rmsnorm(P1, r1, d["gamma"], 1e-6, nthreads=1)
    one = time.perf_counter() - t0
    if bufs is not None and bufs.kernels == 3:
        # the three-kernel composition rounds the all-reduce to bf16 before the residual add:
        # its reference is the oracle's composition of the same three blocks
        ar = oracle.reduce(d["partials"])
        r_ro, r_out = oracle.reduce_add_rmsnorm(ar[None], d["residual"], d["gamma"], 1e-6, nthreads=threads)
        ref = (r_ro, r_out) + oracle.quant_group(r_out)
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "threads": threads,
            "cores_in_affinity_mask": affinity, "cpu_share": share, "kind": "oracle",
            "sample": f"{passes} full pass(es) over the workload ({cfg.T} rows), {spent:.1f} s",
            "ms_per_call": round(spent / passes * 1e3, 2),
            "one_thread": {"GBps": round(nbytes(cfg, quant, emit_out) * rows / cfg.T / one / 1e9, 3),
                           "sample": f"{rows} rows, {one:.2f} s"},
            "cpu_model": cpu_model()}, (None if bufs is None else parity_report(ref, bufs, quant, emit_out))


def oracle_threads():
    """Threads for the oracle: every core in this process's affinity mask, capped at the CPU
    share the environment states (OMP_NUM_THREADS, when set), since a shared host's mask can
    list more cores than this process is meant to use. Returns (threads, cores in the mask,
    the stated share or None)."""
    affinity = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    share = int(share) if share and share.isdigit() and int(share) > 0 else None
    return (min(affinity, share) if share else affinity), affinity, share


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_ceiling(dev, reps=5):
    """Streaming references beside the published peak, each moving 1 GiB in and 1 GiB out and
    timed with events (median of reps): torch's device copy, and this library's all-reduce of a
    single rank (farn_reduce with R = 1: a bf16 copy through the kernels' own access pattern)."""
    def median_time(fn):
        fn()
        times = []
        for _ in range(reps):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            fn()
            end.record()
            torch.cuda.synchronize()
            times.append(start.elapsed_time(end) * 1e-3)
        return statistics.median(times)
    src = torch.empty((1 << 16, 1 << 13), dtype=torch.bfloat16, device=dev)   # 1 GiB
    src.view(torch.int16).random_(-0x4000, 0x4000)                            # finite bf16 patterns
    dst = torch.empty_like(src)
    out = {}
    for name, fn in (("torch_copy", lambda: dst.copy_(src)), ("farn_reduce_R1", lambda: F.reduce([src], out=dst))):
        gbps = 2 * (1 << 30) / median_time(fn) / 1e9
        out[name] = {"GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    out["what"] = f"1 GiB read + 1 GiB written per call, median of {reps}"
    return out


def recorded_traffic(workload):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sha") != kernel_hash():
        return None  # counters were taken on another version of the kernel
    return rec.get("bytes_per_launch")


def secondary(dev, steps):
    """Decode shapes in us/call: eager (one Python call per launch, host-bound), and graph
    replay, hot (one buffer set, cache-resident) and cold (sets rotated over >= 1 GiB, so
    every call streams from HBM); plus the plain, MXFP4 and bf16-output-free FP8 prefill calls."""
    out = {}
    for name in ("decode_ds", "decode_fp8", "decode_fp8_noout"):
        cfg, quant, emit = WORKLOADS[name]
        d = make_inputs(cfg)
        b = Bufs(d, dev, quant, emit)
        nb = nbytes(cfg, quant, emit)
        eager, _ = time_calls([b], F.VARIANT_AUTO, steps, 20)
        hot = median_graph([b], F.VARIANT_AUTO, 200, 10)
        k = max(1, -(-(1 << 30) // nb))
        sets = [b] + [b.clone(dev) for _ in range(k - 1)]
        calls = k * max(1, 200 // k)
        cold = median_graph(sets, F.VARIANT_AUTO, calls, max(2, 2000 // calls))
        out[name] = {"us_per_call_graph_hot": round(hot * 1e3, 2),
                     "us_per_call_graph_cold": round(cold * 1e3, 2),
                     "us_per_call_eager": round(eager * 1e3, 2),
                     "GBps_graph_cold": round(nb / (cold * 1e-3) / 1e9, 1), "rotation_sets": k,
                     "bytes_per_call": nb}
        del sets, b
        torch.cuda.empty_cache()
    for name in ("prefill", "prefill_mxfp4", "prefill_fp8_noout"):
        cfg, quant, emit = WORKLOADS[name]
        b = Bufs(make_inputs(cfg), dev, quant, emit)
        nb = nbytes(cfg, quant, emit)
        ms, _ = time_calls([b], F.VARIANT_AUTO, 50, 20)
        out[name] = {"us_per_call": round(ms * 1e3, 2), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                     "bytes_per_call": nb}
        del b
        torch.cuda.empty_cache()
    cfg, quant, emit = WORKLOADS["decode_ds_mxfp4"]
    b = Bufs(make_inputs(cfg), dev, quant, emit)
    out["decode_ds_mxfp4"] = {"us_per_call_graph_hot": round(median_graph([b], F.VARIANT_AUTO, 200, 10) * 1e3, 2)}
    out["launch_floor"] = launch_floor(dev)
    return out


class _Fill:
    """A one-element fill: torch's smallest kernel, as a bare-launch reference."""

    def __init__(self, dev):
        self.x = torch.zeros(1, dtype=torch.float32, device=dev)

    def call(self, variant):
        self.x.fill_(1.0)


def launch_floor(dev):
    """What a decode call costs before it moves any data, by graph replay (median of 3),
    cache-hot: a bare launch (a one-element fill), the fused call on one row of one wave
    (R = 1, T = 1, H = 512), and one row of the decode shape (R = 8, T = 1, H = 7168: the
    dependent chain of loads, fold, row statistics and stores that every row of a decode
    call runs, on one compute unit)."""
    res = {"bare_launch_us": round(median_graph([_Fill(dev)], 0, 200, 10) * 1e3, 2)}
    for label, (R, T, H) in (("fused_one_wave_us", (1, 1, 512)), ("fused_one_decode_row_us", (8, 1, 7168))):
        cfg = Config(label, R=R, T=T, H=H, quant=(False,))
        b = Bufs(make_inputs(cfg), dev, False, True)
        res[label] = round(median_graph([b], F.VARIANT_AUTO, 200, 10) * 1e3, 2)
        del b
    res["what"] = "graph replay, cache-hot, median of 3; us per call"
    return res


def sweep(dev):
    """The message-size sweep (R = 8, H = 8192, T = 2 .. 4096, plain call) in us/call by graph
    replay: hot (one buffer set, cache-resident) and cold (sets rotated over >= 1 GiB, so every
    call streams from HBM rather than the 256 MB last-level cache), with the cold rate, and
    both launch shapes forced (hot) beside the one the dispatch rule picks."""
    out = {"what": "R=8, H=8192, plain call, shape chosen by the dispatch rule; graph replay, median of 3; "
                   "hot = one buffer set (cache-resident), cold = sets rotated over >= 1 GiB (streams from HBM); "
                   "forced_hot_us = both launch shapes forced, hot",
           "peak_GBps": PEAK_HBM_GBPS, "points": []}
    for T in SWEEP_T:
        cfg = sweep_config(T)
        b = Bufs(make_inputs(cfg), dev, False, True)
        nb = nbytes(cfg, False, True)
        hot = median_graph([b], F.VARIANT_AUTO, 200, 10)
        # both launch shapes forced, timed right after (hot), as the dispatch rule was set; before
        # the cold leg, whose rotation over 1 GiB leaves the caches in another state
        forced = {name: round(median_graph([b], v, 200, 10) * 1e3, 2)
                  for name, v in (("wide", F.VARIANT_WIDE), ("narrow", F.VARIANT_NARROW))}
        k = max(1, -(-(1 << 30) // nb))
        sets = [b] + [b.clone(dev) for _ in range(k - 1)]
        calls = k * max(1, 200 // k)
        cold = median_graph(sets, F.VARIANT_AUTO, calls, max(2, 2000 // calls))
        gbps = nb / (cold * 1e-3) / 1e9
        pt = {"T": T, "bytes": nb, "hot_us": round(hot * 1e3, 2), "cold_us": round(cold * 1e3, 2),
              "cold_GBps": round(gbps, 1), "cold_pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 1),
              "shape": {1: "wide", 2: "narrow"}[F.select_variant(cfg.R, T, cfg.H, False)],
              "forced_hot_us": forced, "rotation_sets": k}
        out["points"].append(pt)
        log(f"sweep T={T}: {pt}")
        del sets, b
        torch.cuda.empty_cache()
    return out


def shape_points(n, seed):
    """n random call shapes, seeded: R in 2..8, H a multiple of 128 in 1024..8192, T log-uniform
    over 16..8192, plain / FP8 / MXFP4 calls (45 / 35 / 20 %), at most 3 GiB of inputs and
    outputs per call."""
    rng = np.random.default_rng(seed)
    pts = []
    while len(pts) < n:
        R = int(rng.integers(2, 9))
        H = int(rng.integers(8, 65)) * 128
        T = int(np.exp(rng.uniform(np.log(16), np.log(8192))))
        u = rng.random()
        quant = False if u < 0.45 else (True if u < 0.8 else "mxfp4")
        if (R + 3) * T * H * 2 <= (3 << 30):
            pts.append((R, H, T, quant))
    return pts


def shapes_check(dev, n, seed, cold=False):
    """Both launch shapes forced at n random call shapes (graph replay, interleaved, median of
    5; cache-hot for calls up to 128 MiB, buffer sets rotated over >= 1 GiB above, or rotated
    at every size with cold=True, as when each call's inputs stream from HBM), and what the
    automatic rule loses at each against the faster of the two."""
    points = []
    for (R, H, T, quant) in shape_points(n, seed):
        cfg = Config("shape", R=R, T=T, H=H, quant=(False,))
        b = Bufs(make_inputs(cfg, seed=R * 1000 + T + H), dev, quant, True)
        nb = nbytes(cfg, quant, True)
        us_est = max(3.0, nb / 6.0e12 * 1e6)
        if nb <= (128 << 20) and not cold:
            sets, calls, replays = [b], max(10, min(200, int(8000 / us_est))), 5
        else:
            k = max(1, -(-(1 << 30) // nb))
            sets = [b] + [b.clone(dev) for _ in range(k - 1)]
            calls = k * max(1, int(8000 / us_est) // k)
            replays = max(2, int(20000 / (us_est * calls)))
        t = {F.VARIANT_WIDE: [], F.VARIANT_NARROW: []}
        for _ in range(5):
            for v in t:
                t[v].append(time_graph(sets, v, calls, replays))
        w, nr = (statistics.median(t[v]) * 1e3 for v in (F.VARIANT_WIDE, F.VARIANT_NARROW))
        auto = F.select_variant(R, T, H, quant)
        pt = {"R": R, "H": H, "T": T, "quant": {False: "plain", True: "fp8"}.get(quant, quant),
              "wide_us": round(w, 3), "narrow_us": round(nr, 3), "auto": {1: "wide", 2: "narrow"}[auto],
              "auto_loss_pct": round(100 * ((w if auto == F.VARIANT_WIDE else nr) / min(w, nr) - 1), 2)}
        points.append(pt)
        log(f"shapes: {pt}")
        del sets, b
        torch.cuda.empty_cache()
    losses = sorted((p["auto_loss_pct"] for p in points), reverse=True)
    return {"what": "both launch shapes at random call shapes; auto_loss_pct = the automatic rule's "
                    "time over the faster shape's, in per cent",
            "inputs": "streaming from HBM at every size" if cold else "cache-hot up to 128 MiB, streaming above",
            "seed": seed, "points": len(points), "auto_loss_mean_pct": round(statistics.mean(losses), 3),
            "auto_loss_max_pct": losses[0], "points_over_5pct": sum(1 for x in losses if x > 5),
            "always_wide_loss_mean_pct": round(statistics.mean(
                100 * (p["wide_us"] / min(p["wide_us"], p["narrow_us"]) - 1) for p in points), 3),
            "detail": points}


def unfused(dev):
    """What fusion buys: the FP8 step as one kernel (fused), two (fused AR+RMSNorm, then quant)
    and three (all-reduce, add+RMSNorm, quant), as the sglang benchmark compares them. Prefill:
    eager, streaming from HBM. Decode: graph replay, cache-hot."""
    res = {}
    for name in ("prefill_fp8", "decode_fp8", "decode_ds"):
        cfg = WORKLOADS[name][0]
        b = Bufs(make_inputs(cfg), dev, True, True)
        rec = {}
        for method, label in (("call", "1_kernel"), ("call_2kernel", "2_kernel"), ("call_3kernel", "3_kernel")):
            if name.startswith("prefill"):
                ms, _ = time_calls([b], F.VARIANT_AUTO, 30, 3, method=method)
            else:
                ms = median_graph([b], F.VARIANT_AUTO, 100, 10, method=method)
            rec[label + "_us"] = round(ms * 1e3, 2)
        rec["speedup_vs_3_kernel"] = round(rec["3_kernel_us"] / rec["1_kernel_us"], 2)
        rec["speedup_vs_2_kernel"] = round(rec["2_kernel_us"] / rec["1_kernel_us"], 2)
        res[name] = rec
        del b
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_fp8", choices=sorted(WORKLOADS))
    ap.add_argument("--variant", default="auto", choices=sorted(VARIANT_NAMES))
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run the step back to back for this long before the warmup steps, so the "
                         "GPU clocks reach their sustained state (the first ~100 calls run slower)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the message-size sweep (R=8, H=8192, T=2..4096), hot and cache-cold")
    ap.add_argument("--cold", action="store_true",
                    help="rotate the timed calls over buffer sets of >= 1 GiB in all (every call streams "
                         "from HBM); for workloads that fit the last-level cache")
    ap.add_argument("--kernels", type=int, default=1, choices=(1, 2, 3),
                    help="time the FP8 step as the fused call (1), fused AR+RMSNorm then the quant (2), "
                         "or all-reduce, add+RMSNorm, quant (3); FP8 workloads only")
    ap.add_argument("--shapes", type=int, default=0, metavar="N",
                    help="instead of the bench: time both launch shapes at N random call shapes and "
                         "report what the automatic rule loses against the faster one (one JSON line)")
    ap.add_argument("--shapes-seed", type=int, default=13)
    ap.add_argument("--shapes-cold", action="store_true",
                    help="with --shapes: time every call with its inputs streaming from HBM")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one torch copy of 1 GiB (for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.shapes > 0:
        print(json.dumps({"shapes_check": shapes_check(dev, args.shapes, args.shapes_seed, args.shapes_cold)}),
              flush=True)
        return
    cfg, quant, emit_out = WORKLOADS[args.workload]
    variant = VARIANT_NAMES[args.variant]
    if args.kernels != 1 and not (quant is True and emit_out):
        print("--kernels 2/3 time the FP8 step with the bf16 output: pick an FP8 workload", file=sys.stderr)
        sys.exit(2)

    log(f"generating {args.workload}")
    d = make_inputs(cfg)
    bufs = Bufs(d, dev, quant, emit_out)
    bufs.kernels = args.kernels
    nb = nbytes(cfg, quant, emit_out)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written")
        del src, dst

    # the buffer sets the timed loop rotates over: one, or (--cold) enough for >= 1 GiB, so
    # that every call streams its inputs from HBM rather than the 256 MB last-level cache
    sets = [bufs]
    if args.cold:
        sets += [bufs.clone(dev) for _ in range(max(1, -(-(1 << 30) // nb)) - 1)]
    settle_calls = 0
    if args.settle_ms > 0:
        t_end = time.perf_counter() + args.settle_ms / 1e3
        while time.perf_counter() < t_end:
            for i in range(10):
                sets[(settle_calls + i) % len(sets)].call(variant)
            settle_calls += 10
            torch.cuda.synchronize()
    log(f"timing {args.steps} steps after {settle_calls} settle calls and {args.warmup} warmup "
        f"over {len(sets)} buffer set(s)")
    ms, wall_ms = time_calls(sets, variant, args.steps, args.warmup)
    del sets[1:]
    gbps = nb / (ms * 1e-3) / 1e9
    ran = F.select_variant(cfg.R, cfg.T, cfg.H, quant) if variant == F.VARIANT_AUTO else variant
    traffic = recorded_traffic(args.workload) if args.kernels == 1 else None
    result = {
        "metric": METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(cfg, quant, emit_out), "name": args.workload, "R": cfg.R,
                   "T": cfg.T, "H": cfg.H, "quant": quant, "emit_bf16_out": emit_out,
                   "variant": {1: "wide", 2: "narrow"}[ran], "bytes_per_step": nb,
                   "kernels_per_step": args.kernels, "buffer_sets": "rotated over >= 1 GiB" if args.cold else 1,
                   "seed": cfg.seed},
        "us_per_call": round(ms * 1e3, 2), "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 1),
        "settle_calls": settle_calls,
        "wall_us_per_call": round(wall_ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1),
                     "traffic_source": None if traffic is None else (
                         "recorded rocprofv3 FETCH_SIZE + WRITE_SIZE counters of this kernel source (sha256[:16] "
                         f"{kernel_hash()}), scaled by a 1 GiB copy, in profiles/traffic.json; HBM bytes per "
                         "launch / this run's time per launch"),
                     "kernel": "farn_rows (" + {1: "wide", 2: "narrow"}[ran] + " shape)"
                               + ("" if args.kernels == 1 else f" + {args.kernels - 1} unfused kernel(s)"),
                     "kernel_sha": kernel_hash(),
                     "algorithmic_bytes_per_launch": nb,
                     "hbm_bytes_per_launch": traffic},
        "parity": None,
    }
    if not args.no_secondary:
        log("copy ceiling")
        result["copy_ceiling"] = copy_ceiling(dev)
    if args.cpu_budget > 0:
        log("timing the CPU oracle (its last pass also checks the timed call's outputs)")
        result["cpu_baseline"], result["parity"] = cpu_baseline(
            d, cfg, quant, emit_out, args.cpu_budget, None if args.no_parity else bufs)
        log(f"parity: {result['parity']}")
        if result["parity"] is not None and not result["parity"]["ok"]:
            print(json.dumps({"metric": METRIC, "error": "parity check failed", "parity": result["parity"]}))
            sys.exit(1)
    if not args.no_secondary:
        del bufs
        torch.cuda.empty_cache()
        log("secondary decode shapes")
        result["secondary"] = secondary(dev, 200)
        log("unfused compositions")
        result["secondary"]["unfused_fp8"] = unfused(dev)
    if not args.no_sweep:
        log("message-size sweep")
        result["sweep"] = sweep(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
