#!/usr/bin/env python3
"""Benchmark of the FP32 GEMM hot path on one MI355X.

A step is one C = A.B of the 4096 x 4096 x 4096 workload (A, B, C row-major,
entries uniform[-1, 1], seed 1) with the operands already resident in HBM.
W untimed warm-up steps, then exactly K timed steps bracketed by device
synchronisation; rank 0 prints one JSON line:

  value      TFLOPS = 2*M*N*K * K_steps / wall time
  roofline   the GEMM kernel's own average duration (HIP events on the
             stream it is launched on) against the FP32 matrix peak
  cpu_baseline  the CPU oracle timed on a bounded row sample of the same
             workload on this host's cores

Before the W warm-up steps the step runs untimed for ``--settle-s`` seconds
of GPU time (default 0.25 s): under sustained matrix-core load the engine
clock ramps for about 0.1 s, and a few warm-up steps of a 1 ms kernel do not
cover that.  The timed region is still exactly K steps.

``configs`` in the line: the other workloads of the metric (256^3, 4096^3
with column-major B, the ragged 5003 x 4097 x 2049, the FFN and the skinny
16 x 4096 x 4096 shapes), each timed in the same run with its own kernel
average (the skinny one over 8 rotating operand sets, so B comes from HBM).

Other workloads: ``--workload ffn`` etc. (see workloads.WORKLOADS);
``--all`` also appends a line per workload to the file given by ``--all-out``.
``--layout-a col`` stores A column-major; ``--epilogue relu|gelu|bias``
times the fused linear-layer epilogue act(A.B + bias) (``bias``: no
activation).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HEADLINE = "sq4096"
METRIC = "FP32 GEMM TFLOPS (2MNK/t) and % of MI355X FP32 matrix peak at 4096^3"

# HBM traffic of the GEMM kernel per launch, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch) over
#   bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline --calibrate-copy 512
# scaled by what the same counters read for the 512 MiB elementwise copy in
# that run (FETCH_SIZE 262161 KiB -> x2.000, WRITE_SIZE 524288 KiB -> x1.000);
# the summary is profiles/dma_256x256x16_w4x2_s4_sq4096_counters.md.
# Valid only for the kernel sources they were taken on: the entry carries the
# SHA-1 of the tiled-kernel sources, and the field is null when they differ.
TRAFFIC_SOURCES = ("device_common.hpp", "mfma_gemm.hpp", "mfma_dma_gemm.hpp")
TRAFFIC_COUNTERS = {
    "sq4096": {"kernel": "dma_256x256x16_w4x2_s4",
               "sources_sha1": "72a0065f3a3f4f9925b330e49eea83347ac410e9",
               "fetch_kib": 196677.8, "write_kib": 65536.0,
               "fetch_factor": 2.000, "write_factor": 1.000},
}


def kernel_sources_sha1():
    import hashlib

    h = hashlib.sha1()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "dense_gemm_optimisation_fp32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes(workload, kernel):
    """Counter-derived HBM bytes per launch, or None when not measured for
    this kernel as it stands."""
    t = TRAFFIC_COUNTERS.get(workload)
    if not t or t["kernel"] != kernel or t["sources_sha1"] != kernel_sources_sha1():
        return None
    return t["fetch_kib"] * 1024 * t["fetch_factor"] + t["write_kib"] * 1024 * t["write_factor"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=200,
                   help="untimed steps first; the GPU clock needs ~0.1 s of load to settle")
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--variant", type=int, default=None, help="force a kernel variant")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the baseline")
    p.add_argument("--all", action="store_true", help="also time every workload")
    p.add_argument("--all-out", default="bench_all.jsonl")
    p.add_argument("--rotate", type=int, default=1,
                   help="cycle through this many operand sets (defeats the Infinity Cache for small workloads)")
    p.add_argument("--layout-a", choices=["row", "col"], default="row")
    p.add_argument("--epilogue", choices=["none", "bias", "relu", "gelu"], default="none")
    p.add_argument("--settle-s", type=float, default=0.25,
                   help="untimed GPU time before the warm-up steps, so the engine clock has ramped")
    p.add_argument("--no-configs", action="store_true", help="skip the other workloads of the metric")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="first run one elementwise copy of MIB MiB (reads and writes MIB MiB), "
                        "the reference kernel for scaling the FETCH_SIZE/WRITE_SIZE counters")
    return p.parse_args()


class ClockSampler:
    """Samples the engine clock the driver reports (the current level of
    pp_dpm_sclk in sysfs, in MHz) every few milliseconds from a thread, to
    turn a fraction of the 2.4 GHz peak into one of the peak at the clock the
    kernel actually ran at.  Only on a host with one GPU in sysfs, so that
    the clock is the measured GPU's; otherwise no samples."""

    def __init__(self, period_s=0.002):
        import glob

        paths = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
        self.path = paths[0] if len(paths) == 1 else None
        self.period = period_s
        self.samples = []
        self._stop = None
        self._thread = None

    def _read(self):
        import re

        with open(self.path) as f:
            for line in f:
                if "*" in line:
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    return int(m.group(1)) if m else None
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except OSError:
                return
            if v:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        import threading

        if self.path:
            self._stop = threading.Event()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()

    def mean_mhz(self):
        return sum(self.samples) / len(self.samples) if self.samples else None


def time_workload(name, steps, warmup, variant=None, rotate=1, layout_a=0, epilogue="none", settle_s=0.0):
    import numpy as np
    import torch

    import dense_gemm_optimisation_fp32_amd as g
    from dense_gemm_optimisation_fp32_amd import perfmodel as pm
    from workloads import WORKLOADS, epilogue_operands, random_operands, workload_operands

    w = WORKLOADS[name]
    if layout_a == 0:
        A, B = workload_operands(w)
    else:
        A, B = random_operands(w.m, w.n, w.k, w.layout_b, w.dist, w.seed, layout_a=layout_a)
    dev = torch.device("cuda", 0)
    lda = w.k if layout_a == 0 else w.m
    ldb = w.n if w.layout_b == 0 else w.k
    # `rotate` distinct operand sets, used in turn, so that a workload smaller
    # than the 256 MB Infinity Cache is still read from HBM at every step.
    sets = []
    for r in range(rotate):
        dA = torch.from_numpy(A).to(dev)
        dB = torch.from_numpy(B).to(dev)
        dC = torch.empty((w.m, w.n), dtype=torch.float32, device=dev)
        sets.append((dA, dB, dC))
    ptrs = [(a.data_ptr(), b.data_ptr(), c.data_ptr()) for a, b, c in sets]
    fused = epilogue != "none"
    plan = g.get_plan(w.m, w.n, w.k, w.layout_b, lda, ldb, w.n, variant, 0, layout_a, 1 if fused else 0)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    if fused:
        bias = torch.from_numpy(epilogue_operands(1, w.n, seed=w.seed + 2000)[1]).to(dev)
        act = {"bias": 0, "relu": 1, "gelu": 2}[epilogue]

        def plan_run(a, b, c, st):
            plan.run_ex(a, b, c, 1.0, 0.0, bias.data_ptr(), act, st)
    else:
        plan_run = plan.run

    # Clock settle: launches until settle_s of GPU time has passed (timed
    # with one event pair around a first launch), then the warm-up steps.
    if settle_s > 0:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plan_run(*ptrs[0], sh)
        e1.record(stream)
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1) / 1e3, 1e-6)
        for i in range(int(settle_s / one)):
            plan_run(*ptrs[i % rotate], sh)
    for i in range(warmup):
        plan_run(*ptrs[i % rotate], sh)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` launches, wall clock bracketed by syncs.
    t0 = time.perf_counter()
    for i in range(steps):
        plan_run(*ptrs[i % rotate], sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Average launch duration: one pair of HIP events on the launch stream
    # around `steps` back-to-back launches (an event pair per launch would
    # add its own overhead to microsecond kernels).  The engine clock is
    # sampled meanwhile only for launches of 50 us or more (the clock-adjusted
    # fraction is reported for the compute-bound workloads; the sampler's
    # thread competes with the launch loop).  For microsecond kernels the
    # pair still times the gaps between launches as well: 256^3 reads about
    # 4.0 us here against 3.2 us per step by the wall clock and 3.21 us in a
    # kernel trace.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    clock = ClockSampler() if wall / steps >= 50e-6 else None
    if clock:
        clock.__enter__()
    try:
        ev0.record(stream)
        for i in range(steps):
            plan_run(*ptrs[i % rotate], sh)
        ev1.record(stream)
        torch.cuda.synchronize()
    finally:
        if clock:
            clock.__exit__(None, None, None)
    kernel_avg = ev0.elapsed_time(ev1) / 1e3 / steps
    assert all(torch.isfinite(c).all().item() for _, _, c in sets), "non-finite output"

    flops = pm.gemm_flops(w.m, w.n, w.k)
    return {
        "workload": w,
        "plan": plan.info,
        "wall_s": wall,
        "ms_per_step": wall / steps * 1e3,
        "tflops": flops * steps / wall / 1e12,
        "kernel_avg_s": kernel_avg,
        "sclk_mhz": clock.mean_mhz() if clock else None,
        "sclk_samples": len(clock.samples) if clock else 0,
        "flops": flops,
        "bytes": pm.compulsory_bytes(w.m, w.n, w.k),
    }


def cpu_baseline(name, target_s):
    """The CPU oracle (as it stands) on a bounded sample of the workload: the
    first R rows of C, with R grown until the run takes about target_s."""
    import numpy as np

    import oracle
    from dense_gemm_optimisation_fp32_amd import perfmodel as pm
    from workloads import WORKLOADS, workload_operands

    w = WORKLOADS[name]
    A, B = workload_operands(w)
    rows = 8
    while True:
        a = np.ascontiguousarray(A[:rows])
        t0 = time.perf_counter()
        oracle.gemm_f64(a, B, rows, w.n, w.k, w.layout_b)
        t = time.perf_counter() - t0
        if t >= target_s / 3 or rows >= w.m:
            break
        rows = min(w.m, max(rows * 2, int(rows * target_s / 3 / max(t, 1e-3))))
    out = {
        "value": pm.gemm_flops(rows, w.n, w.k) / t / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"first {rows} of {w.m} rows of C for {w.name} ({w.m}x{w.n}x{w.k}), "
                  f"float64 triple loop, {t:.2f} s",
        "cpu_model": cpu_model(),
    }
    # The 256^3 case, whole, on one thread and on all of them.
    s = WORKLOADS["sq256"]
    A, B = workload_operands(s)
    t_all = _time_oracle(oracle, A, B, s)
    before = oracle.set_num_threads(1)
    try:
        t_one = _time_oracle(oracle, A, B, s)
    finally:
        oracle.set_num_threads(before)
    out["sq256_seconds"] = {"threads_1": round(t_one, 5), f"threads_{before}": round(t_all, 5)}
    return out


def _time_oracle(oracle, A, B, w, repeats=3):
    best = None
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.gemm_f64(A, B, w.m, w.n, w.k, w.layout_b)
        t = time.perf_counter() - t0
        best = t if best is None else min(best, t)
    return best


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


MIN_CLOCK_SAMPLES = 5


def clock_adjusted(achieved_tflops, peak_tflops, sclk_mhz, samples):
    """(clock, fraction of the peak at that clock, note).  The published
    peaks assume the 2.4 GHz peak engine clock; the driver's reported level
    (pp_dpm_sclk) is only trusted when enough samples were taken and it
    implies a fraction of at most 1 (a kernel cannot run above the peak of
    its clock): otherwise the reading did not track the running clock, and
    the fraction is null."""
    from dense_gemm_optimisation_fp32_amd import perfmodel as pm

    if not sclk_mhz:
        return None, None, "no engine-clock reading on this host"
    if samples < MIN_CLOCK_SAMPLES:
        return sclk_mhz, None, f"only {samples} clock samples"
    frac = achieved_tflops / (peak_tflops * sclk_mhz * 1e6 / pm.MI355X_PEAK_SCLK_HZ)
    if frac > 1.0:
        return sclk_mhz, None, (f"the reported clock ({sclk_mhz:.0f} MHz) is below what the measured rate "
                                f"needs ({achieved_tflops / peak_tflops * pm.MI355X_PEAK_SCLK_HZ / 1e6:.0f} MHz): "
                                f"it did not track the running clock")
    return sclk_mhz, round(frac, 4), None


def roofline(res):
    from dense_gemm_optimisation_fp32_amd import perfmodel as pm

    w = res["workload"]
    intensity = pm.arithmetic_intensity(w.m, w.n, w.k)
    ridge = pm.ridge_point(pm.MI355X_FP32_MATRIX_PEAK, pm.MI355X_HBM_BANDWIDTH)
    kind = res["plan"]["kind"]
    if intensity >= ridge:
        peak = pm.MI355X_FP32_MATRIX_PEAK if kind != 1 else pm.MI355X_FP32_VECTOR_PEAK
        achieved = res["flops"] / res["kernel_avg_s"] / 1e12
        out = {"bound": "mfma" if kind != 1 else "alu", "achieved": round(achieved, 3),
               "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(achieved / (peak / 1e12), 4)}
        # The peaks assume the 2.4 GHz peak engine clock; the same fraction
        # against the peak at the clock measured during the timed launches.
        sclk, frac_clk, note = clock_adjusted(achieved, peak / 1e12, res.get("sclk_mhz"), res.get("sclk_samples", 0))
        out["sclk_mhz"] = round(sclk, 1) if sclk else None
        out["frac_at_sclk"] = frac_clk
        if note:
            out["sclk_note"] = note
    else:
        achieved = res["bytes"] / res["kernel_avg_s"] / 1e9
        out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": pm.MI355X_HBM_BANDWIDTH / 1e9,
               "unit": "GB/s", "frac": round(achieved / (pm.MI355X_HBM_BANDWIDTH / 1e9), 4)}
    out["traffic"] = traffic_bytes(w.name, res["plan"]["name"])
    out["kernel"] = res["plan"]["name"]
    out["kernel_avg_us"] = round(res["kernel_avg_s"] * 1e6, 2)
    return out


# The other workloads of the metric, by the labels the metric's configs use.
CONFIGS = (("C1", "sq256", 1), ("C3", "sq4096t", 1), ("C4", "ragged", 1), ("C5a", "ffn", 1),
           ("C5b", "skinny", 8))


def config_lines(steps, warmup, settle_s):
    """Each other workload timed in this run: its kernel average (HIP events
    on the launch stream) and the rate against its roofline."""
    out = {}
    for label, name, rotate in CONFIGS:
        r = time_workload(name, steps, warmup, None, rotate, settle_s=settle_s)
        rf = roofline(r)
        out[label] = {"workload": name, "kernel": r["plan"]["name"], "grid": r["plan"]["grid"],
                      "operand_sets": rotate, "kernel_avg_us": rf["kernel_avg_us"],
                      "tflops_wall": round(r["tflops"], 3), "bound": rf["bound"],
                      "achieved": rf["achieved"], "unit": rf["unit"], "frac": rf["frac"],
                      "stream_k": r["plan"]["stream_k"], "split_k": r["plan"]["split_k"]}
        if rf["bound"] == "hbm":
            out[label]["tflops_kernel"] = round(r["flops"] / r["kernel_avg_s"] / 1e12, 3)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    from dense_gemm_optimisation_fp32_amd import perfmodel as pm

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)          # one kernel: reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        del src, dst

    res = time_workload(args.workload, args.steps, args.warmup, args.variant, args.rotate,
                        0 if args.layout_a == "row" else 1, args.epilogue, args.settle_s)
    w = res["workload"]
    line = {
        "metric": METRIC if w.name == HEADLINE else f"FP32 GEMM TFLOPS (2MNK/t), {w.name}",
        "value": round(res["tflops"], 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: C=A.B, M={w.m} N={w.n} K={w.k}, "
                               f"A {'row' if args.layout_a == 'row' else 'column'}-major, C row-major, "
                               f"B {'row' if w.layout_b == 0 else 'column'}-major, {w.dist}, seed {w.seed}"
                               + ("" if args.epilogue == "none" else f", fused epilogue: {args.epilogue}"
                                  + ("" if args.epilogue == "bias" else " of A.B + bias")),
                   "operand_sets": args.rotate,
                   "m": w.m, "n": w.n, "k": w.k, "layout_b": "row" if w.layout_b == 0 else "col",
                   "kernel": res["plan"]["name"], "grid": res["plan"]["grid"],
                   "pct_of_fp32_matrix_peak": round(100 * res["tflops"] / (pm.MI355X_FP32_MATRIX_PEAK / 1e12), 2),
                   "settle_s": args.settle_s},
        "roofline": roofline(res),
    }
    if not args.no_configs and args.workload == HEADLINE and args.variant is None and args.layout_a == "row" \
            and args.epilogue == "none":
        line["configs"] = config_lines(max(20, args.steps), max(5, args.warmup), args.settle_s)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(line), flush=True)

    if args.all:
        from workloads import WORKLOADS
        os.makedirs(os.path.dirname(args.all_out) or ".", exist_ok=True)
        with open(args.all_out, "a") as f:
            for name in WORKLOADS:
                r = time_workload(name, max(20, args.steps // 5), max(20, args.warmup // 5), None,
                                  8 if name == "skinny" else 1)
                rec = {"workload": name, "kernel": r["plan"]["name"], "grid": r["plan"]["grid"],
                       "rotate": 8 if name == "skinny" else 1,
                       "tflops": round(r["tflops"], 3), "kernel_avg_us": round(r["kernel_avg_s"] * 1e6, 2),
                       "roofline": roofline(r)}
                f.write(json.dumps(rec) + "\n")
                print(json.dumps(rec), file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
