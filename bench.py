#!/usr/bin/env python3
"""Throughput of the tiled dense product on one MI355X, against its roofline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one call of the library's C ABI (tdm_gemm_f32_path /
tdm_gemm_bf16_f32acc_path, which with the auto path are gemm_f32 /
gemm_bf16_f32acc) on one set of synthetic inputs already resident in HBM:
cost model and path choice on the host, then the tiled kernel (tile
schedule, coalesced loads, LDS staging, pipelined K loop, MFMA/FMA
accumulation, C write-back). With no flags the workload is the square bf16
8192 product (bf16 in, fp32 accumulate and out) on the matrix cores, the
largest square product of the measured set. The square fp32 4096 product
(--workload f32_4096) runs on the vector-ALU kernel; the matrix-core kernel
that the auto path picks for it is then timed as well and reported under
config.auto_path (--path mfma makes it the main measurement). Every other
workload runs on the auto path; bf16_mlp_gelu is the MLP product finished in the kernel (+
bias, GELU, bf16 output, through gemm_bf16_epilogue), and its line also
times the same steps unfused (config.unfused).
Consecutive steps rotate over several copies of (A, B, C) whose total size
exceeds the 256 MB last-level cache, so every step reads its operands from
HBM.

Before the warm-up steps the step runs for --prewarm-s seconds of wall time
(0.25 by default; the count is reported as config.prewarm_calls): after the
host-side input generation the engine clock takes tens of milliseconds to
leave its idle state, and with 5 warm-up steps the first timed steps of the
8192^3 product ran 9% slower than in steady state.

The timed region is bracketed by device synchronisation, with HIP events
recorded on the stream the kernels are launched on. It is also the only
region a profiler started with `rocprofv3 --selected-regions` records
(roctxProfilerResume before its first launch, roctxProfilerPause after its
last), so a kernel trace of the same command covers exactly the timed
launches. One JSON line is printed; besides the throughput it carries:
  roofline      achieved rate of the product's kernel (algorithmic FLOPs or
                bytes per launch / average launch time) against MI355X's
                published peak for the bound that applies; `traffic` is the
                measured HBM bytes per launch from rocprofv3 counters when a
                counter record for the current kernel source exists;
  cpu_baseline  the CPU oracle (plain fp64 triple loop) timed on a bounded
                sample of the same workload on this host's cores;
  vendor_blas   (with --vendor) torch.mm on the same resident inputs, timed
                the same way: context, not part of the measurement.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

# MI355X published peaks (dense).
PEAK = {
    "mfma_fp8": 5033.2,   # TFLOP/s (twice the bf16 figure; AMD quotes 5.0 PFLOP/s)
    "mfma_bf16": 2516.6,  # TFLOP/s
    "mfma_f32": 157.3,    # TFLOP/s
    "alu_f32": 157.3,     # TFLOP/s, fp32 vector
    "hbm": 8000.0,        # GB/s
}
KERNEL = {  # path -> (dominant kernel, source file, every kernel one call launches)
    "edge": ("edge_kernel", "gemm_edge.hip", ["edge_kernel"]),
    # small fp32 products on the edge path (M, N, K <= 512, K and N multiples of 4)
    "edge_small": ("small_f32_kernel", "gemm_edge.hip", ["small_f32_kernel"]),
    "valu": ("valu_f32_kernel", "gemm_valu_f32.hip", ["valu_f32_kernel"]),
    "mfma": ("mfma_bf16_kernel", "gemm_mfma_bf16.hip", ["mfma_bf16_kernel"]),
    "mfma_f32": ("mfma_f32_kernel", "gemm_mfma_f32.hip", ["mfma_f32_kernel"]),
    "skinny": ("skinny_bf16_kernel", "gemm_skinny_bf16.hip",
               ["skinny_bf16_kernel", "skinny_reduce_kernel"]),
    "skinny_nk": ("skinny_nk_bf16_kernel", "gemm_skinny_nk_bf16.hip", ["skinny_nk_bf16_kernel"]),
    "mfma_fp8": ("mfma_fp8_kernel", "gemm_mfma_fp8.hip", ["mfma_fp8_kernel"]),
    "attention": ("attention_fwd_kernel", "attention_fwd.hip", ["attention_fwd_kernel"]),
}
DEFAULT_WORKLOAD = "bf16_8192"
# The path each workload is specified on when --path is not given: the square
# fp32 4096 product is the register- and LDS-tiled vector-ALU kernel; the
# others take the library's own choice (matrix cores, or the streaming path
# for M = 16).
DEFAULT_PATH = {"f32_4096": "valu"}
ROTATE_BYTES = 640 << 20  # working set across rotated copies


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--path", default=None,
                    help="force a path (auto/edge/valu/mfma/skinny); default: the workload's "
                         "specified path (valu for f32_4096), else auto")
    ap.add_argument("--prewarm-s", type=float, default=0.25,
                    help="seconds of untimed steps before the warm-up steps (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true",
                    help="epilogue workloads: skip timing the unfused steps (for profiler runs, "
                         "whose kernel statistics would mix both)")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch.mm (PyTorch's ROCm BLAS) on the same resident inputs "
                         "and report it under vendor_blas, for context")
    ap.add_argument("--summarize-trace", metavar="DIR", default=None,
                    help="instead of running, summarize a rocprofv3 --kernel-trace output "
                         "directory of a bench.py run with the same --workload/--steps/--warmup: "
                         "per kernel, all dispatches and the timed ones (markdown on stdout)")
    ap.add_argument("--summarize-counters", metavar="DIR", nargs="+", default=None,
                    help="instead of running, average the per-dispatch counters of rocprofv3 "
                         "--pmc output directories for the workload's dominant kernel (markdown)")
    ap.add_argument("--bench-line", metavar="FILE", default=None,
                    help="with --summarize-trace: the JSON line the profiled run printed")
    ap.add_argument("--kernel", default=None,
                    help="with --summarize-counters: the kernel to summarize (default: the "
                         "workload's dominant kernel)")
    ap.add_argument("--fetch-scale", type=float, default=2.0,
                    help="bytes per FETCH_SIZE KiB / 1024, from a plain copy of known size")
    ap.add_argument("--write-scale", type=float, default=1.0,
                    help="bytes per WRITE_SIZE KiB / 1024, from a plain copy of known size")
    ap.add_argument("--traffic-json", metavar="FILE", default=None,
                    help="with --summarize-counters over FETCH_SIZE and WRITE_SIZE runs: write "
                         "the kernel's HBM bytes per launch as the record bench.py reads")
    ap.add_argument("--sample-power", action="store_true",
                    help="sample the socket power and engine clock (amd-smi) every ~0.25 s over "
                         "the timed region and add their medians to the line as `power`; give "
                         "it enough --steps for a few seconds")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the product, run a plain device copy of this many MiB "
                         "(reference for HBM byte counters)")
    return ap.parse_args()


def src_digest(fname: str) -> str:
    path = os.path.join(ROOT, "tiled_dense_matrix_amd", "csrc", fname)
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


class ProfilerRegion:
    """roctxProfilerResume / roctxProfilerPause of the ROCm profiler SDK.

    Under `rocprofv3 --selected-regions` only the launches between the two
    calls are recorded; without a profiler the calls do nothing. When the
    library cannot be loaded the region is a no-op too."""

    def __init__(self):
        import ctypes
        self._lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            try:
                lib = ctypes.CDLL(name)
            except OSError:
                continue
            lib.roctxProfilerResume.argtypes = [ctypes.c_uint64]
            lib.roctxProfilerPause.argtypes = [ctypes.c_uint64]
            self._lib = lib
            break

    def resume(self):
        if self._lib is not None:
            self._lib.roctxProfilerResume(0)

    def pause(self):
        if self._lib is not None:
            self._lib.roctxProfilerPause(0)


REGION = None


class PowerSampler:
    """Socket power and engine clock as `amd-smi metric -p -c` reports them,
    sampled from a thread between start() and stop()."""

    CMD = ["amd-smi", "metric", "-p", "-c"]

    def __init__(self, interval_s: float = 0.25):
        self.interval_s = interval_s
        self.samples = []  # (watts, MHz)
        self._stop = None
        self._thread = None

    def _one(self):
        import re
        import subprocess
        try:
            r = subprocess.run(self.CMD, capture_output=True, text=True, timeout=10)
        except (OSError, subprocess.SubprocessError):
            return None
        p = re.search(r"SOCKET_POWER:\s*([0-9.]+)", r.stdout)
        c = re.search(r"^\s*CLK:\s*([0-9.]+)", r.stdout, re.M)
        return (float(p.group(1)), float(c.group(1))) if p and c else None

    def _run(self):
        while not self._stop.is_set():
            v = self._one()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.interval_s)

    def start(self):
        import threading
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        self._stop.set()
        self._thread.join()

    def summary(self):
        import statistics
        if not self.samples:
            return {"samples": 0, "tool": " ".join(self.CMD)}
        w = [x for x, _ in self.samples]
        c = [y for _, y in self.samples]
        return {"samples": len(self.samples), "tool": " ".join(self.CMD),
                "socket_w_median": statistics.median(w), "socket_w_min": min(w),
                "socket_w_max": max(w), "sclk_mhz_median": statistics.median(c),
                "sclk_mhz_min": min(c), "sclk_mhz_max": max(c)}


POWER = None  # a PowerSampler over the timed region, with --sample-power


def timed_region():
    global REGION
    if REGION is None:
        REGION = ProfilerRegion()
    return REGION


def traffic_record(kernels, src: str, workload: str):
    """HBM bytes per call (all its kernels) from committed counter records.

    None unless every kernel has a record taken from the current source.
    """
    total = 0.0
    for kernel in kernels:
        path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.traffic.json")
        if not os.path.exists(path):
            return None
        with open(path) as fh:
            rec = json.load(fh)
        if rec.get("source_sha") != src_digest(src):
            return None  # the kernel changed since the counters were taken
        total += float(rec["hbm_bytes_per_launch"])
    return total


def _csv_rows(root: str, suffix: str):
    """Rows of every rocprofv3 CSV file under root whose name ends in suffix."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(root):
        for f in sorted(files):
            if f.endswith(suffix):
                with open(os.path.join(dirpath, f), newline="") as fh:
                    rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {root}")
    return rows


def _short(name: str, kernels):
    """The kernel (of `kernels`) whose name the demangled trace name holds."""
    for k in kernels:
        if k in name:
            return k
    return None


def workload_kernels(name: str, path=None):
    """(dominant kernel, source, kernels of one call) of a workload on the
    given path (a --path name), else on the path bench.py runs it on by
    default."""
    import tiled_dense_matrix_amd as tdm
    from tiled_dense_matrix_amd import inputs
    if name in inputs.ATTN_WORKLOADS:
        return KERNEL["attention"]
    w = inputs.WORKLOADS[name]
    if w.kind == "fp8":
        return KERNEL["mfma_fp8"]
    kind = tdm.Kind.F32 if w.kind == "f32" else tdm.Kind.BF16_F32ACC
    layout = tdm.Layout((tdm.Layout.NK if w.b_layout == "nk" else 0)
                        | (tdm.Layout.KM_KN if w.a_layout == "km" else 0))
    pname = path if path not in (None, "auto") else DEFAULT_PATH.get(name)
    pname = pname or tdm.path_name(tdm.tdm_select_path_ex(kind, layout, w.M, w.N, w.K))
    if pname == "mfma" and w.kind == "f32":
        pname = "mfma_f32"
    if pname == "skinny" and w.b_layout == "nk":
        pname = "skinny_nk"
    if (pname == "edge" and w.kind == "f32" and int(layout) == 0 and max(w.M, w.N, w.K) <= 512
            and w.K % 4 == 0 and w.N % 4 == 0 and w.N >= 4 and w.K >= 4):
        pname = "edge_small"
    return KERNEL[pname]


def summarize_trace(args):
    """Markdown summary of a kernel trace: for each kernel of the workload,
    all its dispatches and the timed ones (dispatches p + warmup .. p +
    warmup + steps - 1 of that kernel, in start order, p = the pre-warm
    calls the run's line reports), in microseconds."""
    _, src, kernels = workload_kernels(args.workload, args.path)
    line = None
    if args.bench_line:
        with open(args.bench_line) as fh:
            line = json.loads([x for x in fh.read().splitlines() if x.startswith("{")][-1])
    first = int((line or {}).get("config", {}).get("prewarm_calls", 0)) + args.warmup
    by = {}
    for r in _csv_rows(args.summarize_trace, "kernel_trace.csv"):
        k = _short(r["Kernel_Name"], kernels)
        if k is not None:
            by.setdefault(k, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = ["| kernel | dispatches | average (us) | timed dispatches | timed average (us) | "
           "timed min (us) | timed median (us) | timed max (us) |",
           "|---|---:|---:|---:|---:|---:|---:|---:|"]
    timed_total = 0.0
    for k in kernels:
        us = [(e - b) / 1e3 for b, e in sorted(by.get(k, []))]
        t = sorted(us[first:first + args.steps])
        if not t:
            raise SystemExit(f"{k}: {len(us)} dispatches, none in the timed window")
        avg_t = sum(t) / len(t)
        timed_total += avg_t
        out.append(f"| {k} | {len(us)} | {sum(us) / len(us):.1f} | {len(t)} | {avg_t:.1f} | "
                   f"{t[0]:.1f} | {t[len(t) // 2]:.1f} | {t[-1]:.1f} |")
    print("\n".join(out))
    if line is not None:
        step_us = line["ms_per_step"] * 1e3
        roof = line["roofline"]
        print(f"\nbench.py line of the same run: {step_us:.1f} us per step, {line['value']} "
              f"{line['unit']}, roofline {roof['achieved']} {roof['unit']} of {roof['peak']} "
              f"(frac {roof['frac']}). Timed kernel time per step {timed_total:.1f} us = "
              f"{timed_total / step_us:.3f} of the step.")
    print(f"\nKernel source `{src}` sha256[:16] = {src_digest(src)} when measured.")


def summarize_counters(args):
    """Markdown table of per-dispatch counter values (each counter summed
    over the GPU within a dispatch, then averaged over the dispatches of the
    workload's dominant kernel) from one or more rocprofv3 --pmc outputs,
    with derived rates. GRBM_GUI_ACTIVE counts each XCD's engine cycles, so
    its eighth is the cycles of the clock the counters ran at."""
    kernel, src, _ = workload_kernels(args.workload, args.path)
    kernel = args.kernel or kernel
    per, durations = {}, []
    for root in args.summarize_counters:
        disp = {}
        for r in _csv_rows(root, "counter_collection.csv"):
            if kernel not in r["Kernel_Name"]:
                continue
            d = disp.setdefault(r.get("Dispatch_Id") or r.get("Correlation_Id"), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                d["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        for d in disp.values():
            for c, v in d.items():
                (durations if c == "_us" else per.setdefault(c, [])).append(v)
    if not per:
        raise SystemExit(f"no counters of {kernel}")
    avg = {c: sum(v) / len(v) for c, v in per.items()}
    print("| counter | per dispatch |\n|---|---:|")
    for c in sorted(avg):
        print(f"| {c} | {avg[c]:,.0f} |")
    simds, xcds = 1024, 8
    rows = []
    if durations:
        rows.append(("average dispatch under the counters (us)",
                     f"{sum(durations) / len(durations):.1f}"))
    # The counters' window is a few microseconds longer than the dispatch, so
    # GRBM_GUI_ACTIVE gives the clock only for long dispatches; short ones are
    # rated against the 2.4 GHz peak clock over their duration.
    us = sum(durations) / len(durations) if durations else 0.0
    clk, where = None, ""
    if avg.get("GRBM_GUI_ACTIVE") and us >= 200.0:
        clk, where = avg["GRBM_GUI_ACTIVE"] / xcds, "at the measured clock"
        rows.append(("engine clock from GRBM_GUI_ACTIVE (GHz)", f"{clk / us / 1e3:.3f}"))
    elif us:
        clk, where = us * 2.4e3, "at 2.4 GHz over the dispatch (too short to measure the clock)"
    if clk:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            rows.append((f"MFMA busy / SIMD cycles {where}",
                         f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / simds / clk:.3f}"))
        if "SQ_ACTIVE_INST_VALU" in avg:
            rows.append((f"VALU-active / SIMD cycles {where}",
                         f"{avg['SQ_ACTIVE_INST_VALU'] / simds / clk:.3f}"))
    if avg.get("SQ_INSTS_MFMA") and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        rows.append(("MFMA busy cycles per MFMA instruction",
                     f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / avg['SQ_INSTS_MFMA']:.1f}"))
    if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
        rows.append(("LDS bank-conflict cycles / LDS active cycles",
                     f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.4f}"))
    if avg.get("SQ_WAVE_CYCLES"):
        for c, what in (("SQ_WAIT_INST_ANY", "waiting on dependencies"),
                        ("SQ_WAIT_INST_LDS", "waiting on LDS")):
            if c in avg:
                rows.append((f"{what} / wave cycles", f"{avg[c] / avg['SQ_WAVE_CYCLES']:.3f}"))
    if "FETCH_SIZE" in avg and "WRITE_SIZE" in avg:
        fetch = avg["FETCH_SIZE"] * 1024 * args.fetch_scale
        write = avg["WRITE_SIZE"] * 1024 * args.write_scale
        rows.append(("HBM bytes read per launch (FETCH_SIZE, scaled)", f"{fetch:,.0f}"))
        rows.append(("HBM bytes written per launch (WRITE_SIZE, scaled)", f"{write:,.0f}"))
        rows.append(("HBM bytes per launch", f"{fetch + write:,.0f}"))
        if args.traffic_json:
            rec = {"kernel": kernel, "workload": args.workload, "source": src,
                   "source_sha": src_digest(src), "fetch_kib_raw": avg["FETCH_SIZE"],
                   "write_kib_raw": avg["WRITE_SIZE"], "fetch_scale": args.fetch_scale,
                   "write_scale": args.write_scale, "hbm_bytes_per_launch": fetch + write}
            with open(args.traffic_json, "w") as fh:
                json.dump(rec, fh, indent=1)
                fh.write("\n")
    if rows:
        print("\n| derived | value |\n|---|---:|")
        for k, v in rows:
            print(f"| {k} | {v} |")
    print(f"\nKernel source `{src}` sha256[:16] = {src_digest(src)} when measured.")


def copy_probe(mib: int):
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 5}), flush=True)


def cpu_baseline(w, A, B, C_gpu, target_s: float, bias=None):
    """Time the oracle on the first rows of C (with the workload's epilogue,
    if any); also check those rows."""
    import oracle
    threads = oracle.default_threads()
    # Calibrate on one row per thread (the second of two calls: the first
    # also starts the thread pool), then size the sample to ~target_s.
    rows = min(w.M, threads)
    for _ in range(2):
        t0 = time.perf_counter()
        oracle.gemm_block(A, B, (0, rows), (0, w.N), threads)
        per_row = max(time.perf_counter() - t0, 1e-6) / rows
    rows = int(max(1, min(w.M, math.floor(target_s / per_row))))
    if rows >= threads:
        rows -= rows % threads  # whole rows per thread
    # A product much shorter than the budget is computed whole, repeatedly,
    # so that the timed region is long enough to mean something.
    reps = 1
    if rows == w.M and per_row * w.M < target_s / 4:
        t0 = time.perf_counter()
        oracle.gemm_block(A, B, (0, rows), (0, w.N), threads)
        per_call = max(time.perf_counter() - t0, 1e-6)
        reps = int(max(1, min(10000, math.floor(target_s / per_call))))
    t0 = time.perf_counter()
    for _ in range(reps):
        R = oracle.gemm_block(A, B, (0, rows), (0, w.N), threads)
        if w.has_epilogue:
            R = oracle.epilogue(R, bias, None, w.gelu)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K * reps
    ma = float(np.abs(oracle.widen(A)).max())
    mb = float(np.abs(oracle.widen(B)).max())
    got = oracle.widen(C_gpu[:rows]) if C_gpu.dtype == np.uint16 else C_gpu[:rows]
    p = oracle.parity(got, R, ma, mb, w.K)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"rows 0..{rows - 1} of C ({rows}x{w.N}x{w.K}"
                   + (f", computed {reps} times" if reps > 1 else "")
                   + f", {flops / 1e9:.1f} GFLOP) in {dt:.1f} s, fp64 triple loop"),
        "sample_parity": {k: float(f"{v:.3e}") for k, v in p.items()},
    }


def main():
    args = parse()
    global POWER
    if args.sample_power:
        POWER = PowerSampler()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_counters:
        return summarize_counters(args)
    # The profiler's region markers register with the profiler when their
    # library loads, which has to happen before the GPU runtime starts.
    timed_region()
    import torch
    import tiled_dense_matrix_amd as tdm
    from tiled_dense_matrix_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return

    if args.workload in inputs.ATTN_WORKLOADS:
        return main_attention(args, inputs.ATTN_WORKLOADS[args.workload])
    w = inputs.WORKLOADS[args.workload]
    if w.kind == "fp8":
        return main_fp8(args, w)
    kind = tdm.Kind.F32 if w.kind == "f32" else tdm.Kind.BF16_F32ACC
    pname_arg = args.path or DEFAULT_PATH.get(w.name, "auto")
    path = tdm.Path[pname_arg.upper()]
    nk = w.b_layout == "nk"  # B stored N x K: C = A @ B.T
    km = w.a_layout == "km"  # A stored K x M: C = A.T @ B
    layout = tdm.Layout((tdm.Layout.NK if nk else 0) | (tdm.Layout.KM_KN if km else 0))
    chosen = tdm.tdm_select_path_ex(kind, layout, w.M, w.N, w.K) if path == tdm.Path.AUTO \
        else path
    pname = tdm.path_name(chosen)
    kernel, ksrc, kernels = workload_kernels(w.name, pname)

    A, B = inputs.make_inputs(w)

    def dev(X):
        if X.dtype == np.uint16:
            X = X.view(np.int16)
        return torch.from_numpy(X).cuda()

    # A workload with a fused epilogue (bias, GELU, bf16 output) runs the
    # product through gemm_bf16_epilogue; its output has the epilogue's type.
    epi = w.has_epilogue
    out_bf16 = epi and w.out == "bf16"
    out_size = 2 if out_bf16 else 4
    bias_np = inputs.make_bias(w) if epi and w.bias_sigma > 0 else None

    A0, B0 = dev(A), dev(B)
    bias_d = None if bias_np is None else dev(bias_np)
    set_bytes = A0.numel() * A0.element_size() + B0.numel() * B0.element_size() + \
        w.M * w.N * out_size
    rot = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    out_t = torch.bfloat16 if out_bf16 else torch.float32
    sets = [(A0, B0, torch.empty((w.M, w.N), dtype=out_t, device="cuda"))]
    for _ in range(rot - 1):
        sets.append((A0.clone(), B0.clone(), torch.empty_like(sets[0][2])))

    fn = tdm.tdm_gemm_f32_path if w.kind == "f32" else tdm.tdm_gemm_bf16_f32acc_path
    stream = torch.cuda.current_stream()

    def call(i, p):
        a, b, c = sets[i % rot]
        if w.kind == "f32" and (nk or km):
            tdm.tdm_gemm_f32_ex_path(a, b, layout, c, path=p, stream=stream)
        elif epi or nk or km:
            tdm.tdm_gemm_bf16_ex_path(a, b, layout, c, bias=bias_d, gelu=w.gelu, path=p,
                                      stream=stream)
        else:
            fn(a, b, c, path=p, stream=stream)

    def time_steps(step) -> float:
        """Average ms per step(i) over args.steps steps after args.warmup."""
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        region = timed_region() if profiled else None
        if region:
            region.resume()
            if POWER:
                POWER.start()
        start.record(stream)
        for i in range(args.steps):
            step(args.warmup + i)
        end.record(stream)
        torch.cuda.synchronize()
        if region:
            region.pause()
            if POWER:
                POWER.stop()
        return start.elapsed_time(end) / args.steps

    profiled = True  # only the main measurement is the profiler's region

    def timed(p) -> float:
        return time_steps(lambda i: call(i, p))

    prewarm_calls = prewarm(lambda i: call(i, path), args.prewarm_s)
    ms = timed(path)
    profiled = False

    roof = tdm.gemm_roofline(kind, w.M, w.N, w.K)
    # Bytes with every array crossing HBM once: A and B read, the bias read,
    # the output written in its own element type.
    alg_bytes = roof.bytes if not epi else \
        2 * (w.M * w.K + w.K * w.N) + out_size * w.M * w.N + \
        (out_size * w.N if bias_np is not None else 0)
    tflops = roof.flops / (ms * 1e-3) / 1e12
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    if pname == "skinny":
        bound, unit, achieved, peak = "hbm", "GB/s", gbs, PEAK["hbm"]
    elif pname == "mfma":
        bound, unit, achieved, peak = "mfma", "TFLOP/s", tflops, PEAK[
            "mfma_f32" if w.kind == "f32" else "mfma_bf16"]
    else:
        bound, unit, achieved, peak = "alu", "TFLOP/s", tflops, PEAK["alu_f32"]
    traffic = traffic_record(kernels, ksrc, w.name)

    # Every rotated copy must hold the same product (spot check: first rows).
    C_last = sets[(args.warmup + args.steps - 1) % rot][2]
    C_gpu = C_last.view(torch.int16).cpu().numpy().view(np.uint16) if out_bf16 else \
        C_last.cpu().numpy()
    if args.warmup + args.steps >= rot:
        for a, b, c in sets[1:]:
            assert torch.equal(c[:4], sets[0][2][:4]), "rotated copies disagree"

    # When the workload is specified on another path than the one gemm_* would
    # pick, time the library's own choice too (after the main measurement).
    auto_choice = tdm.path_name(tdm.tdm_select_path_ex(kind, layout, w.M, w.N, w.K))
    auto_info = None
    if path != tdm.Path.AUTO and auto_choice != pname:
        ms_auto = timed(tdm.Path.AUTO)
        tf_auto = roof.flops / (ms_auto * 1e-3) / 1e12
        gb_auto = alg_bytes / (ms_auto * 1e-3) / 1e9
        # the bound of the path the library chose, as for the main measurement
        if auto_choice == "skinny":
            bound_auto, ach_auto, peak_auto = "hbm", gb_auto, PEAK["hbm"]
        elif auto_choice == "mfma":
            bound_auto, ach_auto = "mfma", tf_auto
            peak_auto = PEAK["mfma_f32" if w.kind == "f32" else "mfma_bf16"]
        else:
            bound_auto, ach_auto, peak_auto = "alu", tf_auto, PEAK["alu_f32"]
        auto_info = {"path": auto_choice, "ms_per_call": round(ms_auto, 6),
                     "tflops": round(tf_auto, 3), "bound": bound_auto,
                     "roofline_frac": round(ach_auto / peak_auto, 4)}

    # The same epilogue unfused: this library's product with fp32 output, then
    # the bias add, GELU and bf16 conversion as separate torch operations.
    unfused = None
    if epi and not args.no_unfused:
        cf = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        bias_f = None if bias_d is None else \
            (bias_d.view(torch.bfloat16).float() if out_bf16 else bias_d)

        def unfused_step(i):
            a, b, c = sets[i % rot]
            tdm.tdm_gemm_bf16_ex_path(a, b, layout, cf, path=path, stream=stream)
            t = cf if bias_f is None else cf + bias_f
            if w.gelu:
                t = torch.nn.functional.gelu(t)
            c.copy_(t)

        ms_u = time_steps(unfused_step)
        unfused = {"what": "gemm_bf16_f32acc, then bias add, GELU and conversion in torch",
                   "ms_per_call": round(ms_u, 6), "fused_speedup": round(ms_u / ms, 4)}
        del cf

    # Context only: the vendor BLAS through torch on the same inputs (bf16
    # with fp32 output, like this library's product; for an epilogue
    # workload torch.addmm with the bias and bf16 output, then GELU), timed
    # the same way.
    vendor = None
    if args.vendor:
        if w.kind == "f32":
            vsets = [(a, b) for a, b, _ in sets]
            vmm, vop = torch.mm, "torch.mm"
            if km or nk:  # the transposed views of the stored operands
                vmm = lambda a, b: torch.mm(a.t() if km else a, b.t() if nk else b)  # noqa: E731
                vop = "torch.mm with " + " and ".join(
                    x for x, on in (("A.t()", km), ("B.t()", nk)) if on)
        else:
            vsets = [(a.view(torch.bfloat16), b.view(torch.bfloat16)) for a, b, _ in sets]
            if not epi:
                if km:  # a 2-D product with A's transposed view (not batched)
                    vmm = lambda a, b: torch.mm(a.t(), b, out_dtype=torch.float32)  # noqa: E731
                    vop = "torch.mm with A.t() (out_dtype=float32)"
                elif nk:  # a 2-D product with the weight's transposed view (not batched)
                    vmm = lambda a, b: torch.mm(a, b.t(), out_dtype=torch.float32)  # noqa: E731
                    vop = "torch.mm with B.t() (out_dtype=float32)"
                else:
                    vmm = lambda a, b: torch.mm(a, b, out_dtype=torch.float32)  # noqa: E731
                    vop = "torch.mm (out_dtype=float32)"
            else:
                if not out_bf16:
                    raise SystemExit("--vendor covers epilogue workloads with bf16 output")
                bias_v = None if bias_d is None else bias_d.view(torch.bfloat16)

                def vmm(a, b):
                    if nk:
                        t = torch.nn.functional.linear(a, b, bias_v)
                    else:
                        t = torch.mm(a, b) if bias_v is None else torch.addmm(bias_v, a, b)
                    return torch.nn.functional.gelu(t) if w.gelu else t
                vop = ("torch.nn.functional.linear" if nk else "torch.addmm") + \
                    " (bf16 out), then GELU"
        ms_v = time_steps(lambda i: vmm(*vsets[i % rot]))
        vendor = {"op": vop, "ms_per_call": round(ms_v, 6),
                  "tflops": round(roof.flops / (ms_v * 1e-3) / 1e12, 3),
                  "this_library_over_vendor": round(ms_v / ms, 4)}

    line = {
        "metric": "GEMM TFLOP/s and % of MFMA/VALU/HBM roofline per shape, 1x MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.kind == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "inputs": f"seed {w.seed}, {w.dist}",
                   "path": pname, "kernel": kernel, "kernels_per_call": kernels,
                   "rotated_copies": rot, "prewarm_calls": prewarm_calls,
                   "auto_path": auto_info,
                   "b_layout": w.b_layout, "a_layout": w.a_layout,
                   "epilogue": None if not epi else {"bias": bias_np is not None,
                                                     "gelu": w.gelu, "out": w.out},
                   "unfused": unfused,
                   "gbps_algorithmic": round(gbs, 1)},
        # One launch of the dominant kernel is timed as one call; a path that
        # launches a second kernel (the skinny path's reduction) is timed
        # with it, and `scope` says so.
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                     "scope": "kernel" if len(kernels) == 1 else "call (" + " + ".join(kernels) + ")",
                     "frac": round(achieved / peak, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes": int(alg_bytes), "algorithmic_flops": int(roof.flops)},
    }
    if vendor is not None:
        line["vendor_blas"] = vendor
    if not args.no_cpu_baseline:
        B_kn = np.ascontiguousarray(B.T) if nk else B  # the oracle takes B as K x N
        A_mk = np.ascontiguousarray(A.T) if km else A  # ... and A as M x K
        line["cpu_baseline"] = cpu_baseline(w, A_mk, B_kn, C_gpu, args.cpu_seconds, bias_np)
    if POWER:
        line["power"] = POWER.summary()
    print(json.dumps(line), flush=True)


def prewarm(step, seconds: float) -> int:
    """Run step(i) in bursts of four until `seconds` of wall time have
    passed; return the number of calls."""
    import torch
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_calls(step, warmup: int, steps: int, stream, profiled: bool = False) -> float:
    """Average ms per step(i) over `steps` calls after `warmup`, with events
    on the stream the kernels run on."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    region = timed_region() if profiled else None
    if region:
        region.resume()
        if POWER:
            POWER.start()
    start.record(stream)
    for i in range(steps):
        step(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    if region:
        region.pause()
        if POWER:
            POWER.stop()
    return start.elapsed_time(end) / steps


def cpu_baseline_fp8(w, A, B, sa, sb, C_gpu, target_s: float):
    """Time the FP8 oracle (decode, scale, fp64 sum) on the first rows of C;
    also check those rows against the GPU output."""
    import oracle
    fa, fb = w.fp8
    threads = oracle.default_threads()

    def timed_rows(r):
        t0 = time.perf_counter()
        oracle.gemm_fp8(A[:r], fa, B, fb, None if sa is None else sa[:r], sb, threads)
        return time.perf_counter() - t0

    # Each call also decodes all of B, a fixed cost: calibrate on two sample
    # sizes and size the sample from the cost per added row.
    r1, r2 = min(w.M, threads), min(w.M, 4 * threads)
    t1, t2 = timed_rows(r1), timed_rows(r2)
    per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-6)
    fixed = max(t1 - r1 * per_row, 0.0)
    rows = int(max(1, min(w.M, math.floor((target_s - fixed) / per_row))))
    if rows >= threads:
        rows -= rows % threads
    t0 = time.perf_counter()
    R = oracle.gemm_fp8(A[:rows], fa, B, fb, None if sa is None else sa[:rows], sb, threads)
    if w.has_epilogue:
        R = oracle.epilogue(R, None, None, w.gelu)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    got = oracle.widen(C_gpu[:rows]) if C_gpu.dtype == np.uint16 else C_gpu[:rows]
    rel = float(np.linalg.norm(got - R) / max(np.linalg.norm(R), 1e-300))
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of C ({rows}x{w.N}x{w.K}, {flops / 1e9:.1f} GFLOP) "
                  f"in {dt:.1f} s: FP8 decode and block scales, then the fp64 triple loop",
        "sample_parity": {"rel_fro": float(f"{rel:.3e}")},
    }


def main_fp8(args, w):
    """One FP8 product per step (gemm_fp8: E4M3/E5M2 codes, block scales,
    the workload's output type)."""
    import torch
    import tiled_dense_matrix_amd as tdm
    from tiled_dense_matrix_amd import inputs

    kernel, ksrc, kernels = KERNEL["mfma_fp8"]
    A, B, sa, sb = inputs.make_fp8_inputs(w)
    fmt = {"e4m3": tdm.Fp8Format.E4M3, "e5m2": tdm.Fp8Format.E5M2}
    fa, fb = fmt[w.fp8[0]], fmt[w.fp8[1]]
    out_bf16 = w.out == "bf16"
    out_t = torch.bfloat16 if out_bf16 else torch.float32
    out_size = 2 if out_bf16 else 4

    def dev(X):
        return None if X is None else torch.from_numpy(X).cuda()

    A0, B0, sa0, sb0 = dev(A), dev(B), dev(sa), dev(sb)
    scale_bytes = 0 if sa is None else sa.size + sb.size
    set_bytes = A.size + B.size + scale_bytes + w.M * w.N * out_size
    rot = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    sets = [(A0, B0, sa0, sb0, torch.empty((w.M, w.N), dtype=out_t, device="cuda"))]
    for _ in range(rot - 1):
        sets.append((A0.clone(), B0.clone(), None if sa0 is None else sa0.clone(),
                     None if sb0 is None else sb0.clone(), torch.empty_like(sets[0][4])))
    stream = torch.cuda.current_stream()

    def call(i):
        a, b, s_a, s_b, c = sets[i % rot]
        tdm.gemm_fp8(a, b, fa, fb, s_a, s_b, D=c, gelu=w.gelu, stream=stream)

    prewarm_calls = prewarm(call, args.prewarm_s)
    ms = time_calls(call, args.warmup, args.steps, stream, profiled=True)
    flops = 2.0 * w.M * w.N * w.K
    alg_bytes = A.size + B.size + scale_bytes + out_size * w.M * w.N
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    traffic = traffic_record(kernels, ksrc, w.name)

    C_last = sets[(args.warmup + args.steps - 1) % rot][4]
    C_gpu = C_last.view(torch.int16).cpu().numpy().view(np.uint16) if out_bf16 else \
        C_last.cpu().numpy()
    if args.warmup + args.steps >= rot:
        for st in sets[1:]:
            assert torch.equal(st[4][:4], sets[0][4][:4]), "rotated copies disagree"

    # Context only: the vendor's FP8 product through torch._scaled_mm with
    # one scale per tensor (it takes no 32-k block scales), bf16 output.
    vendor = None
    if args.vendor:
        try:
            dt8 = {tdm.Fp8Format.E4M3: torch.float8_e4m3fn, tdm.Fp8Format.E5M2: torch.float8_e5m2}
            one = torch.ones((), dtype=torch.float32, device="cuda")
            vsets = [(st[0].view(dt8[fa]), st[1].view(dt8[fb])) for st in sets]

            def vstep(i):
                a, b = vsets[i % rot]
                torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=out_t)

            ms_v = time_calls(vstep, args.warmup, args.steps, stream)
            vendor = {"op": "torch._scaled_mm with B.t(), per-tensor scales (no block scales)",
                      "ms_per_call": round(ms_v, 6),
                      "tflops": round(flops / (ms_v * 1e-3) / 1e12, 3),
                      "this_library_over_vendor": round(ms_v / ms, 4)}
        except (RuntimeError, TypeError, AttributeError) as e:
            vendor = {"op": "torch._scaled_mm", "error": str(e).splitlines()[0][:200]}

    line = {
        "metric": "GEMM TFLOP/s and % of MFMA/VALU/HBM roofline per shape, 1x MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "inputs": f"seed {w.seed}, normal, "
                             + ("32-k block scales" if w.scaled else "no scales"),
                   "formats": list(w.fp8), "b_layout": "nk", "out": w.out,
                   "path": "mfma", "kernel": kernel, "kernels_per_call": kernels,
                   "rotated_copies": rot, "prewarm_calls": prewarm_calls,
                   "gbps_algorithmic": round(gbs, 1)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK["mfma_fp8"],
                     "unit": "TFLOP/s", "scope": "kernel",
                     "frac": round(tflops / PEAK["mfma_fp8"], 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes": int(alg_bytes), "algorithmic_flops": int(flops)},
    }
    if vendor is not None:
        line["vendor_blas"] = vendor
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_fp8(w, A, B, sa, sb, C_gpu, args.cpu_seconds)
    if POWER:
        line["power"] = POWER.summary()
    print(json.dumps(line), flush=True)


def cpu_baseline_attention(w, Q, K, V, O_gpu, target_s: float):
    """Time the attention oracle on whole heads (batch-major order) for about
    target_s; also check them against the GPU output."""
    import oracle
    heads_total = w.batch * w.heads
    r = np.arange(w.seq)
    t0 = time.perf_counter()
    oracle.attention_rows(Q[0, 0], K[0, 0], V[0, 0], r, w.scale, w.causal)
    per_head = max(time.perf_counter() - t0, 1e-6)
    heads = int(max(1, min(heads_total, math.floor(target_s / per_head))))
    t0 = time.perf_counter()
    outs = []
    for i in range(heads):
        b, h = divmod(i, w.heads)
        outs.append(oracle.attention_rows(Q[b, h], K[b, h], V[b, h], r, w.scale, w.causal)[0])
    dt = time.perf_counter() - t0
    visible = (r + 1).sum() if w.causal else w.seq * w.seq
    flops = 4.0 * w.head_dim * visible * heads
    num = den = 0.0
    for i, R in enumerate(outs):
        b, h = divmod(i, w.heads)
        got = oracle.widen(O_gpu[b, h])
        num += float(np.linalg.norm(got - R) ** 2)
        den += float(np.linalg.norm(R) ** 2)
    rel = (num / max(den, 1e-300)) ** 0.5
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.default_threads(),
        "kind": "oracle",
        "sample": f"{heads} of {heads_total} heads, all {w.seq} query rows ({flops / 1e9:.1f} "
                  f"GFLOP) in {dt:.1f} s: fp64 scores, softmax and P V with NumPy",
        "sample_parity": {"rel_fro": float(f"{rel:.3e}")},
    }


def main_attention(args, w):
    """One attention forward per step (attention_fwd: bf16 Q, K, V, O, the
    row logsumexp in fp32)."""
    import torch
    import tiled_dense_matrix_amd as tdm
    from tiled_dense_matrix_amd import inputs

    kernel, ksrc, kernels = KERNEL["attention"]
    Q, K, V = inputs.make_attention_inputs(w)

    def dev(X):
        return torch.from_numpy(X.view(np.int16)).cuda().view(torch.bfloat16)

    base = (dev(Q), dev(K), dev(V))
    bh = w.batch * w.heads
    set_bytes = 4 * Q.size * 2 + bh * w.seq * 4
    rot = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    sets = [base + (torch.empty_like(base[0]), torch.empty((w.batch, w.heads, w.seq),
                                                           dtype=torch.float32, device="cuda"))]
    for _ in range(rot - 1):
        sets.append(tuple(t.clone() for t in base) + (torch.empty_like(base[0]),
                                                      torch.empty_like(sets[0][4])))
    stream = torch.cuda.current_stream()
    lib = tdm.load()

    def call(i):
        q, k, v, o, lse = sets[i % rot]
        st = lib.attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), bh, w.seq, w.seq, w.head_dim, w.scale,
                               1 if w.causal else 0, stream.cuda_stream)
        assert st == 0, st

    prewarm_calls = prewarm(call, args.prewarm_s)
    ms = time_calls(call, args.warmup, args.steps, stream, profiled=True)
    flops = w.flops
    alg_bytes = 4 * Q.size * 2 + bh * w.seq * 4  # Q, K, V read once; O and lse written
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = traffic_record(kernels, ksrc, w.name)
    O_last = sets[(args.warmup + args.steps - 1) % rot][3]
    O_gpu = O_last.view(torch.int16).cpu().numpy().view(np.uint16)
    if args.warmup + args.steps >= rot:
        for st in sets[1:]:
            assert torch.equal(st[3][0, 0, :4], sets[0][3][0, 0, :4]), "rotated copies disagree"

    # Context only: PyTorch's fused attention on the same resident inputs.
    vendor = None
    if args.vendor:
        def vstep(i):
            q, k, v = sets[i % rot][:3]
            torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=w.causal,
                                                             scale=w.scale)
        ms_v = time_calls(vstep, args.warmup, args.steps, stream)
        vendor = {"op": "torch.nn.functional.scaled_dot_product_attention (bf16)",
                  "ms_per_call": round(ms_v, 6),
                  "tflops": round(flops / (ms_v * 1e-3) / 1e12, 3),
                  "this_library_over_vendor": round(ms_v / ms, 4)}

    line = {
        "metric": "GEMM TFLOP/s and % of MFMA/VALU/HBM roofline per shape, 1x MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq": w.seq,
                   "head_dim": w.head_dim, "causal": w.causal,
                   "inputs": f"seed {w.seed}, normal", "kernel": kernel,
                   "kernels_per_call": kernels, "rotated_copies": rot,
                   "prewarm_calls": prewarm_calls,
                   "flops_counted": "4 * head_dim per visible (query, key) pair"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK["mfma_bf16"],
                     "unit": "TFLOP/s", "scope": "kernel",
                     "frac": round(tflops / PEAK["mfma_bf16"], 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes": int(alg_bytes), "algorithmic_flops": int(flops)},
    }
    if vendor is not None:
        line["vendor_blas"] = vendor
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_attention(w, Q, K, V, O_gpu, args.cpu_seconds)
    if POWER:
        line["power"] = POWER.summary()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
