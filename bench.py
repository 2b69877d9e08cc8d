"""Benchmark of the fp32 row-major SGEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sq8192]
                    [--path auto] [--no-cpu-baseline]

A step is one C = A.B call through the C ABI (sgemm_f32_path) on inputs
already resident in HBM: the whole hot path (tile loader, LDS staging,
register/matrix-core micro-kernel, store) over one product.  W untimed
steps, then exactly K timed steps between torch.cuda.synchronize() calls,
timed with HIP events recorded on the stream the kernels are launched on.
Prints ONE JSON line:

  value     GFLOP/s = 2*M*N*K / (average step time) at 8192^3
  roofline  the (only) kernel of the step against the FP32 matrix peak of
            157.3 TFLOP/s: achieved = 2*M*N*K / average launch time;
            traffic = HBM bytes per launch from the committed rocprofv3 PMC
            summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
            size), or null if the kernel sources changed since it was taken
  cpu_baseline  the CPU oracle (fp64, OpenMP) timed on this host on a bounded
            sample of the same product (whole rows)
  configs   every configuration: the 4x4x1024 micro-GEMM (us per launch over
            1000 launches), 1024^3, 2048^3, 1000x1500x777 and 8192^3 (GFLOP/s
            from the mean of back-to-back launches, median and best of
            launches timed one by one, fraction of the FP32 peak, PMC
            traffic); beside each time, the oracle's check of the C those
            launches wrote and the oracle's own time (the full product up to
            2048^3; at 8192^3 a row and a column per 128 band and an entry per
            64 x 64 tile)
  sclk_mhz  the shader clock amd-smi reports while the 8192^3 step runs
  secondary the 2048^3 line (the metric names both sizes)
  paths     every path's GFLOP/s on both sizes, for comparison
  fused_epilogue  sgemm_f32_ex with alpha, beta (C read), bias and ReLU
            against the plain product on both sizes, alternating blocks
  lowp      gemm_bf16_f32 and gemm_f16_f32 (16-bit A and B, fp32 accumulate)
            on both sizes, against the 2.5 PFLOP/s dense bf16/fp16 peak
  skinny    HBM-bound shapes (1x8192x8192, 8192x1x8192, 8x65536x8192,
            65536x4x8192) on the default path: GB/s of compulsory traffic
            against 8 TB/s

Other modes:
  --profile-run   only run the workload step a few times plus one plain
                  1 GiB device copy (the counter calibration), for rocprofv3;
                  with --epilogue the step is the fused-epilogue call, with
                  --lowp bf16|f16 the 16-bit-input call
  --summarize-profile DIR --out FILE [--kind trace|pmc]
                  condense rocprofv3 CSV output under DIR into a short text
                  summary (used for the files under profiles/)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3      # MI355X dense FP32 (vector packed and matrix)
PEAK_16BIT_TFLOPS = 2500.0    # MI355X dense bf16 / fp16 matrix
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "FP32 GEMM GFLOP/s (2MNK/t) at 2048³ and 8192³; % of FP32 peak"
COPY_BYTES = 1 << 30          # calibration copy in --profile-run
SCLK_MAX_GHZ = 2.4           # MI355X peak shader clock
PROFILES = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILES, "sgemm_mfma_sq8192_pmc.txt")
# The workloads of the five configurations, in order.
CONFIGS = ["micro", "sq1024", "sq2048", "ragged", "sq8192"]


# The sources each path's kernels are compiled from (a summary records the
# hash of its own path's files; the PMC traffic figure is only reported while
# it still describes the kernel that runs).
PATH_SOURCES = {
    "f32": ["sgemm_mfma.hip", "tiles.h", "lds_dma.h", "sgemm_api.hip"],
    "skinny": ["sgemm_skinny.hip", "tiles.h", "sgemm_api.hip"],
    "lowp": ["sgemm_lowp.hip", "tiles.h", "lds_dma.h", "sgemm_api.hip"],
    "valu": ["sgemm_valu.hip", "tiles.h", "sgemm_api.hip"],
    "micro": ["sgemm_micro.hip", "tiles.h", "sgemm_api.hip"],
}


def hash_path(args) -> str:
    """Which path's sources a profile of these arguments describes."""
    from register_lds_tiled_amd import workloads as W
    if args.lowp:
        return "lowp"
    if args.workload == "micro":
        return "micro"
    if (getattr(args, "path", "auto") in ("valu", "valu_page")
            or getattr(args, "valu_tile", None) is not None):
        return "valu"
    return "skinny" if args.workload in W.SKINNY else "f32"


def source_hash(path: str = "f32") -> str:
    """Hash of one path's HIP sources and the ABI header."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "register_lds_tiled_amd", "csrc")
    files = [os.path.join(csrc, n) for n in PATH_SOURCES[path]]
    files.append(os.path.join(ROOT, "include", "sgemm.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- GPU timing --
def setup(workload):
    import torch
    from register_lds_tiled_amd import workloads as W
    w = W.workload(workload)
    A, B = W.inputs_for(w)
    dev = "cuda:0"
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    return w, A, B, dA, dB, dC


def time_path(w, dA, dB, dC, path, steps, warmup):
    """Average ms per step over `steps` timed launches after `warmup`."""
    import torch
    from register_lds_tiled_amd import binding as b
    h = torch.cuda.current_stream().cuda_stream

    def step():
        b.sgemm_f32_path(w.M, w.N, w.K, dA, w.K, dB, w.N, dC, w.N, h, path)

    return time_steps(step, steps, warmup)


def time_ex(w, dA, dB, dC, dbias, steps, warmup):
    """As time_path, for sgemm_f32_ex with every epilogue term on (alpha,
    beta != 0 so C is read, a bias vector, ReLU)."""
    import torch
    from register_lds_tiled_amd import binding as b
    h = torch.cuda.current_stream().cuda_stream

    def step():
        b.sgemm_f32_ex(w.M, w.N, w.K, dA, w.K, dB, w.N, dC, w.N, 0.5, 1.0, dbias, b.ACT_RELU, h)

    return time_steps(step, steps, warmup)


def setup_lowp(workload, fmt):
    """16-bit storage of the workload's inputs on the device (int16 tensors)."""
    import numpy as np
    import torch
    from register_lds_tiled_amd import workloads as W
    w = W.workload(workload)
    A16, B16 = W.lowp_inputs(w.M, w.N, w.K, seed=w.seed, fmt=fmt, dist=w.dist)
    dA = torch.from_numpy(A16.view(np.int16)).to("cuda:0")
    dB = torch.from_numpy(B16.view(np.int16)).to("cuda:0")
    dC = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    return w, dA, dB, dC


def time_lowp(w, dA, dB, dC, fmt, steps, warmup):
    """As time_path, for gemm_bf16_f32 / gemm_f16_f32."""
    import torch
    from register_lds_tiled_amd import binding as b
    h = torch.cuda.current_stream().cuda_stream
    fn = {"bf16": b.gemm_bf16_f32, "f16": b.gemm_f16_f32}[fmt]

    def step():
        fn(w.M, w.N, w.K, dA, w.K, dB, w.N, dC, w.N, h)

    return time_steps(step, steps, warmup)


def lowp_lines(workloads, steps, warmup):
    out = []
    for name in workloads:
        for fmt in ("bf16", "f16"):
            w, dA, dB, dC = setup_lowp(name, fmt)
            n = steps if w.flops > 1e11 else max(steps, 100)
            ms = time_lowp(w, dA, dB, dC, fmt, n, warmup)
            tf = w.flops / (ms * 1e-3) / 1e12
            out.append({"workload": f"gemm {w.M}x{w.N}x{w.K} row-major, {fmt} A and B "
                                    f"(the draws of '{w.describe()}' rounded to {fmt}), "
                                    "fp32 C", "inputs": fmt, "accumulate": "f32",
                        "entry": f"gemm_{fmt}_f32", "value": round(tf * 1e3, 1),
                        "unit": "GFLOP/s", "steps": n, "ms_per_step": round(ms, 4),
                        "roofline": {"bound": "mfma", "achieved": round(tf, 2),
                                     "peak": PEAK_16BIT_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(tf / PEAK_16BIT_TFLOPS, 4)}})
            del dA, dB, dC
    return out


def skinny_lines(steps, warmup):
    """The skinny shapes on the default path: HBM-bound, so the roofline is
    the compulsory traffic 4(MK + KN + MN) bytes per launch against 8 TB/s."""
    import torch
    from register_lds_tiled_amd import binding as b
    from register_lds_tiled_amd import workloads as W
    out = []
    for name, w in W.SKINNY.items():
        A, B = W.inputs_for(w)
        dA = torch.from_numpy(A).to("cuda:0")
        dB = torch.from_numpy(B).to("cuda:0")
        dC = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        ms = time_path(w, dA, dB, dC, b.PATH_AUTO, max(steps, 100), warmup)
        byts = 4.0 * (w.M * w.K + w.K * w.N + w.M * w.N)
        gbs = byts / (ms * 1e-3) / 1e9
        out.append({"workload": w.describe(), "value": round(gbs, 1), "unit": "GB/s",
                    "gflops": round(w.flops / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms, 5),
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                 "bytes_per_launch": byts}})
        del dA, dB, dC
    return out


def epilogue_cost(w, dA, dB, dC, steps, path):
    """Fused epilogue against the plain product on the same buffers, timed
    in alternating blocks (so clock drift hits both alike); medians."""
    import statistics
    import torch
    dbias = torch.linspace(-1.0, 1.0, w.N, dtype=torch.float32, device=dA.device)
    plain, fused = [], []
    for _ in range(3):
        plain.append(time_path(w, dA, dB, dC, path, steps, 1))
        fused.append(time_ex(w, dA, dB, dC, dbias, steps, 1))
    mp, mf = statistics.median(plain), statistics.median(fused)
    return {"workload": w.describe(), "epilogue": "alpha=0.5 beta=1 bias relu",
            "plain_ms": round(mp, 4), "fused_ms": round(mf, 4),
            "fused_gflops": round(w.flops / (mf * 1e-3) / 1e9, 1),
            "overhead_pct": round(100.0 * (mf - mp) / mp, 2),
            "extra_hbm_bytes_algorithmic": 4 * w.M * w.N + 4 * w.N}


def warm(step, warmup):
    """`warmup` untimed steps, then more until 0.25 s have passed (clocks up)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + 0.25
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()


def time_steps(step, steps, warmup):
    """Mean ms per step over `steps` back-to-back steps between two events
    recorded on torch's current stream (the stream the kernels run on)."""
    import torch
    stream = torch.cuda.current_stream()
    warm(step, warmup)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_each(step, reps):
    """ms of each of `reps` launches, each between its own pair of events on
    the launch stream (after time_steps has warmed the same step)."""
    import torch
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, e in evs:
        a.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(e) for a, e in evs]


class SclkSampler:
    """Samples the shader clock with amd-smi in a background thread while a
    GPU loop runs.  Falls back to the sysfs DPM table; records nothing if
    neither is readable."""

    def __init__(self):
        import threading
        self.samples, self.source, self._stop = [], None, threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _amd_smi():
        """Mean over the XCDs of amd-smi's current gfx clocks (MHz): the
        clock.gfx_<n>.clk.value entries of `amd-smi metric --clock --json`."""
        import subprocess
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"],
                           capture_output=True, text=True, timeout=10)
        if r.returncode != 0:
            return None
        d = json.loads(r.stdout)
        gpus = d.get("gpu_data", d) if isinstance(d, dict) else d
        vals = []
        for g in gpus if isinstance(gpus, list) else [gpus]:
            for k, v in (g.get("clock") or {}).items():
                if k.startswith("gfx") and isinstance(v, dict):
                    clk = v.get("clk")
                    val = clk.get("value") if isinstance(clk, dict) else clk
                    if isinstance(val, (int, float)):
                        vals.append(float(val))
        return sum(vals) / len(vals) if vals else None

    @staticmethod
    def _sysfs():
        import re
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            with open(f) as fh:
                for line in fh:
                    if "*" in line:
                        m = re.search(r"([0-9]+)\s*Mhz", line, re.I)
                        if m:
                            return float(m.group(1))
        return None

    def _run(self):
        while not self._stop.is_set():
            v = None
            for src, fn in (("amd-smi metric --clock", self._amd_smi), ("pp_dpm_sclk", self._sysfs)):
                try:
                    v = fn()
                except Exception:   # tool missing or output not understood
                    v = None
                if v:
                    self.source = src
                    break
            if v:
                self.samples.append(v)
            self._stop.wait(0.05)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=15)

    def result(self):
        import statistics
        if not self.samples:
            return None
        return {"median": statistics.median(self.samples), "min": min(self.samples),
                "max": max(self.samples), "samples": len(self.samples), "source": self.source}


def read_pmc_traffic(path=PMC_SUMMARY):
    """(bytes per launch, note) from a committed PMC summary, or (None, why)."""
    if not os.path.exists(path):
        return None, "no PMC summary committed"
    kv = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash():
        return None, "kernel changed since the PMC counters were taken"
    try:
        return float(kv["hbm_bytes_per_launch"]), "FETCH_SIZE+WRITE_SIZE scaled by copy calibration"
    except (KeyError, ValueError):
        return None, "PMC summary incomplete"


def pmc_summary_path(workload):
    return os.path.join(PROFILES, f"sgemm_mfma_{workload}_pmc.txt")


# Products the oracle computes whole within seconds (2048^3 included).
FULL_LIMIT = 1.3e10


def measure_config(name, path, steps, warmup):
    """Time one configuration on the GPU: the mean of back-to-back launches
    (its `value`), then each launch between its own events (median, best).
    C starts as NaN; the C the timed launches wrote is returned for the
    oracle's check.  Returns (entry, workload, A, B, C, device buffers)."""
    import statistics
    import torch
    from register_lds_tiled_amd import binding as b
    w, A, B, dA, dB, dC = setup(name)
    dC.fill_(float("nan"))
    h = torch.cuda.current_stream().cuda_stream
    if name == "micro":
        def step():
            b.sgemm_micro4x4_f32(w.K, dA, dB, dC, h)
        reps = 1000
    else:
        def step():
            b.sgemm_f32_path(w.M, w.N, w.K, dA, w.K, dB, w.N, dC, w.N, h, path)
        reps = steps if w.flops > 1e11 else max(steps, 200)
    mean = time_steps(step, reps, warmup)
    each = sorted(time_each(step, reps))
    med, best = statistics.median(each), each[0]
    C = dC.cpu().numpy()
    e = {"config": name, "workload": w.describe(), "M": w.M, "N": w.N, "K": w.K, "reps": reps}
    if name == "micro":
        e.update({"unit": "us", "value": round(mean * 1e3, 2), "mean_us": round(mean * 1e3, 2),
                  "median_us": round(med * 1e3, 2), "best_us": round(best * 1e3, 2),
                  "roofline": {"bound": "latency",
                               "note": "one thread, 32,768 flops over 32,832 bytes: "
                                       "launch latency, not a roofline fraction"}})
    else:
        def tf(ms):
            return w.flops / (ms * 1e-3) / 1e12
        traffic, note = read_pmc_traffic(pmc_summary_path(name))
        e.update({"unit": "GFLOP/s", "value": round(tf(mean) * 1e3, 1),
                  "mean_ms": round(mean, 5), "median_ms": round(med, 5), "best_ms": round(best, 5),
                  "gflops_median": round(tf(med) * 1e3, 1), "gflops_best": round(tf(best) * 1e3, 1),
                  "roofline": {"bound": "mfma", "achieved": round(tf(mean), 2),
                               "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(tf(mean) / PEAK_FP32_TFLOPS, 4),
                               "frac_median": round(tf(med) / PEAK_FP32_TFLOPS, 4),
                               "traffic": traffic, "traffic_note": note}})
    return e, w, A, B, C, (dA, dB, dC, step)


def cpu_leg(w, A, B, C):
    """The CPU baseline of one configuration -- the oracle as it stands,
    timed on this host -- and, with the oracle's values it produced (plus
    untimed columns and entries at 8192^3), the check of the C that the
    timed GPU launches wrote.  Returns (cpu_baseline, check)."""
    import numpy as np
    import oracle
    from register_lds_tiled_amd import workloads as W
    threads = oracle.num_threads()
    rule = "max|C - C_ref| <= 1e-4 max|C_ref| over the compared outputs, no NaN"
    if w.name == "micro":
        n = 1000
        t0 = time.perf_counter()
        for _ in range(n):
            R = oracle.micro4x4_seq_fma_f32(A, B)
        dt = (time.perf_counter() - t0) / n
        exact = bool(np.array_equal(C.view(np.uint32), R.view(np.uint32)))
        ok, err, ref, tol = oracle.parity(C, oracle.sgemm_ref_f64(A, B))
        cpu = {"value": round(dt * 1e6, 2), "unit": "us", "cores": 1, "kind": "oracle",
               "sample": "the whole 4x4x1024 product: one thread, fp32 fused multiply-add "
                         "in ascending k, mean of 1000 calls (ctypes call included)"}
        check = {"ok": exact and ok, "bit_exact_vs_oracle_fp32_fma": exact,
                 "max_abs_diff_vs_f64": err, "tol": tol, "compared": 16, "of": 16,
                 "C0": [float("%.6f" % v) for v in C[0]]}
        return cpu, check
    if w.M * w.N * w.K <= FULL_LIMIT:
        t0 = time.perf_counter()
        R = oracle.sgemm_ref_f64(A, B)
        dt = time.perf_counter() - t0
        ok, err, ref, tol = oracle.parity(C, R)
        cpu = {"value": round(w.flops / dt / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
               "kind": "oracle", "sample": f"the whole product, fp64 ascending-k sums, "
                                           f"{dt:.2f} s wall"}
        check = {"ok": bool(ok), "max_abs_diff": err, "tol": tol, "max_abs_ref": ref,
                 "compared": w.M * w.N, "of": w.M * w.N, "rule": rule}
        return cpu, check
    rows, cols, er, ec = W.tile_samples(w.M, w.N, seed=4242)
    t0 = time.perf_counter()
    R_rows = oracle.sgemm_ref_f64(A[rows], B)
    dt = time.perf_counter() - t0
    R_cols = oracle.sgemm_ref_f64(A, np.ascontiguousarray(B[:, cols]))
    R_e = oracle.sgemm_ref_f64_entries(A, B, er, ec)
    unwritten = int(np.isnan(C).sum())
    got = np.concatenate([C[rows].ravel(), C[:, cols].ravel(), C[er, ec]])
    exp = np.concatenate([R_rows.ravel(), R_cols.ravel(), R_e])
    ok, err, ref, tol = oracle.parity(got, exp)
    cpu = {"value": round(2.0 * len(rows) * w.N * w.K / dt / 1e9, 3), "unit": "GFLOP/s",
           "cores": threads, "kind": "oracle",
           "sample": f"{len(rows)} whole rows of the {w.M}x{w.N}x{w.K} product (one per "
                     f"128-row band; all columns, full K), fp64 ascending-k sums, "
                     f"{dt:.1f} s wall"}
    check = {"ok": bool(ok) and unwritten == 0, "max_abs_diff": err, "tol": tol,
             "max_abs_ref": ref, "compared": int(got.size), "of": w.M * w.N,
             "unwritten": unwritten, "rule": rule,
             "samples": "a row and a column in each 128 band, an entry in each 64x64 tile; "
                        "every output checked written"}
    return cpu, check


def bench(args):
    import torch
    from register_lds_tiled_amd import binding as b
    torch.cuda.set_device(0)
    path = b.PATHS[args.path]

    # The five configurations; the headline is the 8192^3 one (args.workload).
    configs, keep = [], {}
    sclk = None
    paths = {"mfma": {}, "valu": {}, "valu_page": {}}
    epi = []
    head = sec = None
    for name in CONFIGS:
        steps = args.steps if name == args.workload else max(args.steps, 100)
        e, w, A, B, C, (dA, dB, dC, step) = measure_config(name, path, steps, args.warmup)
        configs.append(e)
        keep[name] = (w, A, B, C)
        if name == args.workload:
            head = e
            # the shader clock while this step runs back to back for ~1.5 s
            with SclkSampler() as smp:
                t_end = time.perf_counter() + 1.5
                while time.perf_counter() < t_end:
                    for _ in range(10):
                        step()
                    torch.cuda.synchronize()
            sclk = smp.result()
        if name in (args.workload, args.secondary):
            for pname in paths:
                pms = e["mean_ms"] if b.PATHS[pname] == path else time_path(
                    w, dA, dB, dC, b.PATHS[pname], max(2, steps // 4), 2)
                paths[pname][name] = round(w.flops / (pms * 1e-3) / 1e9, 1)
            epi.append(epilogue_cost(w, dA, dB, dC, max(5, steps // 2), path))
        if name == args.secondary:
            sec = {"workload": w.describe(), "value": e["value"], "unit": "GFLOP/s",
                   "steps": e["reps"], "ms_per_step": e["mean_ms"],
                   "frac_of_fp32_peak": e["roofline"]["frac"]}
        del dA, dB, dC, step
        torch.cuda.empty_cache()

    lowp = lowp_lines([args.workload, args.secondary], args.steps, args.warmup)
    skinny = skinny_lines(args.steps, args.warmup)

    # CPU legs last, so the GPU timings above never follow an idle spell.
    cpu = None
    if not args.no_cpu_baseline:
        for e in configs:
            w, A, B, C = keep[e["config"]]
            e["cpu_baseline"], e["check"] = cpu_leg(w, A, B, C)
        cpu = head["cpu_baseline"]

    w = W_of(args.workload)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": head["reps"],
        "warmup": args.warmup,
        "ms_per_step": head["mean_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.describe(), "M": w.M, "N": w.N, "K": w.K,
                   "path": args.path, "device": torch.cuda.get_device_name(0)},
        "roofline": {k: v for k, v in head["roofline"].items() if k != "frac_median"},
        "cpu_baseline": cpu,
        "check": head.get("check"),
        "sclk_mhz": sclk,
        "configs": configs,
        "secondary": sec,
        "paths": paths,
        "fused_epilogue": epi,
        "lowp": lowp,
        "skinny": skinny,
    }
    print(json.dumps(line), flush=True)


def valu_sweep(args):
    """Every VALU tile configuration (sgemm_f32_valu_tile) on square and
    ragged shapes, interleaved in rounds so clock drift hits all alike:
    median GFLOP/s per configuration and shape.  One JSON line."""
    import statistics
    import torch
    from register_lds_tiled_amd import binding as b
    from register_lds_tiled_amd import workloads as W
    torch.cuda.set_device(0)
    shapes = [(8192, 8192, 8192), (4096, 4096, 4096), (3072, 3072, 3072), (2048, 2048, 2048),
              (1536, 1536, 1536), (1024, 1024, 1024), (1000, 1500, 777)]
    tiles = b.valu_tiles()
    out = {"sweep": "valu tiles", "unit": "GFLOP/s", "tiles": tiles, "results": {}}
    h = torch.cuda.current_stream().cuda_stream
    for (M, N, K) in shapes:
        A, B = W.random_inputs(M, N, K, seed=M + N + K)
        dA, dB = torch.from_numpy(A).to("cuda:0"), torch.from_numpy(B).to("cuda:0")
        dC = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        flops = 2.0 * M * N * K
        reps = max(3, min(200, int(2e12 / flops)))
        res = {t: [] for t in tiles}
        for _ in range(3):
            for t in tiles:
                ms = time_steps(lambda: b.sgemm_f32_valu_tile(M, N, K, dA, K, dB, N, dC, N, h, t),
                                reps, 1)
                res[t].append(flops / (ms * 1e-3) / 1e9)
        key = f"{M}x{N}x{K}"
        out["results"][key] = {t: round(statistics.median(v), 1) for t, v in res.items()}
        print(f"# {key}: " + ", ".join(f"{t}:{v:.0f}" for t, v in out["results"][key].items()),
              file=sys.stderr, flush=True)
        del dA, dB, dC
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def W_of(name):
    from register_lds_tiled_amd import workloads as W
    return W.workload(name)


def profile_run(args):
    """A short fixed run for rocprofv3: warmup + N launches of the workload
    step, then one plain device copy of COPY_BYTES (counter calibration)."""
    import torch
    from register_lds_tiled_amd import binding as b
    torch.cuda.set_device(0)
    if args.lowp:
        w, dA, dB, dC = setup_lowp(args.workload, args.lowp)
        time_lowp(w, dA, dB, dC, args.lowp, args.steps, args.warmup)
    elif args.epilogue:
        w, _, _, dA, dB, dC = setup(args.workload)
        dbias = torch.linspace(-1.0, 1.0, w.N, dtype=torch.float32, device=dA.device)
        time_ex(w, dA, dB, dC, dbias, args.steps, args.warmup)
    elif args.valu_tile is not None:
        w, _, _, dA, dB, dC = setup(args.workload)
        h = torch.cuda.current_stream().cuda_stream
        time_steps(lambda: b.sgemm_f32_valu_tile(w.M, w.N, w.K, dA, w.K, dB, w.N, dC, w.N, h,
                                                 args.valu_tile), args.steps, args.warmup)
    elif args.workload == "micro":
        w, _, _, dA, dB, dC = setup(args.workload)
        h = torch.cuda.current_stream().cuda_stream
        time_steps(lambda: b.sgemm_micro4x4_f32(w.K, dA, dB, dC, h), args.steps, args.warmup)
    else:
        w, _, _, dA, dB, dC = setup(args.workload)
        time_path(w, dA, dB, dC, b.PATHS[args.path], args.steps, args.warmup)
    del dA, dB, dC
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": args.workload,
                      "path": (f"gemm_{args.lowp}_f32" if args.lowp else
                               "fused epilogue" if args.epilogue else
                               f"valu tile {args.valu_tile}" if args.valu_tile is not None
                               else args.path),
                      "steps": args.steps,
                      "warmup": args.warmup, "copy_bytes": COPY_BYTES,
                      "source_sha256": source_hash(hash_path(args))}), flush=True)


# -------------------------------------------------------- profile summaries --
def _csvs(root, suffix):
    return sorted(glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True))


MOPS_COUNTER = {None: "SQ_INSTS_VALU_MFMA_MOPS_F32", "bf16": "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                "f16": "SQ_INSTS_VALU_MFMA_MOPS_F16"}
# Counter passes, one rocprofv3 run each (at most 8 SQ and 4 TCC counters).
PMC_SETS = {
    "mfma": {
        1: "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
           "{mops} SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
        2: "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
           "SQ_ACTIVE_INST_VMEM SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE",
        3: "FETCH_SIZE",
        4: "WRITE_SIZE TCC_HIT_sum TCC_MISS_sum",
    },
    "valu": {
        1: "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_VALU_FMA_F32 "
           "SQ_ACTIVE_INST_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE",
        2: "SQ_WAIT_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_LDS_IDX_ACTIVE "
           "SQ_THREAD_CYCLES_VALU SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR GRBM_GUI_ACTIVE",
        3: "FETCH_SIZE",
        4: "WRITE_SIZE TCC_HIT_sum TCC_MISS_sum",
    },
}
CU_NUM, SIMD_NUM = 256, 1024


def _agent_value(run_dir, key, default):
    """A field of the GPU agent in a rocprofv3 run's agent_info.csv."""
    for f in _csvs(run_dir, "agent_info.csv"):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r.get("Name", "").startswith("gfx") and r.get(key, "").strip():
                    try:
                        return int(float(r[key]))
                    except ValueError:
                        pass
    return default


def pmc_tag(workload, lowp=None, path="auto", valu_tile=None):
    """Directory tag of one workload's counter passes: pmc<n>_<tag>/."""
    if lowp:
        return f"{lowp}_{workload}"
    if valu_tile is not None:
        return f"valutile{valu_tile}_{workload}"
    if path in ("valu", "valu_page"):
        return f"{path}_{workload}"
    return workload


def summarize_pmc(root, workload, lowp=None, path="auto", valu_tile=None):
    """Condense the four counter passes pmc{1..4}_<tag>/ under root (tag:
    pmc_tag), each a `--profile-run` of this script, into derived figures for
    the last three launches of the GEMM kernel.  The 1 GiB device copy at
    the end of each run calibrates FETCH_SIZE and WRITE_SIZE."""
    from register_lds_tiled_amd import workloads as W
    w = W.workload(workload)
    tag = pmc_tag(workload, lowp, path, valu_tile)
    kind = "valu" if path in ("valu", "valu_page") or valu_tile is not None else "mfma"
    passes = PMC_SETS[kind]
    mops = MOPS_COUNTER[lowp]
    esize = 2 if lowp else 4

    def per_dispatch(n):
        f = _csvs(os.path.join(root, f"pmc{n}_{tag}"), "counter_collection.csv")[0]
        per = {}
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                d = per.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                d["dur_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        return per

    P = {n: per_dispatch(n) for n in passes}
    what = f"{lowp} A and B, " if lowp else ""
    where = f"VALU tile {valu_tile}" if valu_tile is not None else f"path {path}"
    out = [f"# passes ({what}{w.describe()}, {where}):"]
    extra = ((f"--lowp {lowp} " if lowp else "") + (f"--path {path} " if path != "auto" else "")
             + (f"--valu-tile {valu_tile} " if valu_tile is not None else ""))
    for n, c in passes.items():
        out.append(f"#   cd /tmp && rocprofv3 --pmc {c.format(mops=mops)} -d <repo>/{root}/pmc{n}_{tag} "
                   f"-o pmc --output-format csv -- python3 <repo>/bench.py --profile-run "
                   f"{extra}--workload {workload} --steps 3 --warmup 1")
    last = {n: [k for k, d in P[n].items() if "gemm" in d["kernel"]][-3:] for n in P}
    copy = {n: [k for k, d in P[n].items() if "copyBuffer" in d["kernel"]][-1] for n in (3, 4)}
    avg = lambda n, c: sum(P[n][k][c] for k in last[n]) / len(last[n])  # noqa: E731
    out.append(f"kernel: {P[1][last[1][-1]]['kernel']}")
    kib = COPY_BYTES / 1024
    ff, wf = P[3][copy[3]]["FETCH_SIZE"] / kib, P[4][copy[4]]["WRITE_SIZE"] / kib
    out.append(f"copy_calibration: 1 GiB device copy reads FETCH_SIZE "
               f"{P[3][copy[3]]['FETCH_SIZE']:.0f} KiB (factor {ff:.3f}) and WRITE_SIZE "
               f"{P[4][copy[4]]['WRITE_SIZE']:.0f} KiB (factor {wf:.3f})")
    fetch = avg(3, "FETCH_SIZE") * 1024 / ff
    write = avg(4, "WRITE_SIZE") * 1024 / wf
    out.append(f"fetch_kib_per_launch: {avg(3, 'FETCH_SIZE'):.0f}")
    out.append(f"write_kib_per_launch: {avg(4, 'WRITE_SIZE'):.0f}")
    out.append(f"hbm_bytes_per_launch: {fetch + write:.4g}")
    dur3 = sum(P[3][k]["dur_ns"] for k in last[3]) / len(last[3])
    out.append(f"hbm_rate: {(fetch + write) / dur3:.4g} GB/s (those bytes over the "
               f"profiled {dur3 / 1e3:.1f} us of the FETCH_SIZE pass)")
    out.append(f"compulsory_bytes: {esize * (w.M * w.K + w.K * w.N) + 4.0 * w.M * w.N:.4g} "
               "(A and B read once, C written once)")
    # Cycles of the kernel: its own span in this pass times the clock.  The
    # GPU-busy counter (largest over the 8 XCDs) counts over a window that
    # can be longer than a short kernel, which would read as a clock above
    # the chip's maximum; the clock is then taken as the maximum, so the
    # utilisations below are lower bounds.
    gui = max(P[1][k]["GRBM_GUI_ACTIVE"] for k in last[1]) / 8
    dur = sum(P[1][k]["dur_ns"] for k in last[1]) / len(last[1])
    raw_ghz = gui / dur
    ghz = min(raw_ghz, SCLK_MAX_GHZ)
    cyc = dur * ghz
    out.append(f"gpu_busy_cycles_per_xcd: {gui:.4g} over the kernel's {dur / 1e3:.1f} us "
               f"(profiled) -> {raw_ghz:.3f} GHz")
    if raw_ghz > SCLK_MAX_GHZ:
        out.append(f"clock_note: {raw_ghz:.3f} GHz exceeds the {SCLK_MAX_GHZ} GHz maximum: the "
                   "busy counter spans more than the kernel; kernel cycles are taken as "
                   f"{dur / 1e3:.1f} us x {SCLK_MAX_GHZ} GHz, so the utilisations are lower bounds")
    out.append(f"kernel_cycles: {cyc:.4g} ({dur / 1e3:.1f} us at {ghz:.3f} GHz)")
    # SQ_BUSY_CYCLES sums, over the shader engines, the cycles in which an SE
    # holds a wave of the kernel: per SE it is the kernel's active time in
    # cycles, without the counter window's slack.
    se_num = _agent_value(os.path.join(root, f"pmc1_{tag}"), "Num_Shader_Banks", 32)
    busy = avg(1, "SQ_BUSY_CYCLES") / se_num
    out.append(f"se_busy_cycles: {busy:.4g} per shader engine ({se_num} SEs; "
               f"{100 * busy / cyc:.1f} % of kernel_cycles)")
    if kind == "mfma":
        mfma_busy = avg(1, "SQ_VALU_MFMA_BUSY_CYCLES")
        out.append(f"MfmaUtil_pct: {100 * mfma_busy / (cyc * SIMD_NUM):.1f} (over kernel_cycles; "
                   f"{100 * mfma_busy / (busy * SIMD_NUM):.1f} over se_busy_cycles)")
        out.append(f"mfma_{lowp or 'f32'}_flops: {avg(1, mops) * 512:.4g} (2MNK = {w.flops:.4g})")
        out.append(f"lds_instructions: {avg(1, 'SQ_INSTS_LDS'):.4g}  vmem_rd: "
                   f"{avg(2, 'SQ_INSTS_VMEM_RD'):.4g}  vmem_wr: {avg(2, 'SQ_INSTS_VMEM_WR'):.4g}")
        out.append(f"wait_lds_pct_of_wave_cycles: "
                   f"{100 * avg(1, 'SQ_WAIT_INST_LDS') / avg(1, 'SQ_WAVE_CYCLES'):.1f}")
    else:
        fma = avg(1, "SQ_INSTS_VALU_FMA_F32")
        out.append(f"valu_fma_f32_flops: {fma * 64 * 2:.4g} (wave64 FMA instructions x 128; "
                   f"2MNK = {w.flops:.4g})")
        out.append(f"valu_instructions: {avg(1, 'SQ_INSTS_VALU'):.4g} (FMA share "
                   f"{100 * fma / avg(1, 'SQ_INSTS_VALU'):.1f} %)")
        # fp32 FMA peak: 256 flop per clock per CU (64 lanes x 2 flop every
        # two clocks on each of 4 SIMDs)
        out.append(f"FmaRate_pct_of_peak_at_clock: {100 * fma * 128 / (cyc * CU_NUM * 256):.1f} "
                   f"(over kernel_cycles; {100 * fma * 128 / (busy * CU_NUM * 256):.1f} over "
                   "se_busy_cycles)")
        # lanes enabled per VALU instruction cycle (64 = the whole wave):
        # a lane-occupancy figure, not a share of time
        out.append(f"VALU_lanes_active_pct: {100 * avg(2, 'SQ_THREAD_CYCLES_VALU') / (avg(1, 'SQ_ACTIVE_INST_VALU') * 64):.1f}")
        out.append(f"lds_instructions: {avg(1, 'SQ_INSTS_LDS'):.4g} ({avg(1, 'SQ_INSTS_LDS') / fma:.3f} "
                   f"per FMA instruction)  salu: {avg(2, 'SQ_INSTS_SALU'):.4g}  vmem_rd: "
                   f"{avg(2, 'SQ_INSTS_VMEM_RD'):.4g}  vmem_wr: {avg(2, 'SQ_INSTS_VMEM_WR'):.4g}")
        out.append(f"wait_lds_pct_of_wave_cycles: "
                   f"{100 * avg(2, 'SQ_WAIT_INST_LDS') / avg(1, 'SQ_WAVE_CYCLES'):.1f}")
    out.append(f"LdsUtil_pct: {100 * avg(2, 'SQ_LDS_IDX_ACTIVE') / (cyc * CU_NUM):.1f}")
    out.append(f"LDSBankConflict_pct: {100 * avg(1, 'SQ_LDS_BANK_CONFLICT') / (cyc * CU_NUM):.2f}")
    out.append(f"waves: {avg(1, 'SQ_WAVES'):.0f}  se_busy_cycles_sum: {avg(1, 'SQ_BUSY_CYCLES'):.4g} "
               f"({avg(1, 'SQ_BUSY_CYCLES') / cyc:.1f} x kernel_cycles)")
    h, m = avg(4, "TCC_HIT_sum"), avg(4, "TCC_MISS_sum")
    out.append(f"L2_hit_pct: {100 * h / (h + m):.1f}")
    out.append(f"wait_any_pct_of_wave_cycles: "
               f"{100 * avg(2, 'SQ_WAIT_ANY') / avg(1, 'SQ_WAVE_CYCLES'):.1f}")
    return out


def profiled_hash(args):
    """The source hash the profiled run printed (--profile-run's JSON line in
    a pass log next to the counter output), else the tree's own."""
    from register_lds_tiled_amd import workloads as W  # noqa: F401
    root = args.summarize_profile
    logs = []
    if args.kind == "pmc":
        tag = pmc_tag(args.workload, args.lowp, args.path, args.valu_tile)
        logs = [os.path.join(root, f"pmc{n}_{tag}.log") for n in (1, 2, 3, 4)]
    else:
        # the trace run's own log sits beside its directory (<dir>.log)
        logs = [root.rstrip("/") + ".log"] + sorted(glob.glob(os.path.join(root, "*.log")))
    for f in logs:
        if os.path.exists(f):
            with open(f, encoding="utf-8", errors="replace") as fh:
                for line in fh:
                    if line.startswith("{") and '"source_sha256"' in line:
                        try:
                            return json.loads(line)["source_sha256"]
                        except ValueError:
                            pass
    return source_hash(hash_path(args))


def summarize(args):
    out = []
    cmd = args.command or "(command not recorded)"
    out.append(f"# rocprofv3 summary ({args.kind}); summarized by: python bench.py "
               f"--summarize-profile {args.summarize_profile} --kind {args.kind} "
               + (f"--lowp {args.lowp} " if args.lowp else "")
               + (f"--path {args.path} " if args.path != "auto" else "")
               + (f"--valu-tile {args.valu_tile} " if args.valu_tile is not None else "")
               + f"--workload {args.workload} --steps {args.steps}")
    if args.kind == "trace":
        out.append(f"# profiled command: {cmd}")
    out.append(f"source_sha256: {profiled_hash(args)}")
    if args.kind == "trace":
        for f in _csvs(args.summarize_profile, "kernel_trace.csv"):
            per = {}
            with open(f, newline="") as fh:
                for r in csv.DictReader(fh):
                    per.setdefault(r["Kernel_Name"], []).append(r)
            out.append(f"# per kernel: all dispatches, then the last --steps={args.steps} "
                       "dispatches (the timed window of a run with that many steps)")
            for name, rs in per.items():
                d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs]
                last = d[-args.steps:]
                r0 = rs[-1]
                out.append(f"kernel: {name}")
                out.append(f"  dispatches {len(d)} | avg_ns_all {sum(d) / len(d):.0f} | "
                           f"avg_ns_last{len(last)} {sum(last) / len(last):.0f} | "
                           f"min_ns {min(d)} | max_ns {max(d)}")
                # (register counts are left out: for these gfx950 code
                # objects the trace's VGPR field reads half the unified
                # register allocation and its AGPR field 0; the compiler's
                # own report is the figure to use)
                out.append(f"  grid {r0.get('Grid_Size_X')} x {r0.get('Grid_Size_Y')} | "
                           f"workgroup {r0.get('Workgroup_Size_X')} | lds_bytes "
                           f"{r0.get('LDS_Block_Size')} | scratch {r0.get('Scratch_Size')}")
        for f in _csvs(args.summarize_profile, "kernel_stats.csv"):
            with open(f, newline="") as fh:
                rows = list(csv.DictReader(fh))
            out.append("# kernel, calls, average_ns, min_ns, max_ns, total_ns, percent")
            for r in rows:
                out.append(f"kernel: {r.get('Name')} | calls {r.get('Calls')} | avg_ns "
                           f"{r.get('AverageNs')} | min_ns {r.get('MinNs')} | max_ns "
                           f"{r.get('MaxNs')} | total_ns {r.get('TotalDurationNs')} | pct "
                           f"{r.get('Percentage')}")
    else:
        out.extend(summarize_pmc(args.summarize_profile, args.workload, args.lowp, args.path,
                                 args.valu_tile))
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w", encoding="utf-8") as fh:
            fh.write(text)
    print(text, end="")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sq8192")
    ap.add_argument("--secondary", default="sq2048")
    ap.add_argument("--path", default="auto", choices=["auto", "mfma", "valu", "valu_page"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--lowp", choices=["bf16", "f16"], default=None,
                    help="with --profile-run: run the 16-bit-input entry point")
    ap.add_argument("--epilogue", action="store_true",
                    help="with --profile-run: run sgemm_f32_ex (alpha, beta, bias, ReLU)")
    ap.add_argument("--valu-sweep", action="store_true",
                    help="time every VALU tile configuration on square and ragged shapes")
    ap.add_argument("--valu-tile", type=int, default=None,
                    help="with --profile-run: run sgemm_f32_valu_tile at this configuration")
    ap.add_argument("--summarize-profile", default=None)
    ap.add_argument("--kind", default="trace", choices=["trace", "pmc"])
    ap.add_argument("--command", default=None)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    if args.summarize_profile:
        summarize(args)
        return 0
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not "
              "supported (the product shards trivially by C row panels, but no multi-GPU "
              "path is built)", file=sys.stderr)
        return 2
    if args.valu_sweep:
        valu_sweep(args)
    elif args.profile_run:
        profile_run(args)
    else:
        bench(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
