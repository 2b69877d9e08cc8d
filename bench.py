"""Benchmark of the fp32 row-major SGEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sq8192]
                    [--path auto] [--cpu-seconds S] [--no-cpu-baseline]

A step is one C = A.B call through the C ABI (sgemm_f32_path) on inputs
already resident in HBM: the whole hot path (tile loader, LDS staging,
register/matrix-core micro-kernel, store) over one product.  W untimed
steps, then exactly K timed steps between torch.cuda.synchronize() calls,
timed with HIP events recorded on the stream the kernels are launched on.
Prints ONE JSON line:

  value     GFLOP/s = 2*M*N*K / (average step time)
  roofline  the (only) kernel of the step against the FP32 matrix peak of
            157.3 TFLOP/s: achieved = 2*M*N*K / average launch time;
            traffic = HBM bytes per launch from the committed rocprofv3 PMC
            summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
            size), or null if the kernel sources changed since it was taken
  cpu_baseline  the CPU oracle (fp64, OpenMP) timed on this host on the first
            R rows of the same product, R sized to about --cpu-seconds
  secondary the same measurement at 2048^3 (the metric names both sizes)
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
PROFILES = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILES, "sgemm_mfma_sq8192_pmc.txt")


# The sources each path's kernels are compiled from (a summary records the
# hash of its own path's files; the PMC traffic figure is only reported while
# it still describes the kernel that runs).
PATH_SOURCES = {
    "f32": ["sgemm_mfma.hip", "tiles.h", "lds_dma.h", "sgemm_api.hip"],
    "skinny": ["sgemm_skinny.hip", "tiles.h", "sgemm_api.hip"],
    "lowp": ["sgemm_lowp.hip", "tiles.h", "lds_dma.h", "sgemm_api.hip"],
}


def hash_path(args) -> str:
    """Which path's sources a profile of these arguments describes."""
    from register_lds_tiled_amd import workloads as W
    if args.lowp:
        return "lowp"
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


def time_steps(step, steps, warmup):
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Bring the clocks up before timing: keep warming for at least 0.25 s.
    t_end = time.perf_counter() + 0.25
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def read_pmc_traffic():
    """(bytes per launch, note) from the committed PMC summary, or (None, why)."""
    if not os.path.exists(PMC_SUMMARY):
        return None, "no PMC summary committed"
    kv = {}
    with open(PMC_SUMMARY, encoding="utf-8") as f:
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


def cpu_baseline(A, B, target_s):
    """Time the oracle on the first R rows of A.B, R sized to ~target_s."""
    import oracle
    threads = oracle.num_threads()
    dt1, fl1 = oracle.timed_rows(A, B, threads)        # one row per thread
    rows = max(threads, int(threads * max(1.0, target_s / max(dt1, 1e-3))))
    rows = min(rows - rows % threads if rows >= threads else rows, A.shape[0])
    dt, fl = oracle.timed_rows(A, B, rows)
    return {"value": round(fl / dt / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {rows} rows of the {A.shape[0]}x{B.shape[1]}x{A.shape[1]} "
                      f"product (all columns, full K), fp64 ascending-k sums, "
                      f"{dt:.1f} s wall"}


def bench(args):
    import torch
    from register_lds_tiled_amd import binding as b
    torch.cuda.set_device(0)
    path = b.PATHS[args.path]

    w, A, B, dA, dB, dC = setup(args.workload)
    ms = time_path(w, dA, dB, dC, path, args.steps, args.warmup)
    gflops = w.flops / (ms * 1e-3) / 1e9
    achieved = w.flops / (ms * 1e-3) / 1e12
    traffic, traffic_note = read_pmc_traffic()

    paths = {}
    for name in ("mfma", "valu", "valu_page"):
        pms = ms if b.PATHS[name] == path else time_path(
            w, dA, dB, dC, b.PATHS[name], max(2, args.steps // 4), 2)
        paths[name] = {args.workload: round(w.flops / (pms * 1e-3) / 1e9, 1)}

    epi = [epilogue_cost(w, dA, dB, dC, max(5, args.steps // 2), path)]

    sec = None
    if args.secondary and args.secondary != args.workload:
        w2, _, _, dA2, dB2, dC2 = setup(args.secondary)
        steps2 = max(args.steps, 100)
        ms2 = time_path(w2, dA2, dB2, dC2, path, steps2, args.warmup)
        sec = {"workload": w2.describe(), "value": round(w2.flops / (ms2 * 1e-3) / 1e9, 1),
               "unit": "GFLOP/s", "steps": steps2, "ms_per_step": round(ms2, 4),
               "frac_of_fp32_peak": round(w2.flops / (ms2 * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)}
        for name in ("mfma", "valu", "valu_page"):
            pms = ms2 if b.PATHS[name] == path else time_path(
                w2, dA2, dB2, dC2, b.PATHS[name], 20, 2)
            paths[name][args.secondary] = round(w2.flops / (pms * 1e-3) / 1e9, 1)
        epi.append(epilogue_cost(w2, dA2, dB2, dC2, 100, path))
        del dA2, dB2, dC2
    del dA, dB, dC

    lowp = lowp_lines([args.workload] + ([args.secondary] if sec else []), args.steps,
                      args.warmup)
    skinny = skinny_lines(args.steps, args.warmup)

    # CPU oracle last, so the GPU timings above never follow an idle spell.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(A, B, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(gflops, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.describe(), "M": w.M, "N": w.N, "K": w.K,
                   "path": args.path, "device": torch.cuda.get_device_name(0)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                     "traffic": traffic, "traffic_note": traffic_note},
        "cpu_baseline": cpu,
        "secondary": sec,
        "paths": paths,
        "fused_epilogue": epi,
        "lowp": lowp,
        "skinny": skinny,
    }
    print(json.dumps(line), flush=True)


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
                               "fused epilogue" if args.epilogue else args.path),
                      "steps": args.steps,
                      "warmup": args.warmup, "copy_bytes": COPY_BYTES,
                      "source_sha256": source_hash(hash_path(args))}), flush=True)


# -------------------------------------------------------- profile summaries --
def _csvs(root, suffix):
    return sorted(glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True))


MOPS_COUNTER = {None: "SQ_INSTS_VALU_MFMA_MOPS_F32", "bf16": "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                "f16": "SQ_INSTS_VALU_MFMA_MOPS_F16"}
PMC_PASSES = {
    1: "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
       "{mops} SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    2: "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM "
       "SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE",
    3: "FETCH_SIZE",
    4: "WRITE_SIZE TCC_HIT_sum TCC_MISS_sum",
}


def summarize_pmc(root, workload, lowp=None):
    """Condense the four counter passes pmc{1..4}_<workload>/ (for a 16-bit
    run pmc{1..4}_<lowp>_<workload>/) under root, each a `--profile-run` of
    this script, into derived figures for the last three launches of the
    GEMM kernel.  The 1 GiB device copy at the end of each run calibrates
    FETCH_SIZE and WRITE_SIZE."""
    from register_lds_tiled_amd import workloads as W
    w = W.workload(workload)
    tag = f"{lowp}_{workload}" if lowp else workload
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

    P = {n: per_dispatch(n) for n in PMC_PASSES}
    what = f"{lowp} A and B, " if lowp else ""
    out = [f"# passes ({what}{w.describe()}):"]
    extra = f"--lowp {lowp} " if lowp else ""
    for n, c in PMC_PASSES.items():
        out.append(f"#   rocprofv3 --pmc {c.format(mops=mops)} -d {root}/pmc{n}_{tag} -o pmc "
                   f"--output-format csv -- python3 bench.py --profile-run {extra}--workload "
                   f"{workload} --steps 3 --warmup 1")
    last = {n: [k for k, d in P[n].items() if "sgemm" in d["kernel"]][-3:] for n in P}
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
    gui = avg(1, "GRBM_GUI_ACTIVE") / 8          # the counter sums the 8 XCDs
    dur = sum(P[1][k]["dur_ns"] for k in last[1]) / 3
    out.append(f"gpu_busy_cycles_per_xcd: {gui:.4g} over {dur / 1e3:.1f} us "
               f"(profiled) -> {gui / dur:.3f} GHz")
    out.append(f"MfmaUtil_pct: {100 * avg(1, 'SQ_VALU_MFMA_BUSY_CYCLES') / (gui * 1024):.1f}")
    out.append(f"mfma_{lowp or 'f32'}_flops: {avg(1, mops) * 512:.4g} (2MNK = {w.flops:.4g})")
    out.append(f"LdsUtil_pct: {100 * avg(2, 'SQ_LDS_IDX_ACTIVE') / (gui * 256):.1f}")
    out.append(f"LDSBankConflict_pct: {100 * avg(1, 'SQ_LDS_BANK_CONFLICT') / (gui * 256):.2f}")
    out.append(f"lds_instructions: {avg(1, 'SQ_INSTS_LDS'):.4g}  vmem_rd: "
               f"{avg(2, 'SQ_INSTS_VMEM_RD'):.4g}  vmem_wr: {avg(2, 'SQ_INSTS_VMEM_WR'):.4g}")
    h, m = avg(4, "TCC_HIT_sum"), avg(4, "TCC_MISS_sum")
    out.append(f"L2_hit_pct: {100 * h / (h + m):.1f}")
    out.append(f"wait_any_pct_of_wave_cycles: "
               f"{100 * avg(2, 'SQ_WAIT_ANY') / avg(1, 'SQ_WAVE_CYCLES'):.1f}")
    return out


def summarize(args):
    out = []
    cmd = args.command or "(command not recorded)"
    out.append(f"# rocprofv3 summary ({args.kind}); summarized by: python bench.py "
               f"--summarize-profile {args.summarize_profile} --kind {args.kind} "
               + (f"--lowp {args.lowp} " if args.lowp else "")
               + f"--workload {args.workload} --steps {args.steps}")
    if args.kind == "trace":
        out.append(f"# profiled command: {cmd}")
    out.append(f"source_sha256: {source_hash(hash_path(args))}")
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
                out.append(f"  grid {r0.get('Grid_Size_X')} x {r0.get('Grid_Size_Y')} | "
                           f"workgroup {r0.get('Workgroup_Size_X')} | lds_bytes "
                           f"{r0.get('LDS_Block_Size')} | vgpr {r0.get('VGPR_Count')} | "
                           f"agpr {r0.get('Accum_VGPR_Count')} | sgpr {r0.get('SGPR_Count')} | "
                           f"scratch {r0.get('Scratch_Size')}")
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
        out.extend(summarize_pmc(args.summarize_profile, args.workload, args.lowp))
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--lowp", choices=["bf16", "f16"], default=None,
                    help="with --profile-run: run the 16-bit-input entry point")
    ap.add_argument("--epilogue", action="store_true",
                    help="with --profile-run: run sgemm_f32_ex (alpha, beta, bias, ReLU)")
    ap.add_argument("--summarize-profile", default=None)
    ap.add_argument("--kind", default="trace", choices=["trace", "pmc"])
    ap.add_argument("--command", default=None)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    if args.summarize_profile:
        summarize(args)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the product shards trivially by C row panels, but no multi-GPU "
              "path is built)", file=sys.stderr)
        return 2
    if args.profile_run:
        profile_run(args)
    else:
        bench(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
