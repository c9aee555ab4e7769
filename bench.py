#!/usr/bin/env python3
"""Benchmark of the dense GEMM library on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c2|c1|c3|c4|c5|flat16|...]

A step is one call of the library (dg_gemm through the C ABI) on one
workload whose operands are already resident in HBM: scheduler, loader,
inner loop, epilogue (and split-K reduction when planned) all run inside the
timed region.  Timing uses HIP events recorded on the stream the kernels are
launched on, after W untimed warm-up steps, bracketed by device
synchronisation.  Throughput is TFLOPS = 2MNK / t ("GEMM Kernel
Optimization", Verification).

The default workload is the fp32 SGEMM at M = N = K = 4096; the bf16 GEMM at
4096^3 (the other half of the headline metric) is measured in the same run
and reported under "secondary".  The CPU oracle is timed on a bounded,
seeded sample of the same workload's output elements on this host's cores.

Prints exactly one JSON line on stdout; progress goes to stderr.
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

METRIC = "TFLOPS=2MNK/t at 4096³ bf16 & fp32, as % of MI355X MFMA/FP32 peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _dtype_name(p):
    return p.a_type


def _roofline_peak(p, kernel):
    """(bound, peak) of the workload's dominant kernel: its compute peak
    (matrix cores for the MFMA kernels, the unpacked vector-FMA rate for
    the others), or HBM when the algorithmic bytes take longer at 8 TB/s
    than the flops at that peak."""
    from dense_gemm_10_amd import accounting as acc
    if kernel.startswith("mfma_bf16"):
        bound, peak = "mfma", acc.PEAK_BF16_MFMA
    elif kernel.startswith("mfma_f16"):
        bound, peak = "mfma", acc.PEAK_F16_MFMA
    elif kernel.startswith("mfma_f32"):
        bound, peak = "mfma", acc.PEAK_F32
    else:
        bound, peak = "alu", acc.PEAK_F32_VALU_UNPACKED
    if acc.problem_bytes(p) / acc.PEAK_HBM > acc.problem_flops(p) / peak:
        return "hbm", acc.PEAK_HBM
    return bound, peak


def time_workload(name, steps, warmup, **desc_overrides):
    """Run one workload: returns dict with ms/step, TFLOPS, plan string."""
    import torch
    import workloads as W
    from workloads.device import DeviceProblem
    p = W.WORKLOADS[name]
    log(f"[bench] {name}: generating {p.name}")
    x = W.make_inputs(p)
    dp = DeviceProblem(p, x, **desc_overrides)
    plan = dp.describe()
    log(f"[bench] {name}: plan {plan}")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        dp.run(stream.cuda_stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        dp.run(stream.cuda_stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = p.flops()
    return dict(problem=p, inputs=x, ms=ms, tflops=flops / (ms * 1e-3) / 1e12, plan=plan,
                kernel=plan.split()[0].split("=")[1])


def time_copy(steps, warmup, nbytes=512 << 20):
    """Plain device-to-device copy of nbytes (torch's copy kernel): the
    reference for the achievable HBM rate and for scaling the FETCH_SIZE /
    WRITE_SIZE counters (it reads and writes exactly nbytes per step)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        dst.copy_(src)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms,
            "gbps_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}


PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    """Hash of every HIP / C++ source of the library: a profile taken with a
    different hash describes other kernels."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_10_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _rocprof(args, outdir, timeout_s=150):
    """Run rocprofv3 (killed after timeout_s) on a child bench.py; returns
    the CSV rows of the first *<suffix>.csv it produced."""
    import shutil
    import subprocess
    shutil.rmtree(outdir, ignore_errors=True)
    cmd = ["timeout", "-s", "KILL", str(timeout_s), "rocprofv3"] + args + [
        "-f", "csv", "-d", outdir, "-o", "run", "--", sys.executable, os.path.abspath(__file__)]
    return cmd


def _csv_rows(outdir, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(outdir, "**", "*" + suffix), recursive=True)
    if not files:
        raise RuntimeError(f"rocprofv3 wrote no *{suffix} under {outdir}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


# Default timed calls and warmup.  The clock settles over the first ~20 ms
# of a fresh run (the fp32 4096^3 call falls from ~1.27 ms to ~1.07 ms over
# its first 20 calls), so the default warmup covers that before the timed
# calls; the kernel-trace pass of --collect-profile runs the same counts.
DEFAULT_STEPS = 50
DEFAULT_WARMUP = 30


def _timed_means(out, warmup):
    """Mean duration (ns) per kernel over its dispatches after the first
    `warmup` (the bench's timed calls), from a --kernel-trace CSV."""
    import collections
    rows = sorted(_csv_rows(out, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    per = collections.defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return [{"Name": k, "Calls": len(v) - warmup, "AverageNs": sum(v[warmup:]) / (len(v) - warmup)}
            for k, v in per.items() if len(v) > warmup]


def _per_dispatch(rows, name_filter):
    """Mean over dispatches of the per-dispatch sum (over instances) of the
    counter, for kernels whose name contains name_filter."""
    import collections
    per = collections.defaultdict(float)
    for r in rows:
        if name_filter in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise RuntimeError(f"no dispatch of a kernel matching {name_filter!r}")
    return sum(per.values()) / len(per), len(per)


def _shown(cmd, tmp):
    """A recorded command as it reads from the repository root: the
    interpreter as python3, this file as bench.py, temp output as $OUT."""
    text = " ".join(cmd).replace(sys.executable, "python3")
    text = text.replace(os.path.join(ROOT, "bench.py"), "bench.py")
    return text.replace(tmp, "$OUT")


def collect_profile(workload, tmp, out_dir=PROFILES, knobs=()):
    """Kernel-trace statistics, HBM traffic and L2 hit counters of one
    workload, written to profiles/.  FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) are each scaled by the ratio between the bytes a plain device
    copy of known size moves and what the same counter reports for it.  The
    L2 hit rate is TCC_HIT / (TCC_HIT + TCC_MISS) over the GEMM dispatches.
    `knobs` are extra bench.py arguments for the profiled runs (tile order,
    kernel family)."""
    import subprocess
    child = ["--workload", workload, "--secondary", "none", "--no-cpu-baseline"] + list(knobs)
    results = {}
    # 1. kernel trace with statistics
    out = os.path.join(tmp, "trace")
    cmd = _rocprof(["--kernel-trace", "--stats"], out) + child + [
        "--steps", str(DEFAULT_STEPS), "--warmup", str(DEFAULT_WARMUP)]
    log(f"[profile] {' '.join(cmd)}")
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    stats = _csv_rows(out, "kernel_stats.csv")
    results["trace_command"] = _shown(cmd, tmp)
    results["kernel_stats"] = [{k: r[k] for k in ("Name", "Calls", "AverageNs", "MinNs", "MaxNs",
                                                 "Percentage")} for r in stats]
    results["timed_means"] = _timed_means(out, DEFAULT_WARMUP)
    # 2. traffic counters, GEMM and copy calibration
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = os.path.join(tmp, counter)
        cmd = _rocprof(["--pmc", counter], out) + child + ["--steps", "3", "--warmup", "1"]
        log(f"[profile] {' '.join(cmd)}")
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
        kib, n = _per_dispatch(_csv_rows(out, "counter_collection.csv"), "gemm_")
        out_c = os.path.join(tmp, counter + "_copy")
        cmd_c = _rocprof(["--pmc", counter], out_c) + ["--workload", "copy", "--steps", "3",
                                                        "--warmup", "1"]
        subprocess.run(cmd_c, check=True, stdout=subprocess.DEVNULL)
        copy_kib, _ = _per_dispatch(_csv_rows(out_c, "counter_collection.csv"), "copy")
        scale = (512 << 20) / (copy_kib * 1024.0)
        results[counter] = {"kib_per_dispatch": kib, "dispatches": n,
                            "copy_kib_per_dispatch": copy_kib, "copy_bytes": 512 << 20,
                            "scale": scale, "bytes_per_dispatch": kib * 1024.0 * scale,
                            "command": _shown(cmd, tmp), "copy_command": _shown(cmd_c, tmp)}
    # 3. L2 (TCC) hits and misses of the GEMM kernels
    out = os.path.join(tmp, "tcc")
    cmd = _rocprof(["--pmc", "TCC_HIT_sum", "TCC_MISS_sum"], out) + child + ["--steps", "3",
                                                                           "--warmup", "1"]
    log(f"[profile] {' '.join(cmd)}")
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    rows = _csv_rows(out, "counter_collection.csv")
    hit, _ = _per_dispatch([r for r in rows if r["Counter_Name"] == "TCC_HIT_sum"], "gemm_")
    miss, _ = _per_dispatch([r for r in rows if r["Counter_Name"] == "TCC_MISS_sum"], "gemm_")
    results["L2"] = {"hits_per_dispatch": hit, "misses_per_dispatch": miss,
                     "hit_rate": hit / (hit + miss) if hit + miss > 0 else None,
                     "command": _shown(cmd, tmp)}
    # 4. utilisation: matrix-pipe busy share of SIMD cycles, VALU busy share
    # of CU cycles, LDS bank-conflict cycles per LDS cycle (rocprofv3's
    # derived metrics; 4 SQ counters and 1 GRBM counter in one pass)
    out = os.path.join(tmp, "util")
    cmd = _rocprof(["--pmc", "MfmaUtil", "VALUBusy", "LdsBankConflict"], out) + child + [
        "--steps", "3", "--warmup", "1"]
    log(f"[profile] {' '.join(cmd)}")
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    rows = _csv_rows(out, "counter_collection.csv")
    util = {}
    for name in ("MfmaUtil", "VALUBusy", "LdsBankConflict"):
        sel = [r for r in rows if r["Counter_Name"] == name]
        util[name] = _per_dispatch(sel, "gemm_")[0] if sel else None
    util["command"] = _shown(cmd, tmp)
    results["utilisation"] = util
    results["kernel_source_hash"] = kernel_source_hash()
    results["workload"] = workload
    results["knobs"] = list(knobs)
    results["library"] = os.environ.get("DG_LIBRARY") or "in-tree"
    write_profile(results, out_dir)
    return results


def write_profile(results, out_dir=PROFILES):
    """Write traffic_<workload>.json and a markdown summary of `results`."""
    workload = results["workload"]
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"traffic_{workload}.json"), "w") as f:
        json.dump(results, f, indent=1)
    import workloads as W
    p = W.WORKLOADS[workload]
    knobs = " ".join(results.get("knobs", []))
    lib = results.get("library", "in-tree")
    lines = [f"# rocprofv3 summary: {p.name}", "",
             f"Made by `python3 bench.py --workload {workload} --collect-profile"
             f"{' ' + knobs if knobs else ''}` from the repository root, which runs the commands "
             "below ($OUT is a temporary folder).", "",
             f"Kernel sources hash: `{results['kernel_source_hash']}`; library: {lib}", "",
             "## Kernel trace statistics", "", f"Command: `{results['trace_command']}`", "",
             "| kernel | calls | average ns | min ns | max ns | % |", "|---|---|---|---|---|---|"]
    for r in results["kernel_stats"]:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} | "
                     f"{float(r['Percentage']):.2f} |")
    if results.get("timed_means"):
        lines += ["", "The statistics above cover every dispatch, warmup included. Over the "
                  "timed calls only (the dispatches after each kernel's first "
                  f"{DEFAULT_WARMUP}), the same trace gives:", "",
                  "| kernel | timed calls | average ns |", "|---|---|---|"]
        for r in results["timed_means"]:
            lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {r['AverageNs']:.0f} |")
    lines += ["", "## HBM traffic per GEMM dispatch", "",
              "| counter | KiB / dispatch | copy calibration KiB (512 MiB copy) | scale | bytes |",
              "|---|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        t = results[c]
        lines.append(f"| {c} | {t['kib_per_dispatch']:.0f} | {t['copy_kib_per_dispatch']:.0f} | "
                     f"{t['scale']:.3f} | {t['bytes_per_dispatch']:.4g} |")
    lines += ["", f"Commands: `{results['FETCH_SIZE']['command']}`, "
              f"`{results['WRITE_SIZE']['command']}`; calibration: "
              f"`{results['FETCH_SIZE']['copy_command']}`", ""]
    if "utilisation" in results:
        u = results["utilisation"]
        fmt = lambda v, f: "n/a" if v is None else f.format(v)  # noqa: E731
        lines += ["## Utilisation per GEMM dispatch", "",
                  "| MfmaUtil (% of SIMD cycles) | VALUBusy (% of CU cycles) | "
                  "LdsBankConflict (conflict cycles per LDS cycle) |", "|---|---|---|",
                  f"| {fmt(u['MfmaUtil'], '{:.1f}')} | {fmt(u['VALUBusy'], '{:.1f}')} | "
                  f"{fmt(u['LdsBankConflict'], '{:.4f}')} |", "", f"Command: `{u['command']}`", ""]
    if "L2" in results:
        l2 = results["L2"]
        lines += ["## L2 (TCC) hit rate per GEMM dispatch", "",
                  "| TCC_HIT | TCC_MISS | hit rate |", "|---|---|---|",
                  f"| {l2['hits_per_dispatch']:.0f} | {l2['misses_per_dispatch']:.0f} | "
                  f"{l2['hit_rate']:.3f} |", "", f"Command: `{l2['command']}`", ""]
    with open(os.path.join(out_dir, f"{workload}_{p.name}.md"), "w") as f:
        f.write("\n".join(lines))


def traffic_for(workload):
    """HBM bytes per launch from profiles/, or None when missing or taken
    with other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    if t.get("knobs") or t.get("library", "in-tree") != "in-tree":
        return None      # taken with another tile order, family or build
    return t["FETCH_SIZE"]["bytes_per_dispatch"] + t["WRITE_SIZE"]["bytes_per_dispatch"]


def cpu_baseline(name, budget_s=12.0):
    """Oracle throughput on a seeded sample of the workload's outputs."""
    import numpy as np
    import oracle
    import workloads as W
    p = W.WORKLOADS[name]
    x = W.make_inputs(p)
    pb, pi, pj = W.sample_points(p, 8_000_000, seed=777)
    done, chunk, t0 = 0, 2048, time.perf_counter()
    while done < pb.size:
        sl = slice(done, min(done + chunk, pb.size))
        oracle.gemm_points(p, x.A, x.B, x.C, x.bias, pb[sl], pi[sl], pj[sl])
        done = sl.stop
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
        chunk = min(chunk * 2, 262144)
    el = time.perf_counter() - t0
    flops = 2.0 * p.K * done
    return {"value": flops / el / 1e12, "unit": "TFLOPS", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{done} seeded output elements of {p.name} (each a K={p.K} fp64 dot "
                      f"product plus epilogue), {el:.1f} s"}


def _roofline(workload, r):
    """The roofline object of one timed workload: algorithmic flops (or, for
    an HBM-bound kernel, bytes) per call over the measured time per call,
    against the kernel's published peak, and the profiled HBM traffic."""
    from dense_gemm_10_amd import accounting as acc
    p = r["problem"]
    bound, peak = _roofline_peak(p, r["kernel"])
    if bound == "hbm":
        achieved = acc.problem_bytes(p) / (r["ms"] * 1e-3)
        roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": peak / 1e9, "unit": "GB/s",
                "frac": achieved / peak}
    else:
        achieved = p.flops() / (r["ms"] * 1e-3)
        roof = {"bound": bound, "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak}
    roof["traffic"] = traffic_for(workload)
    roof["kernel"] = r["kernel"]
    roof["algorithmic_bytes"] = acc.problem_bytes(p)
    roof["algorithmic_flops"] = p.flops()
    return roof


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    import workloads as W
    ap.add_argument("--workload", default="c2", choices=list(W.WORKLOADS) + ["copy"])
    ap.add_argument("--secondary", default="c3",
                    help="second workload reported in the same line ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--algo", type=int, default=0)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, default=0)
    ap.add_argument("--collect-profile", action="store_true",
                    help="run rocprofv3 (kernel trace, FETCH_SIZE, WRITE_SIZE) on this workload "
                         "and write profiles/traffic_<workload>.json")
    ap.add_argument("--profile-dir", default=PROFILES,
                    help="where --collect-profile writes (default: profiles/)")
    args = ap.parse_args()

    if args.collect_profile:
        import tempfile
        knobs = []
        for flag, v in (("--algo", args.algo), ("--group-m", args.group_m),
                        ("--xcd-remap", args.xcd_remap)):
            if v:
                knobs += [flag, str(v)]
        with tempfile.TemporaryDirectory(dir=os.environ.get("TMPDIR", "/tmp")) as tmp:
            r = collect_profile(args.workload, tmp, args.profile_dir, knobs)
        print(json.dumps({"workload": args.workload,
                          "fetch_bytes": r["FETCH_SIZE"]["bytes_per_dispatch"],
                          "write_bytes": r["WRITE_SIZE"]["bytes_per_dispatch"]}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import dense_gemm_10_amd as dg
    from dense_gemm_10_amd import accounting as acc

    if args.workload == "copy":
        r = time_copy(args.steps, args.warmup)
        print(json.dumps({"workload": "copy_512MiB", **r}), flush=True)
        return

    overrides = dict(algo=args.algo, group_m=args.group_m, xcd_remap=args.xcd_remap)
    main_r = time_workload(args.workload, args.steps, args.warmup, **overrides)
    p = main_r["problem"]
    published = acc.compute_peak_for(p)
    roof = _roofline(args.workload, main_r)

    secondary = None
    if args.secondary != "none" and args.secondary != args.workload:
        s = time_workload(args.secondary, args.steps, args.warmup, **overrides)
        sp = s["problem"]
        secondary = {"workload": sp.name, "value": s["tflops"], "unit": "TFLOPS",
                     "ms_per_step": s["ms"], "dtype": _dtype_name(sp), "plan": s["plan"],
                     "frac_of_published_peak": s["tflops"] * 1e12 / acc.compute_peak_for(sp),
                     "roofline": _roofline(args.secondary, s)}
        del s

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(args.workload)

    line = {
        "metric": METRIC,
        "value": main_r["tflops"],
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": _dtype_name(p),
        "data": "synthetic",
        "config": {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "batch": p.batch,
                   "a_order": p.a_order, "b_order": p.b_order, "c_type": p.c_type,
                   "alpha": p.alpha, "beta": p.beta, "act": p.act, "plan": main_r["plan"],
                   "parallelism": "single_gpu"},
        "frac_of_published_peak": main_r["tflops"] * 1e12 / published,
        "published_peak_tflops": published / 1e12,
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "library_version": dg.dg_version(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
