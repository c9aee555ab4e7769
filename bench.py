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
    (matrix cores for the MFMA kernels, the fp32 vector-FMA rate for the
    others), or HBM when the algorithmic bytes take longer at 8 TB/s
    than the flops at that peak."""
    from dense_gemm_10_amd import accounting as acc
    if kernel.startswith("mfma_bf16"):
        bound, peak = "mfma", acc.PEAK_BF16_MFMA
    elif kernel.startswith("mfma_f16"):
        bound, peak = "mfma", acc.PEAK_F16_MFMA
    elif kernel.startswith("mfma_f32"):
        bound, peak = "mfma", acc.PEAK_F32
    else:
        bound, peak = "alu", acc.PEAK_F32_VALU
    if acc.problem_bytes(p) / acc.PEAK_HBM > acc.problem_flops(p) / peak:
        return "hbm", acc.PEAK_HBM
    return bound, peak


def _event_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


class Flusher:
    """Reads a 512 MiB device buffer (a sum): evicts the L2s and the 256 MB
    Infinity Cache (MALL) between calls with clean lines, so that the next
    call reads its operands from HBM (a cold-cache measurement) without
    also paying for the write-back of a flush written to memory."""

    def __init__(self, nbytes=512 << 20):
        import torch
        self.buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.float32, device="cuda")

    def __call__(self):
        import torch
        torch.sum(self.buf, 0, keepdim=True, out=self.sink)


def run_window(dp, stream, steps, flush=None):
    """`steps` timed calls.  Returns (ms per call, per-call ms list).
    Without `flush` the calls run back to back between one pair of events
    on the launch stream (an event recorded between calls would add its
    own gap to every call), and the list holds that mean once per call.
    With `flush`, the flush runs before each call, outside the call's own
    event pair, and the mean is over those pairs."""
    import torch
    torch.cuda.synchronize()
    if flush is None:
        s, e = _event_pair()
        s.record(stream)
        for _ in range(steps):
            dp.run(stream.cuda_stream)
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / steps
        return ms, [ms] * steps
    pairs = [_event_pair() for _ in range(steps)]
    for s, e in pairs:
        flush()
        s.record(stream)
        dp.run(stream.cuda_stream)
        e.record(stream)
    torch.cuda.synchronize()
    per_call = [s.elapsed_time(e) for s, e in pairs]
    return sum(per_call) / steps, per_call


def _smi_gfx_clocks():
    """Current shader clock of each XCD (MHz) from amd-smi, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True,
                           text=True, timeout=20)
        d = json.loads(r.stdout)
        clk = d["gpu_data"][0]["clock"] if isinstance(d, dict) else d[0]["clock"]
        return [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("gfx_")]
    except Exception:        # no amd-smi, or another output format
        return None


def clock_window(dp, stream, seconds=2.5):
    """Keep the GPU busy with back-to-back calls for `seconds` while a
    thread samples the XCD clocks with amd-smi; returns the samples (one
    list of per-XCD MHz each)."""
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            c = _smi_gfx_clocks()
            if c is None:
                return
            samples.append(c)

    t = threading.Thread(target=sampler, daemon=True)
    batches = []
    t0 = time.perf_counter()
    t.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            dp.run(stream.cuda_stream)
        ev = torch.cuda.Event()
        ev.record(stream)
        batches.append(ev)
        if len(batches) > 2:
            batches.pop(0).synchronize()
    stop.set()
    torch.cuda.synchronize()
    t.join(timeout=30)
    # amd-smi reports a stale idle reading (~0.1-0.2 GHz) until the clock
    # has risen: keep the samples taken under load
    return [c for c in samples[1:] if min(c) >= 500]


def _window_stats(window_ms, per_call):
    """kernel_ms_mean: the time per call the roofline uses (the window mean
    for back-to-back calls; the mean of per-call event pairs with a flush)."""
    srt = sorted(per_call)
    return {"ms_per_step": window_ms, "kernel_ms_mean": sum(per_call) / len(per_call),
            "kernel_ms_min": srt[0], "kernel_ms_max": srt[-1], "calls": len(per_call)}


def time_workload(name, steps, warmup, settle=0, steps_sustained=0, flush=None, clock_s=0.0,
                  **overrides):
    """Run one workload through dg_gemm: `warmup` untimed calls, a timed
    window of `steps` calls, then (settle > 0) `settle` more untimed calls
    and a second timed window of `steps_sustained` calls, the sustained
    rate once the clock has met the power limit.  With `flush` (cold
    caches), the flush runs before every call of the timed windows."""
    import torch
    import workloads as W
    from workloads.device import DeviceProblem
    p = W.WORKLOADS[name]
    log(f"[bench] {name}: generating {p.name}")
    x = W.make_inputs(p)
    dp = DeviceProblem(p, x, **overrides)
    plan = dp.describe()
    log(f"[bench] {name}: plan {plan}")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        dp.run(stream.cuda_stream)
    w, per = run_window(dp, stream, steps, flush)
    out = dict(problem=p, plan=plan, kernel=plan.split()[0].split("=")[1],
               window=_window_stats(w, per), inputs=x)
    out["ms"] = w
    out["kernel_ms"] = out["window"]["kernel_ms_mean"]
    out["tflops"] = p.flops() / (w * 1e-3) / 1e12
    if settle > 0 and steps_sustained > 0:
        for _ in range(settle):
            dp.run(stream.cuda_stream)
        w2, per2 = run_window(dp, stream, steps_sustained, flush)
        out["sustained"] = _window_stats(w2, per2)
    if clock_s > 0:
        smp = clock_window(dp, stream, clock_s)
        if smp:
            flat = [v for c in smp for v in c]
            out["clock_mhz"] = {"samples": smp, "mean": sum(flat) / len(flat),
                                "min": min(flat), "max": max(flat),
                                "source": "amd-smi metric -c, per XCD, during back-to-back calls"}
    del dp
    return out


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
N_XCD = 8          # MI355X: 8 XCDs of 32 compute units


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


# Default timed calls and warmup: the counts the benchmark is run with at
# the end of every build cycle (python3 bench.py --gpus 1 --steps 20
# --warmup 5), so that a plain run and the kernel-trace pass of
# --collect-profile time the same windows.  The chip's clock moves with its
# power state over the first calls of a fresh process (the fp32 4096^3 call
# takes ~1.04 ms per call over the first window and ~0.98 ms once settled;
# the bf16 4096^3 call ~108 us, then 103-106 us), so every workload also
# gets a second, sustained window of max(K, SUSTAINED_MIN) calls after
# SETTLE further untimed calls.
DEFAULT_STEPS = 20
DEFAULT_WARMUP = 5
SETTLE = 300
SUSTAINED_MIN = 50
CLOCK_S = 2.5      # seconds of back-to-back calls while amd-smi samples the clocks


def _sustained_steps(steps):
    return max(steps, SUSTAINED_MIN)


def _timed_means(out, warmup, steps, settle):
    """Mean duration (ns) per kernel over its dispatches in the bench's two
    timed windows: dispatches [warmup, warmup + steps) (first window) and,
    after `settle` more, the next _sustained_steps(steps) (sustained
    window), from a --kernel-trace CSV.  Every call dispatches each of its
    kernels once, so a kernel's n-th dispatch belongs to the n-th call."""
    import collections
    rows = sorted(_csv_rows(out, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    per = collections.defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    res = []
    s0 = warmup + steps + settle
    s1 = s0 + _sustained_steps(steps)
    for k, v in per.items():
        if len(v) < warmup + steps:
            continue
        first = v[warmup:warmup + steps]
        r = {"Name": k, "Calls": len(first), "AverageNs": sum(first) / len(first)}
        if settle > 0 and len(v) >= s1:
            r["SustainedCalls"] = s1 - s0
            r["SustainedAverageNs"] = sum(v[s0:s1]) / (s1 - s0)
        res.append(r)
    return res


def _is_gemm(kernel_name):
    """A call's dominant kernel: the tiled (or generic / vector) GEMM, not
    the stand-alone sliver kernel some plans launch after it."""
    return "gemm_" in kernel_name and "gemm_sliver" not in kernel_name


def _per_dispatch(rows, name_filter):
    """Mean over dispatches of the per-dispatch sum (over instances) of the
    counter, for kernels whose name contains name_filter ("gemm_": the
    call's GEMM kernel, see _is_gemm)."""
    import collections
    per = collections.defaultdict(float)
    for r in rows:
        name = r["Kernel_Name"]
        if (_is_gemm(name) if name_filter == "gemm_" else name_filter in name):
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


def collect_profile(workload, tmp, out_dir=PROFILES, knobs=(), steps=DEFAULT_STEPS,
                    warmup=DEFAULT_WARMUP):
    """Kernel-trace statistics, HBM traffic and L2 hit counters of one
    workload, written to profiles/.  FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) are each scaled by the ratio between the bytes a plain device
    copy of known size moves and what the same counter reports for it.  The
    L2 hit rate is TCC_HIT / (TCC_HIT + TCC_MISS) over the GEMM dispatches.
    `knobs` are extra bench.py arguments for the profiled runs (tile order,
    kernel family)."""
    import subprocess
    child = ["--workload", workload, "--secondary", "none", "--no-extras",
             "--no-cpu-baseline", "--clock-seconds", "0"] + list(knobs)
    short = ["--steps", "3", "--warmup", "1", "--settle", "0"]   # counter passes
    results = {}
    # 1. kernel trace with statistics, the bench's own windows
    out = os.path.join(tmp, "trace")
    cmd = _rocprof(["--kernel-trace", "--stats"], out) + child + [
        "--steps", str(steps), "--warmup", str(warmup)]
    log(f"[profile] {' '.join(cmd)}")
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    stats = _csv_rows(out, "kernel_stats.csv")
    results["trace_command"] = _shown(cmd, tmp)
    results["kernel_stats"] = [{k: r[k] for k in ("Name", "Calls", "AverageNs", "MinNs", "MaxNs",
                                                 "Percentage")} for r in stats]
    results["timed_means"] = _timed_means(out, warmup, steps, SETTLE)
    results["windows"] = {"warmup": warmup, "steps": steps, "settle": SETTLE,
                          "sustained_steps": _sustained_steps(steps)}
    # 2. traffic counters, GEMM and copy calibration
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = os.path.join(tmp, counter)
        cmd = _rocprof(["--pmc", counter], out) + child + short
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
    cmd = _rocprof(["--pmc", "TCC_HIT_sum", "TCC_MISS_sum"], out) + child + short
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
    cmd = _rocprof(["--pmc", "MfmaUtil", "VALUBusy", "LdsBankConflict"], out) + child + short
    log(f"[profile] {' '.join(cmd)}")
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    rows = _csv_rows(out, "counter_collection.csv")
    util = {}
    for name in ("MfmaUtil", "VALUBusy", "LdsBankConflict"):
        sel = [r for r in rows if r["Counter_Name"] == name]
        util[name] = _per_dispatch(sel, "gemm_")[0] if sel else None
    util["command"] = _shown(cmd, tmp)
    results["utilisation"] = util
    # 5. effective shader clock during the GEMM dispatches: GPU-busy cycles
    # (GRBM_GUI_ACTIVE, summed over the XCDs) per XCD over the dispatch's
    # duration
    out = os.path.join(tmp, "clock")
    cmd = _rocprof(["--pmc", "GRBM_GUI_ACTIVE"], out) + child + short
    log(f"[profile] {' '.join(cmd)}")
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
    rows = [r for r in _csv_rows(out, "counter_collection.csv") if _is_gemm(r["Kernel_Name"])]
    clocks = []
    for r in rows:
        try:
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        except (KeyError, ValueError):
            dur = 0
        if dur > 0:
            clocks.append(float(r["Counter_Value"]) / N_XCD / dur)
    results["clock"] = {"ghz_per_dispatch": clocks, "command": _shown(cmd, tmp),
                        "xcds": N_XCD}
    results["kernel_source_hash"] = kernel_source_hash()
    results["workload"] = workload
    results["knobs"] = list(knobs)
    results["library"] = os.environ.get("DG_LIBRARY") or "in-tree"
    write_profile(results, out_dir)
    return results


def profile_tag(workload, knobs=()):
    """File tag of a profile: the workload, then any knobs (e.g. c2_algo2)."""
    k = list(knobs)
    extra = "".join(f"_{k[i].lstrip('-').replace('-', '')}{k[i + 1]}"
                    for i in range(0, len(k) - 1, 2))
    return workload + extra


def write_profile(results, out_dir=PROFILES):
    """Write traffic_<tag>.json and a markdown summary of `results`."""
    workload = results["workload"]
    tag = profile_tag(workload, results.get("knobs", []))
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"traffic_{tag}.json"), "w") as f:
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
        w = results.get("windows", {"warmup": DEFAULT_WARMUP, "steps": DEFAULT_STEPS,
                                    "settle": 0, "sustained_steps": 0})
        lines += ["", "The statistics above cover every dispatch, warmup included. Over the "
                  "bench's timed windows only (first window: each kernel's dispatches "
                  f"{w['warmup']} .. {w['warmup'] + w['steps'] - 1}; sustained window: the "
                  f"{w['sustained_steps']} dispatches after {w['settle']} further untimed "
                  "ones), the same trace gives:", "",
                  "| kernel | first window calls | average ns | sustained calls | "
                  "sustained average ns |", "|---|---|---|---|---|"]
        for r in results["timed_means"]:
            sus = (f"{r['SustainedCalls']} | {r['SustainedAverageNs']:.0f}"
                   if "SustainedCalls" in r else "- | -")
            lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {r['AverageNs']:.0f} | {sus} |")
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
    if results.get("clock", {}).get("ghz_per_dispatch"):
        c = results["clock"]
        g = ", ".join(f"{v:.3f}" for v in c["ghz_per_dispatch"])
        lines += ["## Effective shader clock per GEMM dispatch", "",
                  f"GRBM_GUI_ACTIVE / {c['xcds']} XCDs / dispatch duration: {g} GHz", "",
                  f"Command: `{c['command']}`", ""]
    if "L2" in results:
        l2 = results["L2"]
        lines += ["## L2 (TCC) hit rate per GEMM dispatch", "",
                  "| TCC_HIT | TCC_MISS | hit rate |", "|---|---|---|",
                  f"| {l2['hits_per_dispatch']:.0f} | {l2['misses_per_dispatch']:.0f} | "
                  f"{l2['hit_rate']:.3f} |", "", f"Command: `{l2['command']}`", ""]
    with open(os.path.join(out_dir, f"{tag}_{p.name}.md"), "w") as f:
        f.write("\n".join(lines))


def traffic_for(workload, knobs=()):
    """HBM bytes per launch from profiles/, or None when missing or taken
    with other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{profile_tag(workload, knobs)}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    if list(t.get("knobs", [])) != list(knobs) or t.get("library", "in-tree") != "in-tree":
        return None      # taken with another tile order, family or build
    return t["FETCH_SIZE"]["bytes_per_dispatch"] + t["WRITE_SIZE"]["bytes_per_dispatch"]


def host_cpu():
    """CPU model and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cores_available": len(os.sched_getaffinity(0))}


def cpu_baseline(name, budget_s=12.0):
    """Oracle throughput on a seeded sample of the workload's outputs, on
    every core; and the whole 256^3 workload (all of its outputs) on one
    core."""
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
    out = {"value": flops / el / 1e12, "unit": "TFLOPS", "cores": oracle.max_threads(),
           "kind": "oracle",
           "sample": f"{done} seeded output elements of {p.name} (each a K={p.K} fp64 dot "
                     f"product plus epilogue), {el:.1f} s"}
    p1 = W.WORKLOADS["c1"]
    x1 = W.make_inputs(p1)
    t0 = time.perf_counter()
    oracle.gemm(p1, x1.A, x1.B, x1.C, x1.bias, nthreads=1)
    el1 = time.perf_counter() - t0
    out["one_core_full"] = {"workload": p1.name, "seconds": el1,
                            "gflops": p1.flops() / el1 / 1e9, "cores": 1}
    out["host"] = host_cpu()
    return out


def _roofline(workload, r, ms=None, knobs=()):
    """The roofline object of one timed workload: algorithmic flops (or, for
    an HBM-bound kernel, bytes) per call over the measured kernel time per
    call (the mean of per-call HIP event pairs on the launch stream, unless
    `ms` is given), against the kernel's published peak, and the profiled
    HBM traffic."""
    from dense_gemm_10_amd import accounting as acc
    p = r["problem"]
    ms = r["kernel_ms"] if ms is None else ms
    bound, peak = _roofline_peak(p, r["kernel"])
    if bound == "hbm":
        achieved = acc.problem_bytes(p) / (ms * 1e-3)
        roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": peak / 1e9, "unit": "GB/s",
                "frac": achieved / peak}
    else:
        achieved = p.flops() / (ms * 1e-3)
        roof = {"bound": bound, "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak}
    roof["traffic"] = traffic_for(workload, knobs)
    roof["kernel"] = r["kernel"]
    roof["kernel_ms"] = ms
    roof["algorithmic_bytes"] = acc.problem_bytes(p)
    roof["algorithmic_flops"] = p.flops()
    return roof


def _summary(workload, r, knobs=()):
    """JSON record of one timed workload: both windows, plan and roofline
    (of the sustained window when there is one)."""
    from dense_gemm_10_amd import accounting as acc
    p = r["problem"]
    rec = {"workload": p.name, "key": workload, "plan": r["plan"], "dtype": _dtype_name(p),
           "first_window": dict(r["window"], tflops=p.flops() / (r["ms"] * 1e-3) / 1e12)}
    sus = r.get("sustained")
    if sus:
        rec["sustained"] = dict(sus, tflops=p.flops() / (sus["ms_per_step"] * 1e-3) / 1e12)
        rec["roofline"] = _roofline(workload, r, sus["kernel_ms_mean"], knobs)
        rec["roofline_first_window"] = _roofline(workload, r, None, knobs)
    else:
        rec["roofline"] = _roofline(workload, r, None, knobs)
    rec["frac_of_published_peak"] = (rec.get("sustained", rec["first_window"])["tflops"] * 1e12
                                     / acc.compute_peak_for(p))
    if "clock_mhz" in r:
        rec["clock_mhz"] = r["clock_mhz"]
    return rec


# ---- tile-order ablation ------------------------------------------------------
# Group height G of the grouped tile order x XCD remap on / off, on the two
# headline problems and one whose operands exceed the Infinity Cache
# ("GEMM Kernel Optimization", L2 Cache Grouping and Common Pitfalls on
# GROUP_SIZE_M = 1).
ABLATION_WORKLOADS = ("c2", "c3", "big8192")
ABLATION_GROUPS = (1, 4, 8, 16)
ABLATION_REMAP = (1, -1)          # descriptor xcd_remap: 1 on, -1 off
ABLATION_CHILD_CALLS = 4          # per combination in the counter passes (first one dropped)


def _ablation_problems():
    import workloads as W
    from workloads.device import DeviceProblem
    for w in ABLATION_WORKLOADS:
        p = W.WORKLOADS[w]
        log(f"[ablation] {w}: generating {p.name}")
        x = W.make_inputs(p)
        dp = DeviceProblem(p, x)
        del x
        yield w, dp
        del dp


def _set_order(dp, g, r):
    dp.desc.group_m = g
    dp.desc.xcd_remap = r


def ablation_timing(steps, settle):
    """Sustained kernel time of every combination, timed in two passes
    (combinations in order, then reversed) whose means are averaged, so a
    slow drift of the clock does not favour the first or last."""
    import torch
    stream = torch.cuda.current_stream()
    res = {}
    for w, dp in _ablation_problems():
        combos = [(g, r) for g in ABLATION_GROUPS for r in ABLATION_REMAP]
        for order in (combos, combos[::-1]):
            for g, r in order:
                _set_order(dp, g, r)
                for _ in range(settle):
                    dp.run(stream.cuda_stream)
                _, per = run_window(dp, stream, steps)
                res.setdefault((w, g, r), []).append(sum(per) / len(per))
        log(f"[ablation] {w}: {dp.describe()}")
    return {k: sum(v) / len(v) for k, v in res.items()}


def ablation_child():
    """Every combination in a fixed order, ABLATION_CHILD_CALLS calls each,
    nothing else on the GPU between them: the dispatch order of the GEMM
    kernels identifies the combination in a counter pass."""
    import torch
    stream = torch.cuda.current_stream()
    for w, dp in _ablation_problems():
        for g in ABLATION_GROUPS:
            for r in ABLATION_REMAP:
                _set_order(dp, g, r)
                for _ in range(ABLATION_CHILD_CALLS):
                    dp.run(stream.cuda_stream)
                torch.cuda.synchronize()


def run_ablation(steps, settle, tmp, out_dir=PROFILES):
    import subprocess
    import workloads as W
    from dense_gemm_10_amd import accounting as acc
    times = ablation_timing(steps, settle)
    combos = [(w, g, r) for w in ABLATION_WORKLOADS for g in ABLATION_GROUPS
              for r in ABLATION_REMAP]
    counters = {}
    cmds = {}
    scale = {}
    for name, pmc in (("tcc", ["TCC_HIT_sum", "TCC_MISS_sum"]), ("FETCH_SIZE", ["FETCH_SIZE"]),
                      ("WRITE_SIZE", ["WRITE_SIZE"])):
        out = os.path.join(tmp, name)
        cmd = _rocprof(["--pmc"] + pmc, out, timeout_s=300) + ["--ablation-child"]
        log(f"[ablation] {' '.join(cmd)}")
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL)
        cmds[name] = _shown(cmd, tmp)
        rows = [r for r in _csv_rows(out, "counter_collection.csv") if _is_gemm(r["Kernel_Name"])]
        for cn in pmc:
            per = {}
            for r in rows:
                if r["Counter_Name"] == cn:
                    per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + \
                        float(r["Counter_Value"])
            seq = [per[k] for k in sorted(per)]
            if len(seq) != len(combos) * ABLATION_CHILD_CALLS:
                raise RuntimeError(f"{cn}: {len(seq)} GEMM dispatches, expected "
                                   f"{len(combos) * ABLATION_CHILD_CALLS}")
            for i, c in enumerate(combos):
                chunk = seq[i * ABLATION_CHILD_CALLS + 1:(i + 1) * ABLATION_CHILD_CALLS]
                counters.setdefault(c, {})[cn] = sum(chunk) / len(chunk)
        if name in ("FETCH_SIZE", "WRITE_SIZE"):
            out_c = os.path.join(tmp, name + "_copy")
            cmd_c = _rocprof(["--pmc", name], out_c) + ["--workload", "copy", "--steps", "3",
                                                         "--warmup", "1"]
            subprocess.run(cmd_c, check=True, stdout=subprocess.DEVNULL)
            copy_kib, _ = _per_dispatch(_csv_rows(out_c, "counter_collection.csv"), "copy")
            scale[name] = (512 << 20) / (copy_kib * 1024.0)
            cmds[name + "_copy"] = _shown(cmd_c, tmp)
    table = []
    for c in combos:
        w, g, r = c
        p = W.WORKLOADS[w]
        k = counters[c]
        hit, miss = k["TCC_HIT_sum"], k["TCC_MISS_sum"]
        ms = times[c]
        table.append({"workload": w, "name": p.name, "group_m": g, "xcd_remap": r == 1,
                      "kernel_us": ms * 1e3, "tflops": p.flops() / (ms * 1e-3) / 1e12,
                      "frac_of_peak": p.flops() / (ms * 1e-3) / acc.compute_peak_for(p),
                      "l2_hit_rate": hit / (hit + miss) if hit + miss else None,
                      "l2_misses": miss,
                      "fetch_bytes": k["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"],
                      "write_bytes": k["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"],
                      "algorithmic_bytes": acc.problem_bytes(p)})
    result = {"table": table, "commands": cmds, "scale": scale, "steps": steps, "settle": settle,
              "kernel_source_hash": kernel_source_hash()}
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "tile_order_ablation.json"), "w") as f:
        json.dump(result, f, indent=1)
    lines = ["# Tile-order ablation: group height x XCD remap", "",
             "Made by `python3 bench.py --ablation` from the repository root. Kernel time: mean "
             f"of per-call HIP event pairs over {steps} calls after {settle} untimed ones, per "
             "combination, averaged over two passes (combinations in order, then reversed). "
             "Counters: the commands below ($OUT is a temporary folder), over "
             f"{ABLATION_CHILD_CALLS - 1} calls per combination after one untimed; FETCH_SIZE "
             f"x {scale['FETCH_SIZE']:.3f} and WRITE_SIZE x {scale['WRITE_SIZE']:.3f} "
             "(a 512 MiB device copy's reading).", "",
             f"Kernel sources hash: `{result['kernel_source_hash']}`", "",
             "| problem | G | XCD remap | kernel us | TFLOP/s | of peak | L2 hit | L2 misses "
             "| HBM fetch MB | HBM write MB | algorithmic MB |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for t in table:
        lines.append(f"| {t['name']} | {t['group_m']} | {'on' if t['xcd_remap'] else 'off'} | "
                     f"{t['kernel_us']:.1f} | {t['tflops']:.1f} | {t['frac_of_peak']:.3f} | "
                     f"{t['l2_hit_rate']:.3f} | {t['l2_misses']:.3g} | "
                     f"{t['fetch_bytes'] / 1e6:.1f} | {t['write_bytes'] / 1e6:.1f} | "
                     f"{t['algorithmic_bytes'] / 1e6:.1f} |")
    lines += ["", "Commands:", ""] + [f"- {k}: `{v}`" for k, v in cmds.items()] + [""]
    with open(os.path.join(out_dir, "tile_order_ablation.md"), "w") as f:
        f.write("\n".join(lines))
    return result


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    import workloads as W
    ap.add_argument("--workload", default="c2", choices=list(W.WORKLOADS) + ["copy"])
    ap.add_argument("--secondary", default="c3",
                    help="second workload reported in the same line ('none' to skip)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the vector-FMA SGEMM leg and the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle", type=int, default=SETTLE,
                    help="untimed calls between the first and the sustained window (0: no "
                         "sustained window)")
    ap.add_argument("--clock-seconds", type=float, default=CLOCK_S,
                    help="seconds of back-to-back calls while amd-smi samples the clocks "
                         "(0: skip)")
    ap.add_argument("--algo", type=int, default=0)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, default=0)
    ap.add_argument("--collect-profile", action="store_true",
                    help="run rocprofv3 (kernel trace, FETCH_SIZE, WRITE_SIZE, L2, utilisation) "
                         "on this workload and write profiles/traffic_<tag>.json and a summary")
    ap.add_argument("--profile-dir", default=PROFILES,
                    help="where --collect-profile and --ablation write (default: profiles/)")
    ap.add_argument("--ablation", action="store_true",
                    help="tile-order ablation (group height x XCD remap) with kernel times and "
                         "L2 / HBM counters; writes profiles/tile_order_ablation.md")
    ap.add_argument("--ablation-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.ablation_child:
        ablation_child()
        return
    if args.ablation:
        import tempfile
        with tempfile.TemporaryDirectory(dir=os.environ.get("TMPDIR", "/tmp")) as tmp:
            r = run_ablation(50, 100, tmp, args.profile_dir)
        print(json.dumps({"ablation": [{k: v for k, v in t.items() if k != "name"}
                                       for t in r["table"]]}), flush=True)
        return

    knobs = []
    for flag, v in (("--algo", args.algo), ("--group-m", args.group_m),
                    ("--xcd-remap", args.xcd_remap)):
        if v:
            knobs += [flag, str(v)]

    if args.collect_profile:
        import tempfile
        with tempfile.TemporaryDirectory(dir=os.environ.get("TMPDIR", "/tmp")) as tmp:
            r = collect_profile(args.workload, tmp, args.profile_dir, knobs, args.steps,
                                args.warmup)
        print(json.dumps({"workload": args.workload, "knobs": knobs,
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
    K, Wm, Ks = args.steps, args.warmup, _sustained_steps(args.steps)
    ST, CS = args.settle, args.clock_seconds
    main_r = time_workload(args.workload, K, Wm, ST, Ks, clock_s=CS, **overrides)
    p = main_r["problem"]
    published = acc.compute_peak_for(p)
    roof = _roofline(args.workload, main_r, None, knobs)
    main_sus = main_r.get("sustained")
    if main_sus:
        main_sus = dict(main_sus, tflops=p.flops() / (main_sus["ms_per_step"] * 1e-3) / 1e12,
                        roofline=_roofline(args.workload, main_r, main_sus["kernel_ms_mean"],
                                           knobs))
    main_window = dict(main_r["window"])
    del main_r["inputs"]

    secondary = None
    if args.secondary != "none" and args.secondary != args.workload:
        s = time_workload(args.secondary, K, Wm, ST, Ks, clock_s=CS, **overrides)
        rec = _summary(args.secondary, s, knobs)
        # the sustained window is the value: the first window after a short
        # warmup runs before the power limit applies
        win = rec.get("sustained", rec["first_window"])
        secondary = dict(rec, value=win["tflops"], unit="TFLOPS", ms_per_step=win["ms_per_step"])
        del s

    extras = None
    if not args.no_extras and not knobs:
        extras = {}
        if args.workload == "c2":
            # the register-tiled vector-FMA SGEMM on the same problem
            v = time_workload("c2", K, Wm, ST, Ks, clock_s=CS, algo=dg.DG_ALGO_VALU_F32)
            extras["c2_valu"] = _summary("c2", v, ["--algo", str(dg.DG_ALGO_VALU_F32)])
            del v
        for key in ("c1", "c3_brow", "c4", "c5", "flat16"):
            if key in (args.workload, args.secondary):
                continue
            r = time_workload(key, K, Wm, ST, Ks)
            extras[key] = _summary(key, r)
            del r
        # the split-K batch with the caches flushed before every call: its
        # 134 MB A fits the 256 MB Infinity Cache, so back-to-back calls
        # read it from there, not from HBM
        flush = Flusher()
        r = time_workload("c5", K, Wm, flush=flush)
        extras["c5_cold"] = _summary("c5", r)
        extras["c5_cold"]["note"] = ("512 MiB written between calls (outside the timed "
                                     "event pairs): operands come from HBM")
        del r, flush

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
        "window": main_window,
        "sustained": main_sus,
        "clock_mhz": main_r.get("clock_mhz"),
        "cpu_baseline": cpu,
        "secondary": secondary,
        "extras": extras,
        "library_version": dg.dg_version(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
