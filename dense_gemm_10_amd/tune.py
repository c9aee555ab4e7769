"""Offline tuning sweep for the planner's static table (runs on an MI355X).

    python3 -m dense_gemm_10_amd.tune [--out PATH] [--steps N] [--only NAME ...]

For every shape below, every tile configuration of the kernel family the
library picks for it is timed under both schedules (data-parallel and
stream-K, where stream-K applies, with its own and 4, 8 or 16 K slices per
tail tile) and, where the output tiles alone fill less than a wave of the
256 compute units, with 2 to 16 split-K slices,
next to the library's own heuristic plan
(timed with the table switched off, DG_TUNED=0).  This is the per-size
benchmark-and-keep-the-fastest of "GEMM Kernel Optimization" (Autotune
Configs) and of "Skill: Write a Triton GEMM Kernel" (Required reasoning
process step 7: configurations over tile sizes and pipeline depth, keyed
on M, N, K), done once, offline: the winners are
written as C initialisers to csrc/tuned_table.inc, which the planner
compiles in, and no call ever benchmarks.

A candidate replaces the heuristic's plan only when it is faster by more
than MARGIN (clock and power noise on one device is a few percent);
otherwise the entry pins the heuristic's own tile and schedule.  Each entry
carries the measured times as a comment.

Inputs are the seeded synthetic operands of the workloads package (normal
or uniform values: the MFMA clock under the power limit depends on the
data, so zeros would time a different machine state).
"""
from __future__ import annotations

import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MARGIN = 0.03

# Tile configurations of each family, as named in the kernel files' tables.
TILES = {
    "mfma_bf16": ["mfma_bf16_256x256x64_w2x2_s2", "mfma_bf16_128x128x32_w2x2_s4",
                  "mfma_bf16_256x256x32_w2x2_s4", "mfma_bf16_256x128x32_w2x2_s4",
                  "mfma_bf16_256x128x32_w2x2_s3", "mfma_bf16_128x256x32_w2x2_s3",
                  "mfma_bf16_128x128x64_w2x2_s3", "mfma_bf16_256x128x64_w2x2_s3",
                  "mfma_bf16_128x256x32_w2x2_s2", "mfma_bf16_128x128x32_w2x2_s2"],
    "mfma_f16": ["mfma_f16_256x256x64_w2x2_s2", "mfma_f16_128x128x32_w2x2_s4",
                 "mfma_f16_256x256x32_w2x2_s4", "mfma_f16_256x128x32_w2x2_s4",
                 "mfma_f16_256x128x32_w2x2_s3", "mfma_f16_128x256x32_w2x2_s3",
                 "mfma_f16_128x128x64_w2x2_s3", "mfma_f16_256x128x64_w2x2_s3",
                 "mfma_f16_128x256x32_w2x2_s2", "mfma_f16_128x128x32_w2x2_s2"],
    "mfma_f32": ["mfma_f32_256x256x16_w2x2", "mfma_f32_128x128x16_w2x2",
                 "mfma_f32_256x256x32_w2x2", "mfma_f32_128x128x32_w2x2"],
}
KERNEL_CONST = {"mfma_bf16": "KERNEL_MFMA_BF16", "mfma_f16": "KERNEL_MFMA_F16",
                "mfma_f32": "KERNEL_MFMA_F32"}
SCHED_CONST = {"data_parallel": "DG_SCHED_DATA_PARALLEL", "stream_k": "DG_SCHED_STREAM_K"}


def shapes():
    """The swept problems: the named workloads and a grid of common sizes in
    the same layouts (A row-major, B column-major for 16-bit inputs)."""
    import workloads as W
    out = [W.WORKLOADS[n] for n in ("c1", "c2", "c3", "c4", "c5", "flat16", "flat16_f32",
                                    "tail4352", "f16_4096", "f16_gelu")]
    bf = W.WORKLOADS["c3"]
    for (M, N, K) in [(1024, 1024, 1024), (2048, 2048, 2048), (3072, 3072, 3072),
                      (6144, 6144, 6144), (8192, 8192, 8192), (4096, 4096, 1024),
                      (8192, 8192, 2048), (2048, 2048, 8192), (4096, 14336, 4096),
                      (14336, 4096, 4096), (16384, 4096, 4096), (1024, 4096, 16384)]:
        out.append(bf.replace(name=f"gemm_bf16_{M}x{N}x{K}", M=M, N=N, K=K))
    f16 = W.WORKLOADS["f16_4096"]
    for (M, N, K) in [(2048, 2048, 2048), (8192, 8192, 8192)]:
        out.append(f16.replace(name=f"gemm_f16_{M}x{N}x{K}", M=M, N=N, K=K))
    f32 = W.WORKLOADS["c2"]
    for (M, N, K) in [(1024, 1024, 1024), (2048, 2048, 2048), (8192, 8192, 8192)]:
        out.append(f32.replace(name=f"sgemm_f32_{M}x{N}x{K}", M=M, N=N, K=K))
    return out


def _kv(text):
    return dict(t.split("=", 1) for t in text.split() if "=" in t)


class Timer:
    """Device buffers of one problem and timed calls under a given plan."""

    def __init__(self, p, steps):
        import workloads as W
        from workloads.device import DeviceProblem
        self.p = p
        self.steps = steps
        self.dp = DeviceProblem(p, W.make_inputs(p))
        self.fields = W.desc_fields(p)
        self.fields["bias"] = self.dp.bias.data_ptr() if self.dp.bias is not None else None

    def plan(self, tile=None, schedule=0, split_k=None):
        """(description, desc, workspace bytes) of a candidate.  With a tile,
        the plan a table entry (tile, schedule 1 = data-parallel or 2 =
        stream-K, split_k slices, None = automatic) gives, applied through
        DG_FORCE_PLAN exactly as the planner applies a tuned entry (the
        descriptor leaves schedule and split to the library, so the
        sliver-column split applies as it will at run time); without, the
        heuristic plan (DG_TUNED=0)."""
        import dense_gemm_10_amd as dg
        os.environ["DG_TUNED"] = "0"
        os.environ.pop("DG_FORCE_TILE", None)
        if tile:
            os.environ["DG_FORCE_PLAN"] = f"{tile}:{'sk' if schedule == 2 else 'dp'}:{split_k or 0}"
        else:
            os.environ.pop("DG_FORCE_PLAN", None)
        d = dg.make_desc(**self.fields)
        try:
            ws = dg.dg_gemm_workspace_size(d)
            return dg.dg_gemm_describe(d, ws), d, ws
        except dg.DgError:
            return None, d, 0

    def time(self, d, ws_bytes):
        """Best of three means of `steps` calls, in microseconds."""
        import torch
        import dense_gemm_10_amd as dg
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
        s = torch.cuda.current_stream()
        args = (d, self.dp.A.data_ptr(), self.dp.B.data_ptr(), self.dp.C.data_ptr(),
                ws.data_ptr() if ws is not None else None, ws_bytes, s.cuda_stream)
        for _ in range(3):
            dg.dg_gemm(*args)
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(self.steps):
                dg.dg_gemm(*args)
            e1.record(s)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / self.steps)
        return best


def sweep(p, steps, log):
    """Time the heuristic plan and every candidate; returns a result dict."""
    t = Timer(p, steps)
    # all plan queries below see the environment they set
    text, d, ws = t.plan()
    kv = _kv(text)
    family = kv["kernel"]
    res = {"problem": p, "family": family, "heuristic": (kv["tile"], kv["schedule"]),
           "cands": []}
    if family not in TILES:
        log(f"[tune] {p.name}: family {family} has no alternatives")
        return None
    res["heuristic_us"] = t.time(d, ws)
    for tile in TILES[family]:
        for sched_code, sched in ((1, "data_parallel"), (2, "stream_k")):
            text, d, ws = t.plan(tile=tile, schedule=sched_code)
            if text is None or _kv(text)["tile"] != tile:
                continue
            sk_kind = _kv(text)["schedule"]
            if sched == "stream_k" and sk_kind != "stream_k":
                continue
            res["cands"].append((tile, sched, 0, t.time(d, ws)))
            if sched == "stream_k":
                # other K-slice counts of the tail tiles
                seen = {_kv(text)["tail_splits"]}
                for S in (4, 8, 16):
                    text, d, ws = t.plan(tile=tile, schedule=2, split_k=S)
                    if text is None or _kv(text).get("tail_splits") in seen:
                        continue
                    seen.add(_kv(text)["tail_splits"])
                    res["cands"].append((tile, sched, S, t.time(d, ws)))
                continue
            if sched != "data_parallel" or p.split_k:
                continue
            # explicit split-K counts when the tiles leave compute units idle (at
            # least 64 of K per slice)
            text1, _, _ = t.plan(tile=tile, schedule=1, split_k=1)
            tiles = int(_kv(text1)["programs"])
            for S in (2, 4, 8, 16):
                if tiles >= 256 or tiles * S > 1024 or p.K < 64 * S:
                    continue
                text, d, ws = t.plan(tile=tile, schedule=1, split_k=S)
                if text is None or _kv(text)["splits"] != str(S):
                    continue
                res["cands"].append((tile, sched, S, t.time(d, ws)))
    os.environ.pop("DG_FORCE_PLAN", None)
    os.environ.pop("DG_TUNED", None)
    best = min(res["cands"], key=lambda c: c[3])
    if best[3] < res["heuristic_us"] * (1.0 - MARGIN):
        res["choice"] = (best[0], best[1], best[2], best[3], "tuned")
    else:
        h_tile, h_sched = res["heuristic"]
        res["choice"] = (h_tile, h_sched, 0, res["heuristic_us"], "heuristic")
    log(f"[tune] {p.name}: heuristic {res['heuristic'][0]}/{res['heuristic'][1]} "
        f"{res['heuristic_us']:.1f} us; best {best[0]}/{best[1]}/S{best[2]} {best[3]:.1f} us "
        f"-> {res['choice'][4]}")
    return res


def _entry_blocks(path):
    """The entries of an existing table file: {problem name: its three lines
    (timings, candidates, entry)}, in file order."""
    blocks, lines = {}, open(path).read().splitlines()
    for i, line in enumerate(lines):
        if line.startswith("// ") and ": heuristic " in line and i + 2 < len(lines):
            blocks[line[3:].split(":", 1)[0]] = lines[i:i + 3]
    return blocks


def write_table(results, path, steps, device, keep=None):
    """Write the table of `results`; `keep` (entry blocks of an earlier
    table) supplies the entries of problems not swept this time."""
    lines = [
        "// Offline-tuned plans of the GEMM planner: GENERATED, do not edit.",
        f"// Made by `python3 -m dense_gemm_10_amd.tune` on {device}, "
        f"{time.strftime('%Y-%m-%d')}: best of three",
        f"// means of {steps} calls per candidate, CUDA-event timed; an entry replaces the",
        f"// heuristic's plan only when faster by more than {MARGIN:.0%}, otherwise it pins it.",
        "// Fields: family, M, N, K, batch, tile, schedule, slices (0: automatic; split-K",
        "// slices under data-parallel, K slices per tail tile under stream-K).",
        "// Candidates: tile/schedule (dp, sk; sN for N slices) and microseconds.",
    ]
    swept = {r["problem"].name: r for r in results}
    order = [p.name for p in shapes() if p.name in swept or (keep and p.name in keep)]
    for name in order:
        if name not in swept:
            lines.extend(keep[name])
            continue
        r = swept[name]
        p = r["problem"]
        tile, sched, splits, us, how = r["choice"]
        cands = ", ".join(f"{c[0].split('_', 2)[2]}/{'sk' if c[1] == 'stream_k' else 'dp'}"
                          f"{'/s%d' % c[2] if c[2] else ''} {c[3]:.1f}" for c in r["cands"])
        lines.append(f"// {p.name}: heuristic {r['heuristic'][0]}/{r['heuristic'][1]} "
                     f"{r['heuristic_us']:.1f} us; chosen ({how}) {us:.1f} us")
        lines.append(f"//   candidates: {cands}")
        lines.append(f"{{{KERNEL_CONST[r['family']]}, {p.M}, {p.N}, {p.K}, {p.batch}, "
                     f"\"{tile}\", {SCHED_CONST[sched]}, {splits}}},")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "csrc", "tuned_table.inc"))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--only", nargs="*", default=None, help="problem names to sweep")
    ap.add_argument("--update", action="store_true",
                    help="keep the other entries of the existing --out table")
    args = ap.parse_args()
    keep = _entry_blocks(args.out) if args.update and os.path.exists(args.out) else None
    import torch
    if not torch.cuda.is_available():
        print("the tuning sweep needs a GPU", file=sys.stderr)
        sys.exit(1)

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    results = []
    for p in shapes():
        if args.only and p.name not in args.only:
            continue
        r = sweep(p, args.steps, log)
        if r is not None:
            results.append(r)
        torch.cuda.empty_cache()
    write_table(results, args.out, args.steps, torch.cuda.get_device_name(0), keep)
    log(f"[tune] wrote {len(results)} entries to {args.out}")


if __name__ == "__main__":
    main()
