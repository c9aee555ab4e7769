"""AddressSanitizer and UndefinedBehaviorSanitizer over the host code: the
library's validation, planning, description and tile-scheduler map (built
host-only, so no GPU code is involved), and the CPU oracle.  Each runs a
battery of calls in a child process with the sanitizer runtime preloaded;
any report aborts the child, and its results must equal those of the
normal builds."""
import glob
import json
import os
import subprocess
import sys
import tempfile

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "dense_gemm_10_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"


def _clang_asan_runtime():
    libs = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return libs[0] if libs else None


def _gcc_asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

# The host-code battery, run by the child against DG_LIBRARY: every entry
# point that needs no GPU, on valid and invalid descriptors.
HOST_BATTERY = r'''
import json, sys
sys.path.insert(0, ROOT)
import dense_gemm_10_amd as dg
out = []
A, B, C, W = 1 << 40, 2 << 40, 3 << 40, 4 << 40
def rec(f, *a, **k):
    try:
        out.append(["ok", f(*a, **k)])
    except dg.DgError as e:
        out.append(["err", e.status])
shapes = [(1, 1, 1), (7, 5, 3), (300, 260, 200), (4095, 4097, 1000), (4096, 4096, 4096),
          (128, 128, 16384), (0, 5, 5), (5, 0, 5), (5, 5, 0), (4096, 4096, 16), (1, 8193, 8)]
for (M, N, K) in shapes:
    for at, ct in (("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16")):
        for ao in ("row", "col"):
            for bo in ("row", "col"):
                for extra in ({}, {"split_k": 4}, {"schedule": 2}, {"batch": 3, "stride_b": 0},
                              {"act": "gelu_erf", "alpha": 1.5, "beta": 0.5}, {"group_m": 1},
                              {"xcd_remap": -1}, {"algo": 1}):
                    kw = dict(a_type=at, c_type=ct, a_order=ao, b_order=bo)
                    kw.update(extra)
                    d = dg.make_desc(M, N, K, **kw)
                    rec(dg.dg_gemm_workspace_size, d)
                    for ws in (0, 1 << 20, 1 << 34):
                        rec(dg.dg_gemm_describe, d, ws)
                    out.append(["st", dg.dg_gemm(d, A, B, None, None, 0, None, check=False)])
for bad in ({"M": -1}, {"K": -3}, {"lda": 0}, {"split_k": 1000}, {"group_m": -2},
            {"xcd_remap": 5}, {"algo": 9}, {"schedule": 7}, {"act": 9}):
    kw = dict(M=64, N=48, K=32)
    kw.update(bad)
    d = dg.make_desc(**kw)
    rec(dg.dg_gemm_workspace_size, d)
    out.append(["st", dg.dg_gemm(d, A, B, C, None, 0, None, check=False)])
    out.append(["st", dg.dg_gemm_noalloc(d, A, B, C, None, check=False)])
big = dg.make_desc(4096, 4096, 4096, split_k=2)
out.append(["st", dg.dg_gemm_noalloc(big, A, B, C, None, check=False)])
for (M, N, b, s, bm, bn, g, r) in [(4096, 4096, 1, 1, 256, 256, 0, 0), (4095, 4097, 1, 1, 128, 256, 8, -1),
                                   (128, 128, 32, 8, 128, 128, 4, 0), (1000, 1, 3, 2, 64, 64, 16, -1),
                                   (40 * 64, 39 * 64, 1, 1, 64, 64, 5, 0)]:
    out.append(["map", dg.dg_schedule_map(M, N, b, s, bm, bn, g, r).tolist()])
print(json.dumps(out))
'''

ORACLE_BATTERY = r'''
import json, sys
sys.path.insert(0, ROOT)
import numpy as np
import oracle
import workloads as W
out = []
rng = np.random.default_rng(5)
for (M, N, K, batch) in [(5, 7, 3, 1), (17, 9, 33, 2), (64, 48, 100, 1), (1, 1, 0, 1), (3, 4, 5, 0)]:
    for ao in (W.ROW, W.COL):
        for bo in (W.ROW, W.COL):
            for act in (W.ACT_NONE, W.ACT_GELU_ERF, W.ACT_GELU_TANH):
                p = W.Problem(name="san", M=M, N=N, K=K, batch=batch, a_order=ao, b_order=bo,
                              c_order=W.COL if ao == W.COL else W.ROW, alpha=1.25, beta=0.5,
                              has_bias=True, act=act, seed=3)
                x = W.make_inputs(p)
                ref, mag, o = oracle.gemm(p, x.A, x.B, x.C, x.bias)
                out.append([ref.tolist(), mag.tolist(), o.tolist()])
                if batch and M and N:
                    pts = W.sample_points(p, 20)
                    r2, m2, o2 = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
                    out.append([r2.tolist(), m2.tolist(), o2.tolist()])
for v in rng.standard_normal(200).tolist() + [0.0, -0.0, 65504.0, 65520.0, 1e-8, 3.0e38]:
    out.append([oracle.round_bf16(v), oracle.round_f16(v), oracle.act(v, "gelu_erf"),
                oracle.act(v, "gelu_tanh")])
print(json.dumps(out))
'''


def _run_battery(code, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + code], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stderr[-4000:]}"
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and _clang_asan_runtime()),
                    reason="no hipcc / clang ASan runtime")
def test_host_library_code_under_asan_and_ubsan():
    # Every source with host logic (ABI, validation, planning, tile tables,
    # dispatch); the launchers of the two kernel families whose device code
    # takes minutes to build come from tests/sanitizer_stubs.hip.  Device
    # code is still compiled (the host registers it), at -O1 for time.
    sources = [os.path.join(CSRC, f) for f in (
        "api.cpp", "kernel_generic.hip", "kernel_valu_f32.hip", "kernel_mfma16.hip",
        "kernel_sliver.hip", "tiles_f32.cpp")]
    sources.append(os.path.join(ROOT, "tests", "sanitizer_stubs.hip"))
    with tempfile.TemporaryDirectory() as d:
        objs = []
        procs = []
        for src in sources:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host",
                   "-fno-sanitize-recover=all", "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE))
            objs.append(obj)
        for pr in procs:
            _, err = pr.communicate(timeout=600)
            assert pr.returncode == 0, err.decode()[-3000:]
        lib = os.path.join(d, "libdensegemm_san.so")
        # linked by clang++ with the shared sanitizer runtime
        subprocess.run([CLANGXX, "-shared", "-fPIC", "-shared-libasan",
                        "-fsanitize=address,undefined", "-o", lib] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                       check=True, capture_output=True)
        san = _run_battery(HOST_BATTERY, dict(SAN_ENV, DG_LIBRARY=lib,
                                              LD_PRELOAD=_clang_asan_runtime()))
    plain = _run_battery(HOST_BATTERY, {"DG_LIBRARY": os.path.join(ROOT, "dense_gemm_10_amd",
                                                                    "libdensegemm.so")})
    assert san == plain


@pytest.mark.skipif(_gcc_asan_runtime() is None, reason="no gcc ASan runtime")
def test_oracle_under_asan_and_ubsan():
    src = os.path.join(ROOT, "oracle", "oracle.c")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                        "-fopenmp", "-fPIC", "-shared", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", src, "-o", lib,
                        "-lm"], check=True, capture_output=True)
        san = _run_battery(ORACLE_BATTERY, dict(SAN_ENV, DG_ORACLE_LIBRARY=lib,
                                                LD_PRELOAD=_gcc_asan_runtime()))
    plain = _run_battery(ORACLE_BATTERY, {})
    assert san == plain
