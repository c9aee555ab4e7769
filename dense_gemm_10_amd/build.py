"""Build libdensegemm.so (gfx950) in-tree with hipcc.

    python -m dense_gemm_10_amd.build        # or dense_gemm_10_amd.build.build()

Every HIP source is compiled for gfx950 only, with packed-FP32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into
one shared library next to this file.

Measurement builds with compile-time options go elsewhere:

    python -m dense_gemm_10_amd.build --define DG_LOAD_POLICY_A=nt --out /tmp/lib_nt.so

and are loaded instead of the in-tree library when DG_LIBRARY names them.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdensegemm.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE,
]

SOURCES = [
    "api.cpp",
    "kernel_generic.hip",
    "kernel_valu_f32.hip",
    "kernel_mfma16.hip",
    "kernel_mfma16_bf16a.hip",
    "kernel_mfma16_bf16b.hip",
    "kernel_mfma16_f16a.hip",
    "kernel_mfma16_f16b.hip",
    "kernel_mfma16_mn256.hip",
    "kernel_mfma16_mn128.hip",
    "kernel_mfma_f32.hip",
    "tiles_f32.cpp",
    "kernel_sliver.hip",
]


def _compile(src, defines=(), obj_dir=OUT_DIR):
    path = os.path.join(CSRC, src)
    obj = os.path.join(obj_dir, src + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + [f"-D{d}" for d in defines] + ["-x", "hip", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, defines=(), out=None):
    """Compile and link; `defines` (NAME or NAME=VALUE) are passed to every
    compile, `out` replaces the in-tree library path."""
    defines = tuple(defines)
    lib = out or LIB
    obj_dir = OUT_DIR if not defines else os.path.join(OUT_DIR, "opt_" + "_".join(
        d.replace("=", "-") for d in defines))
    os.makedirs(obj_dir, exist_ok=True)
    workers = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, defines, obj_dir), SOURCES))
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--define", action="append", default=[],
                    help="NAME or NAME=VALUE passed to every compile (measurement builds)")
    ap.add_argument("--out", default=None, help="library path (default: in-tree)")
    a = ap.parse_args()
    build(verbose=True, defines=a.define, out=a.out)
    sys.exit(0)
