"""CPU oracle for C = act(alpha*A*B + beta*C + bias): TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.  The arithmetic lives in ``oracle.c`` (plain C,
float64, one thread per output element); this module only builds that file
with gcc and marshals arguments to it.

Every function here is pinned by CPU tests against values fixed by the
mathematics (exact integer and rational results, identity / permutation /
rank-one closed forms, standard-normal table values for GELU, hand-worked
bf16 and fp16 rounding cases) rather than against itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# DG_ORACLE_LIBRARY may name another build of oracle.c (the sanitizer test's)
_LIB = os.environ.get("DG_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")

_DT = {"f32": 0, "bf16": 1, "f16": 2}
_ACT = {"none": 0, "gelu_erf": 1, "gelu_tanh": 2}

_lock = threading.Lock()
_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("batch", ctypes.c_int64),
        ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32),
        ("c_type", ctypes.c_int32), ("bias_type", ctypes.c_int32),
        ("a_col", ctypes.c_int32), ("b_col", ctypes.c_int32), ("c_col", ctypes.c_int32),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
        ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64),
        ("stride_c", ctypes.c_int64),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double),
        ("has_bias", ctypes.c_int32), ("act", ctypes.c_int32),
    ]


def build(force=False):
    """Compile oracle.c with gcc (plain -O2, no FMA contraction, OpenMP)."""
    if os.environ.get("DG_ORACLE_LIBRARY"):
        return _LIB                     # another build, made by its user
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.POINTER(_Problem)
            vp = ctypes.c_void_p
            lib.oracle_gemm.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32]
            lib.oracle_gemm.restype = ctypes.c_int
            lib.oracle_gemm_points.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                               vp, vp, vp, ctypes.c_int32]
            lib.oracle_gemm_points.restype = ctypes.c_int
            lib.oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.oracle_round_bf16.restype = ctypes.c_uint16
            lib.oracle_round_f16.argtypes = [ctypes.c_double]
            lib.oracle_round_f16.restype = ctypes.c_uint16
            lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_f16_to_double.restype = ctypes.c_double
            lib.oracle_act.argtypes = [ctypes.c_double, ctypes.c_int32]
            lib.oracle_act.restype = ctypes.c_double
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _problem(p):
    return _Problem(
        M=p.M, N=p.N, K=p.K, batch=p.batch,
        a_type=_DT[p.a_type], b_type=_DT[p.b_type], c_type=_DT[p.c_type],
        bias_type=_DT[p.bias_type],
        a_col=int(p.a_order == "col"), b_col=int(p.b_order == "col"),
        c_col=int(p.c_order == "col"),
        lda=p.lda_, ldb=p.ldb_, ldc=p.ldc_,
        stride_a=p.stride_a_, stride_b=p.stride_b_, stride_c=p.stride_c_,
        alpha=float(p.alpha), beta=float(p.beta),
        has_bias=int(bool(p.has_bias)), act=_ACT[p.act])


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _out_dtype(p):
    return np.float32 if p.c_type == "f32" else np.uint16


def gemm(p, A, B, C, bias=None, nthreads=0):
    """Evaluate every output element.

    A, B, C, bias are flat storage buffers (float32, or uint16 bf16 / fp16 bits) laid
    out as ``p`` describes.  Returns (ref, mag, out), each dense
    [batch][M][N]: ref = the float64 result before output rounding,
    mag = |alpha| sum_k |a||b| + |beta||c| + |bias| (the error scale),
    out = ref rounded to the output dtype (float32, or bf16 / fp16 bits)."""
    lib = _load()
    shape = (p.batch, p.M, p.N)
    ref = np.empty(shape, np.float64)
    mag = np.empty(shape, np.float64)
    out = np.empty(shape, _out_dtype(p))
    pr = _problem(p)
    rc = lib.oracle_gemm(ctypes.byref(pr), _ptr(A), _ptr(B), _ptr(C), _ptr(bias),
                         _ptr(ref), _ptr(mag), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm rejected the problem")
    return ref, mag, out


def gemm_points(p, A, B, C, bias, pb, pi, pj, nthreads=0):
    """Evaluate only the elements (pb[t], pi[t], pj[t]); returns 1-D
    (ref, mag, out) indexed by t."""
    lib = _load()
    pb = np.ascontiguousarray(pb, np.int64)
    pi = np.ascontiguousarray(pi, np.int64)
    pj = np.ascontiguousarray(pj, np.int64)
    n = pb.shape[0]
    ref = np.empty(n, np.float64)
    mag = np.empty(n, np.float64)
    out = np.empty(n, _out_dtype(p))
    pr = _problem(p)
    rc = lib.oracle_gemm_points(ctypes.byref(pr), _ptr(A), _ptr(B), _ptr(C), _ptr(bias),
                                _ptr(pb), _ptr(pi), _ptr(pj), n,
                                _ptr(ref), _ptr(mag), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm_points rejected the problem")
    return ref, mag, out


def round_bf16(x):
    """float64 -> bf16 bit pattern (round to nearest, ties to even)."""
    return int(_load().oracle_round_bf16(float(x)))


def round_f16(x):
    """float64 -> IEEE binary16 bit pattern (round to nearest, ties to even)."""
    return int(_load().oracle_round_f16(float(x)))


def f16_to_float(bits):
    """Decode one binary16 bit pattern to float64 (exact), as the oracle does."""
    return float(_load().oracle_f16_to_double(int(bits)))


def act(x, kind):
    return float(_load().oracle_act(float(x), _ACT[kind]))


def max_threads():
    return int(_load().oracle_max_threads())


def bf16_bits_to_float(bits):
    """Decode bf16 bit patterns (uint16 array) to float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_float(bits):
    """Decode fp16 bit patterns (uint16 array) to float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bits_to_float(bits, dtype):
    """Decode a stored output buffer of dtype 'f32' / 'bf16' / 'f16' to float64."""
    if dtype == "f32":
        return np.asarray(bits, np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_float(bits)
    return f16_bits_to_float(bits)
