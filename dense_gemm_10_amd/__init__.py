"""Python binding of the MI355X dense GEMM library (libdensegemm.so).

Argument marshalling only: every step of the GEMM runs in the HIP kernels
behind the C ABI declared in include/densegemm.h.  The functions below carry
the ABI's names (dg_gemm, dg_gemm_workspace_size, dg_gemm_describe,
dg_status_string, dg_version, dg_schedule_map, dg_gemm_noalloc).  ``gemm()`` is a
convenience wrapper for torch tensors; torch is used for device memory and
streams only.

The shared library is built in-tree by ``dense_gemm_10_amd.build``; if it is
missing, loading raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "DG_F32", "DG_BF16", "DG_F16", "DG_ROW_MAJOR", "DG_COL_MAJOR",
    "DG_ACT_NONE", "DG_ACT_GELU_ERF", "DG_ACT_GELU_TANH",
    "DG_ALGO_AUTO", "DG_ALGO_GENERIC", "DG_ALGO_VALU_F32", "DG_ALGO_MFMA_BF16",
    "DG_ALGO_MFMA_F32", "DG_ALGO_MFMA_F16", "DgGemmDesc", "DgError", "make_desc", "dg_version",
    "dg_status_string", "dg_gemm_workspace_size", "dg_gemm", "dg_gemm_describe",
    "dg_schedule_map", "dg_gemm_noalloc", "DG_NOALLOC_SCRATCH_BYTES", "gemm", "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# DG_LIBRARY may name another build of the same sources (a measurement
# build with compile-time options); by default the in-tree library.
_LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(_HERE, "libdensegemm.so")

# status codes
DG_SUCCESS = 0
DG_ERROR_INVALID_VALUE = 1
DG_ERROR_NOT_SUPPORTED = 2
DG_ERROR_INSUFFICIENT_WORKSPACE = 3
DG_ERROR_LAUNCH = 4
# enums
DG_F32, DG_BF16, DG_F16 = 0, 1, 2
DG_ROW_MAJOR, DG_COL_MAJOR = 0, 1
DG_ACT_NONE, DG_ACT_GELU_ERF, DG_ACT_GELU_TANH = 0, 1, 2
(DG_ALGO_AUTO, DG_ALGO_GENERIC, DG_ALGO_VALU_F32, DG_ALGO_MFMA_BF16, DG_ALGO_MFMA_F32,
 DG_ALGO_MFMA_F16) = range(6)
DG_SCHED_AUTO, DG_SCHED_DATA_PARALLEL, DG_SCHED_STREAM_K = range(3)
DG_NOALLOC_SCRATCH_BYTES = 64 << 20     # per-GPU scratch of dg_gemm_noalloc

_DTYPE = {"f32": DG_F32, "bf16": DG_BF16, "f16": DG_F16}
_ORDER = {"row": DG_ROW_MAJOR, "col": DG_COL_MAJOR}
_ACT = {"none": DG_ACT_NONE, "gelu_erf": DG_ACT_GELU_ERF, "gelu_tanh": DG_ACT_GELU_TANH}


class DgGemmDesc(ctypes.Structure):
    """Mirror of dg_gemm_desc (include/densegemm.h)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32), ("c_type", ctypes.c_int32),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("batch", ctypes.c_int64),
        ("a_order", ctypes.c_int32), ("b_order", ctypes.c_int32), ("c_order", ctypes.c_int32),
        ("bias_type", ctypes.c_int32),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
        ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64), ("stride_c", ctypes.c_int64),
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
        ("bias", ctypes.c_void_p),
        ("act", ctypes.c_int32), ("split_k", ctypes.c_int32), ("group_m", ctypes.c_int32),
        ("algo", ctypes.c_int32), ("xcd_remap", ctypes.c_int32), ("schedule", ctypes.c_int32),
    ]


class DgError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {dg_status_string(status)}")


_lock = threading.Lock()
_lib = None


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build it with `python -m dense_gemm_10_amd.build` "
                    "(there is no fallback implementation)")
            lib = ctypes.CDLL(_LIB_PATH)
            D = ctypes.POINTER(DgGemmDesc)
            vp = ctypes.c_void_p
            lib.dg_version.restype = ctypes.c_int
            lib.dg_status_string.argtypes = [ctypes.c_int]
            lib.dg_status_string.restype = ctypes.c_char_p
            lib.dg_gemm_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
            lib.dg_gemm_workspace_size.restype = ctypes.c_int
            lib.dg_gemm.argtypes = [D, vp, vp, vp, vp, ctypes.c_size_t, vp]
            lib.dg_gemm.restype = ctypes.c_int
            lib.dg_gemm_noalloc.argtypes = [D, vp, vp, vp, vp]
            lib.dg_gemm_noalloc.restype = ctypes.c_int
            lib.dg_gemm_describe.argtypes = [D, ctypes.c_size_t, ctypes.c_char_p, ctypes.c_size_t]
            lib.dg_gemm_describe.restype = ctypes.c_int
            lib.dg_schedule_map.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int64]
            lib.dg_schedule_map.restype = ctypes.c_int
            _lib = lib
    return _lib


def _enum(table, v):
    return table[v] if isinstance(v, str) else int(v)


def make_desc(M, N, K, batch=1, a_type="f32", b_type=None, c_type=None,
              a_order="row", b_order="row", c_order="row", lda=None, ldb=None, ldc=None,
              stride_a=None, stride_b=None, stride_c=None, alpha=1.0, beta=0.0,
              bias=None, bias_type="f32", act="none", split_k=0, group_m=0, algo=0,
              xcd_remap=0, schedule=0):
    """Fill a DgGemmDesc.  Leading dimensions default to the packed value
    and batch strides to the packed matrix size; ``bias`` is a device
    address (int) or None."""
    b_type = a_type if b_type is None else b_type
    c_type = a_type if c_type is None else c_type
    ao, bo, co = _enum(_ORDER, a_order), _enum(_ORDER, b_order), _enum(_ORDER, c_order)
    if lda is None:
        lda = max(1, K if ao == DG_ROW_MAJOR else M)
    if ldb is None:
        ldb = max(1, N if bo == DG_ROW_MAJOR else K)
    if ldc is None:
        ldc = max(1, N if co == DG_ROW_MAJOR else M)
    if stride_a is None:
        stride_a = M * K
    if stride_b is None:
        stride_b = K * N
    if stride_c is None:
        stride_c = M * N
    d = DgGemmDesc()
    d.struct_size = ctypes.sizeof(DgGemmDesc)
    d.a_type, d.b_type, d.c_type = _enum(_DTYPE, a_type), _enum(_DTYPE, b_type), _enum(_DTYPE, c_type)
    d.M, d.N, d.K, d.batch = M, N, K, batch
    d.a_order, d.b_order, d.c_order = ao, bo, co
    d.bias_type = _enum(_DTYPE, bias_type)
    d.lda, d.ldb, d.ldc = lda, ldb, ldc
    d.stride_a, d.stride_b, d.stride_c = stride_a, stride_b, stride_c
    d.alpha, d.beta = alpha, beta
    d.bias = bias
    d.act = _enum(_ACT, act)
    d.split_k, d.group_m, d.algo, d.xcd_remap = split_k, group_m, algo, xcd_remap
    d.schedule = schedule
    return d


# ---- the C ABI, one function per entry point ----------------------------------
def dg_version():
    return int(_load().dg_version())


def dg_status_string(status):
    return _load().dg_status_string(int(status)).decode()


def dg_gemm_workspace_size(desc):
    n = ctypes.c_size_t(0)
    st = _load().dg_gemm_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != DG_SUCCESS:
        raise DgError(st, "dg_gemm_workspace_size")
    return int(n.value)


def dg_gemm(desc, A, B, C, workspace=None, workspace_bytes=0, stream=None, check=True):
    """Enqueue the GEMM.  A, B, C, workspace: device addresses (int) or None;
    stream: a hipStream_t as int (None = null stream).  Returns the status;
    raises DgError on failure when ``check``."""
    st = _load().dg_gemm(ctypes.byref(desc), A, B, C, workspace, int(workspace_bytes), stream)
    if check and st != DG_SUCCESS:
        raise DgError(st, "dg_gemm")
    return st


def dg_gemm_noalloc(desc, A, B, C, stream=None, check=True):
    """Enqueue the GEMM with the library's own per-GPU scratch as workspace
    (no allocation).  Same arguments as dg_gemm minus the workspace."""
    st = _load().dg_gemm_noalloc(ctypes.byref(desc), A, B, C, stream)
    if check and st != DG_SUCCESS:
        raise DgError(st, "dg_gemm_noalloc")
    return st


def dg_gemm_describe(desc, workspace_bytes=0):
    buf = ctypes.create_string_buffer(512)
    st = _load().dg_gemm_describe(ctypes.byref(desc), int(workspace_bytes), buf, len(buf))
    if st != DG_SUCCESS:
        raise DgError(st, "dg_gemm_describe")
    return buf.value.decode()


def dg_schedule_map(M, N, batch, split_k, bm, bn, group_m=0, xcd_remap=0):
    """Host evaluation of the kernels' program -> (b, s, pid_m, pid_n) map;
    returns a numpy int32 array of shape (P, 4)."""
    import numpy as np
    P = batch * split_k * (-(-M // bm)) * (-(-N // bn))
    out = np.zeros((max(P, 1), 4), np.int32)
    st = _load().dg_schedule_map(M, N, batch, split_k, bm, bn, group_m, xcd_remap,
                                 out.ctypes.data, out.size)
    if st != DG_SUCCESS:
        raise DgError(st, "dg_schedule_map")
    return out[:P]


# ---- torch convenience -----------------------------------------------------------
def _torch_dtype_name(t):
    import torch
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float16:
        return "f16"
    raise TypeError(f"unsupported dtype {t.dtype}")


def _layout(t, rows, cols):
    """(order, ld, batch_stride) of a 2-D or 3-D tensor; raises on a stride
    pattern that is neither row- nor column-major (no silent copy)."""
    s = t.stride()
    bs = s[0] if t.dim() == 3 else 0
    r, c = s[-2], s[-1]
    if c == 1 and (r >= max(1, cols) or rows <= 1):
        return "row", max(r, cols, 1), bs
    if r == 1 and (c >= max(1, rows) or cols <= 1):
        return "col", max(c, rows, 1), bs
    raise ValueError(f"tensor strides {tuple(s)} are neither row- nor column-major; "
                     "pass a contiguous tensor or its transpose")


def gemm(A, B, C=None, *, alpha=1.0, beta=0.0, bias=None, act="none", out_dtype=None,
         split_k=0, group_m=0, algo=0, xcd_remap=0, workspace=None, stream=None):
    """C = act(alpha * A @ B + beta * C + bias) on the current HIP stream.

    A: (M, K) or (batch, M, K); B: (K, N) or (batch, K, N); a batch
    stride of 0 (``expand``) broadcasts.  Returns C (allocated when None)."""
    import torch
    batched = A.dim() == 3 or B.dim() == 3
    batch = A.shape[0] if A.dim() == 3 else (B.shape[0] if B.dim() == 3 else 1)
    M, K = A.shape[-2], A.shape[-1]
    K2, N = B.shape[-2], B.shape[-1]
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    at = _torch_dtype_name(A)
    if out_dtype is None:
        out_dtype = A.dtype
    if C is None:
        shape = (batch, M, N) if batched else (M, N)
        C = torch.empty(shape, dtype=out_dtype, device=A.device)
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
    ao, lda, sa = _layout(A, M, K)
    bo, ldb, sb = _layout(B, K, N)
    co, ldc, sc = _layout(C, M, N)
    if C.dim() == 2 and batched:
        raise ValueError("batched product needs a 3-D C")
    desc = make_desc(M, N, K, batch, a_type=at, b_type=_torch_dtype_name(B),
                     c_type=_torch_dtype_name(C), a_order=ao, b_order=bo, c_order=co,
                     lda=lda, ldb=ldb, ldc=ldc, stride_a=sa, stride_b=sb,
                     stride_c=sc if C.dim() == 3 else M * N,
                     alpha=alpha, beta=beta,
                     bias=bias.data_ptr() if bias is not None else None,
                     bias_type=_torch_dtype_name(bias) if bias is not None else "f32",
                     act=act, split_k=split_k, group_m=group_m, algo=algo, xcd_remap=xcd_remap)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    ws_ptr, ws_bytes = None, 0
    if split_k != 1:
        need = dg_gemm_workspace_size(desc)
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    dg_gemm(desc, A.data_ptr(), B.data_ptr(), C.data_ptr(), ws_ptr, ws_bytes, stream)
    return C
