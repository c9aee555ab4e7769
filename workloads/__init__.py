"""Seeded synthetic inputs for the dense GEMM workloads.

This module is shared by the CPU oracle side (tests, cpu baseline) and the
GPU side (tests, bench).  It holds no GEMM arithmetic: it only draws random
numbers, converts them to the storage dtype with a library cast (torch's CPU
fp32 -> bfloat16 / float16 casts, round-to-nearest-even) and lays the logical matrices
out in memory with the requested order, leading dimension and batch stride.

The problem statement is the one of "La GEMM, de zero a cuBLAS" section 2.1
(C = alpha*A*B + beta*C) together with the inputs listed in "Skill: Write a
Triton GEMM Kernel", section "Inputs the agent should gather first" (sizes,
dtype, per-operand layout, output dtype, epilogue, batch/broadcast).

Seeds: operand ``o`` of workload ``w`` is drawn from
``numpy.random.default_rng([w, o])`` with o = 0 (A), 1 (B), 2 (C_in), 3 (bias).
Uniform U(a, b) is drawn in fp64 and cast to fp32; normal N(0, s) is
``standard_normal * s`` cast to fp32 (s is the standard deviation).  bf16
and fp16 operands are the RNE rounding of those fp32 values.  The "small integer twin"
of a workload draws every operand from {-2, ..., 2} instead.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"
ROW = "row"
COL = "col"

ACT_NONE = "none"
ACT_GELU_ERF = "gelu_erf"
ACT_GELU_TANH = "gelu_tanh"

_ELEM_BYTES = {F32: 4, BF16: 2, F16: 2}


@dataclasses.dataclass(frozen=True)
class Problem:
    """One GEMM problem: shapes, dtypes, layouts and epilogue.

    Layout conventions (element units):
      A is M x K, B is K x N, C is M x N, each ``batch`` times.
      Row-major X with leading dimension ld stores X[r][c] at r*ld + c;
      column-major stores it at c*ld + r.  Matrix b of a batch starts at
      b*stride.  A or B with stride 0 is broadcast to every batch entry.
    """
    name: str
    M: int
    N: int
    K: int
    batch: int = 1
    a_type: str = F32
    b_type: str = F32
    c_type: str = F32
    a_order: str = ROW
    b_order: str = ROW
    c_order: str = ROW
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    stride_a: Optional[int] = None
    stride_b: Optional[int] = None
    stride_c: Optional[int] = None
    alpha: float = 1.0
    beta: float = 0.0
    has_bias: bool = False
    bias_type: str = F32
    act: str = ACT_NONE
    split_k: int = 0
    # distributions: ("uniform", lo, hi) or ("normal", std)
    dist_a: tuple = ("uniform", -1.0, 1.0)
    dist_b: tuple = ("uniform", -1.0, 1.0)
    dist_c: tuple = ("uniform", -1.0, 1.0)
    dist_bias: tuple = ("uniform", -0.5, 0.5)
    seed: int = 0

    # --- derived layout -------------------------------------------------
    def _ld(self, order, rows, cols, given):
        if given is not None:
            return int(given)
        return max(1, cols if order == ROW else rows)

    @property
    def lda_(self):
        return self._ld(self.a_order, self.M, self.K, self.lda)

    @property
    def ldb_(self):
        return self._ld(self.b_order, self.K, self.N, self.ldb)

    @property
    def ldc_(self):
        return self._ld(self.c_order, self.M, self.N, self.ldc)

    @staticmethod
    def _span(order, rows, cols, ld):
        if rows == 0 or cols == 0:
            return 0
        if order == ROW:
            return (rows - 1) * ld + cols
        return (cols - 1) * ld + rows

    def _stride(self, given, span):
        return int(given) if given is not None else span

    @property
    def stride_a_(self):
        return self._stride(self.stride_a, self._span(self.a_order, self.M, self.K, self.lda_))

    @property
    def stride_b_(self):
        return self._stride(self.stride_b, self._span(self.b_order, self.K, self.N, self.ldb_))

    @property
    def stride_c_(self):
        return self._stride(self.stride_c, self._span(self.c_order, self.M, self.N, self.ldc_))

    def buffer_elems(self, which):
        """Number of elements the storage buffer of operand 'a'|'b'|'c' spans."""
        if which == "a":
            span = self._span(self.a_order, self.M, self.K, self.lda_)
            stride = self.stride_a_
        elif which == "b":
            span = self._span(self.b_order, self.K, self.N, self.ldb_)
            stride = self.stride_b_
        else:
            span = self._span(self.c_order, self.M, self.N, self.ldc_)
            stride = self.stride_c_
        if self.batch == 0 or span == 0:
            return 0
        return (self.batch - 1) * stride + span

    def flops(self):
        return 2.0 * self.batch * self.M * self.N * self.K

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


def elem_bytes(dtype):
    return _ELEM_BYTES[dtype]


# ---------------------------------------------------------------------------
# The five workloads.  Layout readings where the statement is silent:
# C4 and C5 use the C3 layout (A row-major, B column-major, C row-major),
# alpha = 1, beta = 0; N(0, 0.5) means standard deviation 0.5; the C4 bias
# is bf16.
# ---------------------------------------------------------------------------
WORKLOADS = {
    "c1": Problem(
        name="sgemm_f32_256", M=256, N=256, K=256,
        a_type=F32, b_type=F32, c_type=F32,
        alpha=1.5, beta=0.5,
        dist_a=("uniform", -1.0, 1.0), dist_b=("uniform", -1.0, 1.0),
        dist_c=("uniform", -1.0, 1.0), seed=1),
    "c2": Problem(
        name="sgemm_f32_4096", M=4096, N=4096, K=4096,
        a_type=F32, b_type=F32, c_type=F32,
        alpha=1.0, beta=0.0,
        dist_a=("uniform", -1.0, 1.0), dist_b=("uniform", -1.0, 1.0), seed=2),
    "c3": Problem(
        name="gemm_bf16_4096", M=4096, N=4096, K=4096,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=ROW, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=3),
    "c4": Problem(
        name="gemm_bf16_4095x4097x1000_bias_gelu", M=4095, N=4097, K=1000,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=ROW, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0, has_bias=True, bias_type=BF16, act=ACT_GELU_ERF,
        dist_a=("normal", 0.5), dist_b=("normal", 0.5),
        dist_bias=("uniform", -0.5, 0.5), seed=4),
    "c5": Problem(
        name="gemm_bf16_batch32_128x128x16384_splitk", M=128, N=128, K=16384,
        batch=32,
        a_type=BF16, b_type=BF16, c_type=F32,
        a_order=ROW, b_order=COL, c_order=ROW,
        stride_b=0,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=5),
    # Shapes for the further steps.  The flat GEMM is the 4096 x 4096 x 16
    # problem of "La GEMM, de zero a cuBLAS" (self-check questions): almost
    # all of its bytes are the output, so it is bound by HBM writes; 2-byte
    # elements as in that question's arithmetic, same layout as C3.  The
    # long-K ragged shape is one where the last wave of 256 x 256 tiles is
    # nearly empty (17 x 17 = 289 tiles on 256 compute units).
    "flat16": Problem(
        name="gemm_bf16_flat_4096x4096x16", M=4096, N=4096, K=16,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=ROW, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=6),
    "flat16_f32": Problem(
        name="sgemm_f32_flat_4096x4096x16", M=4096, N=4096, K=16,
        a_type=F32, b_type=F32, c_type=F32,
        alpha=1.0, beta=0.0,
        dist_a=("uniform", -1.0, 1.0), dist_b=("uniform", -1.0, 1.0), seed=7),
    # fp16 twins of the 4096^3 GEMM and of the ragged GELU GEMM (fp16 is the
    # dtype of the allclose check in "GEMM Kernel Optimization",
    # Verification): same layouts, distributions and sizes.
    "f16_4096": Problem(
        name="gemm_f16_4096", M=4096, N=4096, K=4096,
        a_type=F16, b_type=F16, c_type=F16,
        a_order=ROW, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=9),
    "f16_gelu": Problem(
        name="gemm_f16_4095x4097x1000_bias_gelu", M=4095, N=4097, K=1000,
        a_type=F16, b_type=F16, c_type=F16,
        a_order=ROW, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0, has_bias=True, bias_type=F16, act=ACT_GELU_ERF,
        dist_a=("normal", 0.5), dist_b=("normal", 0.5),
        dist_bias=("uniform", -0.5, 0.5), seed=10),
    # The bf16 4096^3 problem in the other three operand orders (PyTorch's
    # default, both row-major, first): same sizes, values and output.
    "c3_brow": Problem(
        name="gemm_bf16_4096_arow_brow", M=4096, N=4096, K=4096,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=ROW, b_order=ROW, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=3),
    "c3_acol": Problem(
        name="gemm_bf16_4096_acol_bcol", M=4096, N=4096, K=4096,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=COL, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=3),
    "c3_acol_brow": Problem(
        name="gemm_bf16_4096_acol_brow", M=4096, N=4096, K=4096,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=COL, b_order=ROW, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=3),
    # A problem whose operands (128 MiB each) and output exceed the 256 MB
    # Infinity Cache: where the grouped tile order should show in time.
    "big8192": Problem(
        name="gemm_bf16_8192", M=8192, N=8192, K=8192,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=ROW, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=11),
    "tail4352": Problem(
        name="gemm_bf16_4352x4352x8192", M=4352, N=4352, K=8192,
        a_type=BF16, b_type=BF16, c_type=BF16,
        a_order=ROW, b_order=COL, c_order=ROW,
        alpha=1.0, beta=0.0,
        dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=8),
}


# ---------------------------------------------------------------------------
# Drawing values
# ---------------------------------------------------------------------------
def _draw(rng, dist, n, small_int):
    if small_int:
        return rng.integers(-2, 3, size=n).astype(np.float32)
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=n).astype(np.float32)
    if kind == "normal":
        return (rng.standard_normal(size=n) * dist[1]).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def to_storage(values_f32, dtype):
    """fp32 values -> storage array (float32, or uint16 bf16 / fp16 bit
    patterns).

    bf16 and fp16 use torch's CPU casts (round to nearest, ties to even)."""
    values_f32 = np.ascontiguousarray(values_f32, dtype=np.float32)
    if dtype == F32:
        return values_f32
    import torch
    t = torch.from_numpy(values_f32).to(torch.bfloat16 if dtype == BF16 else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def storage_dtype(dtype):
    return np.float32 if dtype == F32 else np.uint16


def _fill_value(dtype, fill):
    if fill is None:
        return 0
    if dtype == F32:
        return np.float32(fill)
    # 16-bit sentinels as bit patterns (a NaN with a payload)
    if isinstance(fill, float) and np.isnan(fill):
        return np.uint16(0x7FC1 if dtype == BF16 else 0x7E01)
    return to_storage(np.array([fill], np.float32), dtype)[0]


def _strided_view(buf, order, ld, base, rows, cols):
    """Writable view of one rows x cols matrix starting at element ``base``."""
    item = buf.itemsize
    strides = (ld * item, item) if order == ROW else (item, ld * item)
    return np.lib.stride_tricks.as_strided(buf[base:], shape=(rows, cols), strides=strides,
                                           writeable=True)


def lay_out(logical, order, ld, stride, n_elems, dtype, fill=None):
    """Place logical matrices [batch][rows][cols] (storage dtype) into a flat
    buffer with the given order / ld / batch stride.  Positions not covered
    by any matrix element hold ``fill`` (0 unless given: NaN sentinels let
    tests see stray reads)."""
    buf = np.full(n_elems, _fill_value(dtype, fill), dtype=storage_dtype(dtype))
    batch, rows, cols = logical.shape
    if n_elems == 0 or rows == 0 or cols == 0:
        return buf
    for b in range(batch):
        _strided_view(buf, order, ld, b * stride, rows, cols)[...] = logical[b]
        if stride == 0:
            break
    return buf


def read_back(buf, order, ld, stride, batch, rows, cols):
    """Inverse of lay_out: gather logical [batch][rows][cols] from a buffer."""
    out = np.empty((batch, rows, cols), dtype=buf.dtype)
    if rows == 0 or cols == 0:
        return out
    for b in range(batch):
        out[b] = _strided_view(buf, order, ld, b * stride, rows, cols)
    return out


@dataclasses.dataclass
class Inputs:
    """Host buffers of one problem instance (storage dtype, flat)."""
    problem: Problem
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray          # C_in (also the output buffer's initial content)
    bias: Optional[np.ndarray]
    # logical operands (storage dtype) for tests that index them directly
    A_log: np.ndarray
    B_log: np.ndarray
    C_log: np.ndarray


def make_inputs(p: Problem, small_int=False, fill=None, c_fill=None, seed=None):
    """Draw the operands of ``p`` and lay them out.

    ``fill`` is written to every position of the A/B/C buffers that no
    matrix element covers (padding beyond the extent, gaps between batch
    entries).  ``c_fill`` (if given) replaces the drawn C_in values."""
    seed = p.seed if seed is None else seed
    a_batches = 1 if p.stride_a_ == 0 else p.batch
    b_batches = 1 if p.stride_b_ == 0 else p.batch
    rng = np.random.default_rng([seed, 0])
    A_log = to_storage(_draw(rng, p.dist_a, a_batches * p.M * p.K, small_int), p.a_type)
    A_log = A_log.reshape(a_batches, p.M, p.K)
    rng = np.random.default_rng([seed, 1])
    B_log = to_storage(_draw(rng, p.dist_b, b_batches * p.K * p.N, small_int), p.b_type)
    B_log = B_log.reshape(b_batches, p.K, p.N)
    rng = np.random.default_rng([seed, 2])
    if c_fill is None:
        C_log = to_storage(_draw(rng, p.dist_c, p.batch * p.M * p.N, small_int), p.c_type)
    else:
        C_log = np.full(p.batch * p.M * p.N, _fill_value(p.c_type, c_fill),
                        dtype=storage_dtype(p.c_type))
    C_log = C_log.reshape(p.batch, p.M, p.N)
    bias = None
    if p.has_bias:
        rng = np.random.default_rng([seed, 3])
        bias = to_storage(_draw(rng, p.dist_bias, p.N, small_int), p.bias_type)
    A = lay_out(A_log, p.a_order, p.lda_, p.stride_a_, p.buffer_elems("a"), p.a_type, fill)
    B = lay_out(B_log, p.b_order, p.ldb_, p.stride_b_, p.buffer_elems("b"), p.b_type, fill)
    C = lay_out(C_log, p.c_order, p.ldc_, p.stride_c_, p.buffer_elems("c"), p.c_type, fill)
    return Inputs(p, A, B, C, bias, A_log, B_log, C_log)


def sample_points(p: Problem, n, seed=12345):
    """Seeded output coordinates (b, i, j) for sampled parity checks at full
    size.  Always includes the four corners of the first and last batch entry
    so ragged edges are covered."""
    rng = np.random.default_rng([seed, p.M, p.N, p.K, p.batch])
    b = rng.integers(0, max(p.batch, 1), size=n)
    i = rng.integers(0, max(p.M, 1), size=n)
    j = rng.integers(0, max(p.N, 1), size=n)
    corners = []
    for bb in {0, p.batch - 1}:
        for ii in {0, p.M - 1}:
            for jj in {0, p.N - 1}:
                corners.append((bb, ii, jj))
    cb, ci, cj = (np.array(x, dtype=np.int64) for x in zip(*corners))
    return (np.concatenate([cb, b]).astype(np.int64),
            np.concatenate([ci, i]).astype(np.int64),
            np.concatenate([cj, j]).astype(np.int64))


def desc_fields(p: Problem):
    """The descriptor fields of a Problem, as plain values (names follow the
    library's descriptor)."""
    return dict(M=p.M, N=p.N, K=p.K, batch=p.batch, a_type=p.a_type, b_type=p.b_type,
                c_type=p.c_type, a_order=p.a_order, b_order=p.b_order, c_order=p.c_order,
                lda=p.lda_, ldb=p.ldb_, ldc=p.ldc_, stride_a=p.stride_a_,
                stride_b=p.stride_b_, stride_c=p.stride_c_, alpha=p.alpha, beta=p.beta,
                bias_type=p.bias_type, act=p.act, split_k=p.split_k)
