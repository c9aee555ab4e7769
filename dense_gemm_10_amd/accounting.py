"""Algorithmic FLOP and byte accounting for the roofline of a GEMM.

The cost model follows "La GEMM, de zero a cuBLAS", sections 2.1, 2.2 and
2.4: the work is 2MNK flops, the minimum traffic reads every operand once and
writes C once, the intensity is their ratio, and the bound time is work
divided by a peak (or bytes by bandwidth for a memory-bound problem).
Throughput is reported as TFLOPS = 2MNK / t ("GEMM Kernel Optimization",
Verification).

MI355X peaks (AMD's published figures, dense, no sparsity):
  - bf16 and fp16 MFMA 2516.6 TFLOP/s, fp32 (vector and matrix) 157.3 TFLOP/s,
    HBM3E 8 TB/s; 256 compute units at 2.4 GHz.
  - FP32 vector: 256 flop per clock per CU (256 * 256 * 2.4e9 = 157.3
    TFLOP/s), reached on gfx950 by the two-operand accumulate form of the
    fp32 FMA (v_fmac_f32), which issues at twice the rate of the
    three-operand v_fma_f32 without any packed-FP32 instruction.  Measured
    with a loop of independent FMA chains on every CU, with the shader
    clock of each dispatch from GRBM_GUI_ACTIVE: v_fmac_f32 ~234 flop/clk/CU
    at 2.17 GHz, v_fma_f32 ~124 at 2.39 GHz, v_fma_f64 ~119 at 2.30 GHz
    (the fp64 vector peak, 128 flop/clk/CU, 78.6 TFLOP/s).  The vector-FMA
    SGEMM, whose inner loop is v_fmac_f32, is held to the 157.3 figure.
"""
from __future__ import annotations

N_CU = 256
CLOCK_HZ = 2.4e9
PEAK_BF16_MFMA = 2516.6e12          # 256 CU * 4096 flop/clk * 2.4 GHz
PEAK_F16_MFMA = 2516.6e12           # same rate for fp16 inputs
PEAK_F32 = 157.3e12                 # published fp32 vector / matrix peak
PEAK_F32_VALU = N_CU * 256 * CLOCK_HZ            # 157.29e12, fp32 vector (v_fmac_f32)
PEAK_F64_VALU = N_CU * 128 * CLOCK_HZ            # 78.64e12
PEAK_HBM = 8.0e12                   # bytes / s

_ELEM = {"f32": 4, "bf16": 2, "f16": 2}


def flops(M, N, K, batch=1):
    """2MNK per matrix of the batch."""
    return 2.0 * batch * M * N * K


def min_bytes(M, N, K, batch=1, a_bytes=4, b_bytes=4, c_bytes=4, read_c=False,
              a_broadcast=False, b_broadcast=False, bias_bytes=0):
    """Every operand moved once: A and B read (a broadcast operand once for
    the whole batch), C written, C read again when beta != 0, bias read."""
    a = (1 if a_broadcast else batch) * M * K * a_bytes
    b = (1 if b_broadcast else batch) * K * N * b_bytes
    c = batch * M * N * c_bytes * (2 if read_c else 1)
    bias = N * bias_bytes
    return float(a + b + c + bias)


def intensity(M, N, K, **kw):
    return flops(M, N, K, kw.get("batch", 1)) / min_bytes(M, N, K, **kw)


def problem_flops(p):
    return flops(p.M, p.N, p.K, p.batch)


def problem_bytes(p):
    """Algorithmic bytes of a workload Problem (see workloads)."""
    return min_bytes(p.M, p.N, p.K, p.batch,
                     a_bytes=_ELEM[p.a_type], b_bytes=_ELEM[p.b_type],
                     c_bytes=_ELEM[p.c_type], read_c=(p.beta != 0.0),
                     a_broadcast=(p.stride_a_ == 0 and p.batch > 1),
                     b_broadcast=(p.stride_b_ == 0 and p.batch > 1),
                     bias_bytes=_ELEM[p.bias_type] if p.has_bias else 0)


def naive_intensity(elem_bytes=4):
    """One thread per output element, no reuse: per k it reads one element
    of A and one of B (2 * elem_bytes) for one multiply-add (2 flops)."""
    return 2.0 / (2.0 * elem_bytes)


def tiled_intensity(T, elem_bytes=4):
    """Square shared-memory tiles of side T: each element brought from
    global memory is used T times."""
    return T * naive_intensity(elem_bytes)


def bound_time(work_flops, peak_flops):
    return work_flops / peak_flops


def roofline_time(p, peak_flops, peak_bw=PEAK_HBM):
    """max(compute bound, memory bound) for a Problem."""
    return max(problem_flops(p) / peak_flops, problem_bytes(p) / peak_bw)


def compute_peak_for(p):
    """The compute peak that bounds a workload's inner loop on MI355X."""
    if p.a_type == "bf16":
        return PEAK_BF16_MFMA
    if p.a_type == "f16":
        return PEAK_F16_MFMA
    return PEAK_F32
