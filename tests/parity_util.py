"""Comparison of GPU results with the oracle, to the acceptance rules:

  fp32 output:  |gpu - ref| <= 1e-4 * mag elementwise, where ref is the
                oracle's float64 result and mag = |alpha| sum_k |a||b| +
                |beta||c| + |bias| (so mag == 0 forces an exact 0);
  bf16 / fp16 output:
                |gpu - r| <= 1e-2 + 1e-2 |r| with r = the oracle's result
                rounded to the output dtype (torch.allclose form, reference
                in the rtol term; the pages state it for fp16);
  small-integer inputs without a transcendental epilogue: exact equality
                with the oracle's rounded output.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W

F32_RTOL_MAG = 1e-4
BF16_ATOL = 1e-2
BF16_RTOL = 1e-2


def gather(p, c_flat, pts=None):
    """Logical C values [batch][M][N] (or at points) from a flat C buffer,
    decoded to float64."""
    if pts is None:
        v = W.read_back(c_flat, p.c_order, p.ldc_, p.stride_c_, p.batch, p.M, p.N)
    else:
        pb, pi, pj = pts
        off = (pi * p.ldc_ + pj) if p.c_order == W.ROW else (pj * p.ldc_ + pi)
        v = c_flat[pb * p.stride_c_ + off]
    return oracle.bits_to_float(v, p.c_type)


def check(p, c_flat, ref, mag, out, pts=None, exact=False, what=""):
    got = gather(p, c_flat, pts)
    want = oracle.bits_to_float(out, p.c_type)
    both_nan = np.isnan(got) & np.isnan(want)
    if exact:
        bad = ~((got == want) | both_nan)
        _report(bad, got, want, what, "exact")
        return
    if p.c_type == W.F32:
        err = np.abs(got - ref)
        bad = ~((err <= F32_RTOL_MAG * mag) | both_nan | (got == ref))
    else:
        err = np.abs(got - want)
        bad = ~((err <= BF16_ATOL + BF16_RTOL * np.abs(want)) | both_nan | (got == want))
    _report(bad, got, want, what, "tolerance")


def _report(bad, got, want, what, kind):
    n = int(np.count_nonzero(bad))
    if n:
        idx = np.argwhere(bad)[:5]
        details = [(tuple(int(v) for v in i), float(got[tuple(i)]), float(want[tuple(i)]))
                   for i in idx]
        raise AssertionError(f"{what}: {n} of {bad.size} outputs fail the {kind} check; "
                             f"first (index, gpu, oracle): {details}")
