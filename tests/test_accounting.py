"""Pins of the benchmark's FLOP / byte accounting against the figures printed
in "La GEMM, de zero a cuBLAS" (sections 2.1, 2.2, 2.4 and the self-check
questions), stored with their citations in tests/golden/cost_model.txt."""
import pytest

import workloads as W
from conftest import read_golden
from dense_gemm_10_amd import accounting as acc

H100_F32 = 67e12
H100_BF16 = 990e12
H100_BW = 3.35e12


def _computed():
    n = 4096
    return {
        "flops_4096": acc.flops(n, n, n),
        "min_bytes_f32_4096": acc.min_bytes(n, n, n),
        "intensity_f32_4096": acc.intensity(n, n, n),
        "ridge_h100_f32": H100_F32 / H100_BW,
        "bound_ms_h100_f32": acc.bound_time(acc.flops(n, n, n), H100_F32) * 1e3,
        "bound_us_h100_bf16": acc.bound_time(acc.flops(n, n, n), H100_BF16) * 1e6,
        "naive_intensity_f32": acc.naive_intensity(4),
        "naive_tflops_h100": acc.naive_intensity(4) * H100_BW / 1e12,
        "tiled_intensity_T32": acc.tiled_intensity(32, 4),
        "flat_intensity_16": acc.intensity(4096, 4096, 16, a_bytes=2, b_bytes=2, c_bytes=2),
    }


def test_cost_model_matches_page_figures():
    got = _computed()
    rows = read_golden("cost_model.txt")
    assert {r[0] for r in rows} == set(got)
    for key, value, rtol, *_ in rows:
        v, t = float(value), float(rtol)
        g = got[key]
        if key == "bound_us_h100_bf16":
            # the page truncates 138.8 to 138
            assert 138.0 <= g < 139.0
            continue
        assert abs(g - v) <= t * abs(v) + 1e-12, (key, g, v)


def test_exact_work_value():
    assert acc.flops(4096, 4096, 4096) == 137438953472.0
    assert acc.min_bytes(4096, 4096, 4096) == 201326592.0


def test_workload_accounting():
    c2 = W.WORKLOADS["c2"]
    assert acc.problem_bytes(c2) == 3 * 4096 * 4096 * 4
    c3 = W.WORKLOADS["c3"]
    assert acc.problem_bytes(c3) == 3 * 4096 * 4096 * 2
    c1 = W.WORKLOADS["c1"]          # beta != 0: C is read as well
    assert acc.problem_bytes(c1) == 4 * 256 * 256 * 4
    c5 = W.WORKLOADS["c5"]          # B broadcast: read once for the batch
    assert acc.problem_bytes(c5) == 32 * 128 * 16384 * 2 + 16384 * 128 * 2 + 32 * 128 * 128 * 4
    c4 = W.WORKLOADS["c4"]
    assert acc.problem_bytes(c4) == (4095 * 1000 + 1000 * 4097 + 4095 * 4097 + 4097) * 2


def test_mi355x_peaks():
    assert acc.PEAK_BF16_MFMA == pytest.approx(256 * 4096 * 2.4e9, rel=1e-4)
    assert acc.PEAK_F32 == pytest.approx(256 * 256 * 2.4e9, rel=1e-3)
    # the vector-FMA peak from unit counts and clock is the published fp32 figure
    assert acc.PEAK_F32_VALU == pytest.approx(acc.PEAK_F32, rel=1e-3)
    assert acc.PEAK_F64_VALU == pytest.approx(78.6e12, rel=1e-3)
