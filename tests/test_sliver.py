"""GPU parity of the sliver split: when N is a few columns past a whole
number of tile columns, the library runs its tiled plan on the full tile
columns and a one-wavefront-per-row kernel on the last columns.

Every output of the sliver columns is checked against the CPU oracle, with
a seeded sample of the tiled part (the problems are large enough for the
split to apply: at least one tile per compute unit).  On small-integer
inputs every result is exact in fp32, so the split plan must equal the
single tiled plan (forced data-parallel, which never splits) bit for bit."""
import numpy as np
import pytest

import dense_gemm_10_amd as dg
import oracle
import workloads as W
from parity_util import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sliver(text):
    return int(dict(t.split("=", 1) for t in text.split() if "=" in t)["sliver"])


def _points(p, nrem, n=3000):
    """Every output of the last nrem columns, plus a seeded sample."""
    b, i, j = np.meshgrid(np.arange(p.batch), np.arange(p.M), np.arange(p.N - nrem, p.N),
                          indexing="ij")
    sb, si, sj = W.sample_points(p, n)
    return (np.concatenate([b.ravel(), sb]).astype(np.int64),
            np.concatenate([i.ravel(), si]).astype(np.int64),
            np.concatenate([j.ravel(), sj]).astype(np.int64))


CASES = [
    # bf16, bf16 output, every epilogue term, erf GELU
    W.Problem(name="sliver_bf16_gelu", M=4096, N=4096 + 5, K=256, a_type=W.BF16, b_type=W.BF16,
              c_type=W.BF16, a_order=W.ROW, b_order=W.COL, alpha=1.5, beta=0.5, has_bias=True,
              bias_type=W.BF16, act=W.ACT_GELU_ERF, seed=91),
    # fp32 on the fp32 matrix-core kernel, row-major B, tanh GELU
    W.Problem(name="sliver_f32", M=4096, N=4096 + 2, K=128, a_type=W.F32, b_type=W.F32,
              c_type=W.F32, a_order=W.ROW, b_order=W.ROW, ldb=4100, alpha=0.75, beta=-1.0,
              has_bias=True, bias_type=W.F32, act=W.ACT_GELU_TANH, seed=92),
    # fp16, batched with B broadcast (stride 0), fp16 output
    W.Problem(name="sliver_f16_batch", M=2048, N=2048 + 7, K=128, batch=4, a_type=W.F16,
              b_type=W.F16, c_type=W.F16, a_order=W.ROW, b_order=W.COL, stride_b=0,
              alpha=1.0, beta=0.25, seed=93),
    # column-major fp32 output, one sliver column, K = 100 (not a multiple of
    # the 8 elements of a 16-byte load; padded leading dimensions keep A's
    # rows and B's columns 16-byte aligned)
    W.Problem(name="sliver_colmajor_c", M=4096, N=4096 + 1, K=100, lda=112, ldb=104,
              a_type=W.BF16, b_type=W.BF16, c_type=W.F32, a_order=W.ROW, b_order=W.COL,
              c_order=W.COL, alpha=1.0, beta=0.0, seed=94),
    # one column behind a data-parallel 16-bit plan runs inside the tiled
    # kernel (workgroups after its tiles, batch entry from the program id):
    # batched with B broadcast, and a row-major bf16 output with GELU
    W.Problem(name="sliver_inside_f16_batch", M=2048, N=2048 + 1, K=128, batch=4, a_type=W.F16,
              b_type=W.F16, c_type=W.F16, a_order=W.ROW, b_order=W.COL, stride_b=0,
              alpha=1.0, beta=0.25, has_bias=True, bias_type=W.F16, seed=95),
    W.Problem(name="sliver_inside_bf16_gelu", M=4096, N=4096 + 1, K=200, a_type=W.BF16,
              b_type=W.BF16, c_type=W.BF16, a_order=W.ROW, b_order=W.COL, has_bias=True,
              bias_type=W.BF16, act=W.ACT_GELU_ERF, seed=96),
]


@pytest.mark.parametrize("p", CASES, ids=[c.name for c in CASES])
@pytest.mark.parametrize("small_int", [True, False])
def test_sliver_against_oracle(p, small_int):
    from workloads.device import DeviceProblem
    x = W.make_inputs(p, small_int=small_int)
    dp = DeviceProblem(p, x)
    text = dp.describe()
    print(f"[{p.name}] {text}", flush=True)
    nrem = _sliver(text)
    assert 0 < nrem <= 8 and (p.N - nrem) % int(dict(
        t.split("=", 1) for t in text.split() if "=" in t)["bn"]) == 0
    dp.run()
    pts = _points(p, nrem)
    ref, mag, out = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
    check(p, dp.result(), ref, mag, out, pts=pts, exact=small_int and p.act == W.ACT_NONE,
          what=f"{p.name} int={small_int}")


@pytest.mark.parametrize("p", CASES, ids=[c.name for c in CASES])
def test_sliver_matches_single_plan_bitwise(p):
    from workloads.device import DeviceProblem
    p = p.replace(act=W.ACT_NONE)
    x = W.make_inputs(p, small_int=True)
    split = DeviceProblem(p, x)
    single = DeviceProblem(p, x, schedule=dg.DG_SCHED_DATA_PARALLEL)
    assert _sliver(split.describe()) > 0 and _sliver(single.describe()) == 0
    split.run()
    single.run()
    assert np.array_equal(split.result().view(np.uint8), single.result().view(np.uint8))
