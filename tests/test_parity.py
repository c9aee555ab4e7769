"""GPU parity of the five workloads against the CPU oracle, through the C
ABI, in the launch configuration the benchmark times (the library's own
plan for each descriptor).

Small configurations are checked on every output; the 4096-class ones on
every output of a reduced twin that keeps the layout, dtype, epilogue and
ragged edges, and on seeded sampled outputs (corners included) at full
size.  Every configuration also runs with small-integer inputs, where the
GPU must equal the oracle exactly (activation NONE; with GELU the
tolerance applies because a transcendental cannot be bit-exact across
implementations)."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import check

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(p, x, **kw):
    from workloads.device import DeviceProblem
    dp = DeviceProblem(p, x, **kw)
    print(f"[{p.name}] {dp.describe()}", flush=True)
    dp.run()
    return dp.result()


def _full(p, small_int=False, **kw):
    x = W.make_inputs(p, small_int=small_int)
    got = _run(p, x, **kw)
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    exact = small_int and p.act == W.ACT_NONE
    check(p, got, ref, mag, out, exact=exact, what=f"{p.name} int={small_int}")


def _sampled(p, n=3000, small_int=False, **kw):
    x = W.make_inputs(p, small_int=small_int)
    got = _run(p, x, **kw)
    pts = W.sample_points(p, n)
    ref, mag, out = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
    exact = small_int and p.act == W.ACT_NONE
    check(p, got, ref, mag, out, pts=pts, exact=exact, what=f"{p.name} sampled int={small_int}")


# --- C1: fp32 256^3, alpha 1.5, beta 0.5 -------------------------------------
@pytest.mark.parametrize("small_int", [False, True])
def test_c1_sgemm_256(small_int):
    _full(W.WORKLOADS["c1"], small_int)


@pytest.mark.parametrize("small_int", [False, True])
def test_c1_sgemm_256_valu(small_int):
    import dense_gemm_10_amd as dg
    _full(W.WORKLOADS["c1"], small_int, algo=dg.DG_ALGO_VALU_F32)


# --- C2: fp32 4096^3 -----------------------------------------------------------
def test_c2_sgemm_4096_sampled():
    _sampled(W.WORKLOADS["c2"])


def test_c2_sgemm_4096_sampled_int():
    _sampled(W.WORKLOADS["c2"], n=1000, small_int=True)


def test_c2_sgemm_4096_sampled_valu():
    import dense_gemm_10_amd as dg
    _sampled(W.WORKLOADS["c2"], algo=dg.DG_ALGO_VALU_F32)


@pytest.mark.parametrize("small_int", [False, True])
@pytest.mark.parametrize("algo", [0, 2])        # automatic (matrix cores), vector FMA
def test_c2_reduced_twin_ragged(small_int, algo):
    # ragged sizes, leading dimensions padded to multiples of 4 (both fp32
    # kernels need 16-byte rows)
    p = W.WORKLOADS["c2"].replace(name="sgemm_f32_ragged", M=515, N=389, K=301,
                                  lda=304, ldb=392, ldc=396)
    _full(p, small_int, algo=algo)


# --- C3: bf16 4096^3, A row, B col, bf16 out -------------------------------------
def test_c3_bf16_4096_sampled():
    _sampled(W.WORKLOADS["c3"])


def test_c3_bf16_4096_sampled_int():
    _sampled(W.WORKLOADS["c3"], n=1000, small_int=True)


@pytest.mark.parametrize("small_int", [False, True])
def test_c3_reduced_twin(small_int):
    p = W.WORKLOADS["c3"].replace(name="gemm_bf16_reduced", M=768, N=512, K=640)
    _full(p, small_int)


# --- C4: ragged bf16 with bias + GELU ----------------------------------------------
def test_c4_edges_gelu_sampled():
    _sampled(W.WORKLOADS["c4"], n=4000)


def test_c4_edges_gelu_sampled_int():
    _sampled(W.WORKLOADS["c4"], n=1000, small_int=True)


@pytest.mark.parametrize("small_int", [False, True])
def test_c4_reduced_twin(small_int):
    p = W.WORKLOADS["c4"].replace(name="gemm_bf16_ragged_gelu", M=511, N=517, K=1000)
    _full(p, small_int)


def test_c4_no_activation_int_exact():
    p = W.WORKLOADS["c4"].replace(name="gemm_bf16_ragged_bias", M=511, N=517, K=1000,
                                  act=W.ACT_NONE)
    _full(p, small_int=True)


# --- C5: batched, B broadcast, split-K, fp32 out -------------------------------------
@pytest.mark.parametrize("small_int", [False, True])
def test_c5_batched_splitk(small_int):
    _full(W.WORKLOADS["c5"], small_int)



# --- further shapes: flat K = 16 (HBM-bound) and a long-K ragged grid --------------
@pytest.mark.parametrize("name", ["flat16", "flat16_f32"])
@pytest.mark.parametrize("small_int", [False, True])
def test_flat_small_k(name, small_int):
    _full(W.WORKLOADS[name], small_int)


@pytest.mark.parametrize("small_int", [False, True])
def test_tail4352_sampled(small_int):
    _sampled(W.WORKLOADS["tail4352"], n=2000, small_int=small_int)
