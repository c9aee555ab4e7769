"""GPU edge cases against the oracle: ragged M / N / K around every tile
size, all operand orders, padded leading dimensions, batches with and
without a broadcast operand, split-K, every epilogue, forced kernel
families; guard bands around C; NaN semantics of alpha = 0 / beta = 0;
K = 0; bf16 tie rounding; run-to-run determinism."""
import itertools

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


DIMS = [1, 2, 3, 7, 8, 9, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 255, 257]
COMBOS = [(W.F32, W.F32), (W.BF16, W.BF16), (W.BF16, W.F32)]
ALPHA_BETA = [(1.0, 0.0), (1.5, 0.5), (-0.75, 2.0)]
ACTS = [W.ACT_NONE, W.ACT_GELU_ERF, W.ACT_GELU_TANH]
ALGOS = [0, 0, 0, dg.DG_ALGO_GENERIC]


def _ld(order, rows, cols, pad):
    return (cols if order == W.ROW else rows) + pad


def _make_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M, N, K = (int(v) for v in rng.choice(DIMS, 3))
        ta, tc = COMBOS[i % 3]
        ao, bo, co = (W.ROW if v else W.COL for v in rng.integers(0, 2, 3))
        if i % 4 == 1:          # the bf16 matrix-core layout
            ao, bo = W.ROW, W.COL
        pad = int(rng.choice([0, 0, 8, 1, 3]))
        batch = int(rng.choice([1, 1, 3]))
        bcast = rng.choice(["none", "a", "b"]) if batch > 1 else "none"
        split = int(rng.choice([0, 1, 2, 3]))
        alpha, beta = ALPHA_BETA[int(rng.integers(0, 3))]
        act = ACTS[int(rng.integers(0, 3))]
        has_bias = bool(rng.integers(0, 2))
        kw = {}
        if bcast == "a":
            kw["stride_a"] = 0
        if bcast == "b":
            kw["stride_b"] = 0
        p = W.Problem(name=f"edge{i}", M=M, N=N, K=K, batch=batch, a_type=ta, b_type=ta,
                      c_type=tc, a_order=ao, b_order=bo, c_order=co,
                      lda=_ld(ao, M, K, pad), ldb=_ld(bo, K, N, pad), ldc=_ld(co, M, N, pad),
                      alpha=alpha, beta=beta, has_bias=has_bias, bias_type=ta, act=act,
                      split_k=split, seed=1000 + i, **kw)
        algo = ALGOS[i % 4]
        if (ta == W.F32 and i % 4 == 2 and p.lda_ % 4 == 0 and p.ldb_ % 4 == 0 and
                p.stride_a_ % 4 == 0 and p.stride_b_ % 4 == 0):
            algo = dg.DG_ALGO_VALU_F32        # the vector-FMA kernel, where it applies
        cases.append((p, algo))
    return cases


CASES = _make_cases(96, seed=20261202)


def _run(p, x, **kw):
    from workloads.device import DeviceProblem
    dp = DeviceProblem(p, x, **kw)
    dp.run()
    return dp, dp.result()


@pytest.mark.parametrize("p,algo", CASES, ids=[c[0].name for c in CASES])
def test_edge_sweep(p, algo):
    small_int = p.act == W.ACT_NONE
    x = W.make_inputs(p, small_int=small_int, fill=float("nan"))
    dp, got = _run(p, x, algo=algo)
    print(f"{p} -> {dp.describe()}", flush=True)
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, got, ref, mag, out, exact=small_int, what=p.name)
    # guard band: no position of C outside the logical matrices changed
    covered = np.zeros(got.size, bool)
    r = np.arange(p.M)[:, None]
    c = np.arange(p.N)[None, :]
    off = (r * p.ldc_ + c) if p.c_order == W.ROW else (c * p.ldc_ + r)
    for b in range(p.batch):
        covered[b * p.stride_c_ + off] = True
    assert got[~covered].tobytes() == x.C[~covered].tobytes()


@pytest.mark.parametrize("ta,tc", COMBOS)
@pytest.mark.parametrize("algo", [0, dg.DG_ALGO_GENERIC])
def test_beta_zero_never_reads_c(ta, tc, algo):
    p = W.Problem(name="b0", M=130, N=70, K=40, a_type=ta, b_type=ta, c_type=tc,
                  a_order=W.ROW, b_order=W.COL, alpha=1.0, beta=0.0, seed=3)
    x = W.make_inputs(p, small_int=True, c_fill=float("nan"))
    _, got = _run(p, x, algo=algo)
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, got, ref, mag, out, exact=True, what="beta=0")
    assert not np.isnan(ref).any()


@pytest.mark.parametrize("ta,tc", COMBOS)
def test_alpha_zero_never_reads_a_b(ta, tc):
    p = W.Problem(name="a0", M=65, N=33, K=200, a_type=ta, b_type=ta, c_type=tc,
                  a_order=W.ROW, b_order=W.COL, alpha=0.0, beta=0.5, has_bias=True,
                  bias_type=ta, seed=4)
    x = W.make_inputs(p, small_int=True)
    x.A[:] = W.to_storage(np.full(x.A.size, np.nan, np.float32), ta)
    x.B[:] = W.to_storage(np.full(x.B.size, np.nan, np.float32), ta)
    _, got = _run(p, x)
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, got, ref, mag, out, exact=True, what="alpha=0")


def test_k_zero_applies_epilogue_only():
    p = W.Problem(name="k0", M=40, N=50, K=0, alpha=1.0, beta=2.0, has_bias=True,
                  act=W.ACT_GELU_ERF, lda=1, ldb=50, seed=5)
    x = W.make_inputs(p)
    _, got = _run(p, x)
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, got, ref, mag, out, what="K=0")


@pytest.mark.parametrize("algo", [0, dg.DG_ALGO_GENERIC])
def test_bf16_output_ties_round_to_even(algo):
    # row 0 of A . column 0 of B = 1 + 2^-8, exactly halfway between bf16 1.0
    # and 1 + 2^-7: must round to 1.0 (even); 1 + 3*2^-8 must round up.
    M, N, K = 2, 1, 64
    p = W.Problem(name="tie", M=M, N=N, K=K, a_type=W.BF16, b_type=W.BF16, c_type=W.BF16,
                  a_order=W.ROW, b_order=W.COL, alpha=1.0, beta=0.0)
    A_log = np.zeros((1, M, K), np.float32)
    A_log[0, 0, :2] = [1.0, 2 ** -8]
    A_log[0, 1, :2] = [1.0, 3 * 2 ** -8]
    B_log = np.zeros((1, K, N), np.float32)
    B_log[0, :2, 0] = 1.0
    x = W.make_inputs(p)
    x.A[:] = W.lay_out(W.to_storage(A_log, W.BF16), p.a_order, p.lda_, p.stride_a_,
                       p.buffer_elems("a"), W.BF16)
    x.B[:] = W.lay_out(W.to_storage(B_log, W.BF16), p.b_order, p.ldb_, p.stride_b_,
                       p.buffer_elems("b"), W.BF16)
    _, got = _run(p, x, algo=algo)
    assert got[0] == 0x3F80 and got[1] == 0x3F82


@pytest.mark.parametrize("act", [W.ACT_GELU_ERF, W.ACT_GELU_TANH])
@pytest.mark.parametrize("algo", [0, dg.DG_ALGO_GENERIC])
def test_gelu_accuracy_on_a_dense_grid(act, algo):
    # K = 1, B = 1: output (m, n) is act(x_m) of one exact fp32 value x_m,
    # x on a dense grid of [-12, 12].  The erf form is held to the stated
    # bound of its approximation of erfc (1.5e-7 absolute) scaled by |x|, the
    # tanh form to the same bound, both with room for a few fp32 roundings.
    M, N = 4096, 8
    p = W.Problem(name="gelu", M=M, N=N, K=1, a_type=W.F32, b_type=W.F32, c_type=W.F32,
                  alpha=1.0, beta=0.0, act=act)
    xs = np.linspace(-12.0, 12.0, M).astype(np.float32)
    x = W.make_inputs(p)
    x.A[:] = W.lay_out(xs.reshape(1, M, 1), p.a_order, p.lda_, p.stride_a_,
                       p.buffer_elems("a"), W.F32)
    x.B[:] = W.lay_out(np.ones((1, 1, N), np.float32), p.b_order, p.ldb_, p.stride_b_,
                       p.buffer_elems("b"), W.F32)
    _, got = _run(p, x, algo=algo)
    got = got[:M * p.ldc_].reshape(M, p.ldc_)[:, :N].astype(np.float64)
    ref = np.array([oracle.act(float(v), act) for v in xs])
    err = np.abs(got - ref[:, None]) / np.maximum(1.0, np.abs(xs.astype(np.float64)))[:, None]
    assert err.max() <= 4e-7, (err.max(), xs[int(np.argmax(err.max(axis=1)))])


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_run_to_run_bitwise_determinism(name):
    from workloads.device import DeviceProblem
    p = W.WORKLOADS[name]
    if name == "c3":
        p = p.replace(M=1024, N=1024, K=2048)
    x = W.make_inputs(p)
    dp = DeviceProblem(p, x)
    dp.run()
    first = dp.result().copy()
    for _ in range(3):
        dp.reset_c()
        dp.run()
        assert np.array_equal(dp.result().view(np.uint8), first.view(np.uint8))


@pytest.mark.parametrize("ta", [W.F32, W.BF16])
def test_long_k_accumulates_in_fp32(ta):
    # |acc| <= 4K = 32768 < 2^24: exact only with an fp32 accumulator
    p = W.Problem(name="longk", M=64, N=64, K=8192, a_type=ta, b_type=ta, c_type=W.F32,
                  a_order=W.ROW, b_order=W.COL, seed=9)
    x = W.make_inputs(p, small_int=True)
    _, got = _run(p, x)
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, got, ref, mag, out, exact=True, what="long K")


@pytest.mark.parametrize("group_m,xcd", list(itertools.product([1, 4, 8, 16], [0, -1])))
def test_tile_order_knobs_do_not_change_results(group_m, xcd):
    p = W.WORKLOADS["c3"].replace(M=1024 + 64, N=1024 + 96, K=256)
    x = W.make_inputs(p, small_int=True)
    _, got = _run(p, x, group_m=group_m, xcd_remap=xcd)
    pts = W.sample_points(p, 2000)
    ref, mag, out = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
    check(p, got, ref, mag, out, pts=pts, exact=True, what=f"G={group_m} xcd={xcd}")
