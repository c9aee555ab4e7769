"""Seeded randomised GPU parity against the CPU oracle.

Each case draws dtypes (fp32, bf16, fp16 inputs; fp32 or the input type
out), operand orders, padded or misaligned leading dimensions, a batch
with broadcast operands, alpha, beta, bias and activation, and sometimes a
split-K count or the stream-K schedule, then checks every output against
the oracle (bit for bit on small-integer inputs without an activation).
The mix sends cases through every kernel family and every epilogue path:
whole aligned tiles, whole tiles with misaligned rows, edge tiles, partial
K tiles, split-K partials and stream-K fix-ups."""
import numpy as np
import pytest

import dense_gemm_10_amd as dg
import oracle
import workloads as W
from parity_util import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

N_CASES = 200


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i):
    rng = np.random.default_rng([2024, i])
    pick = lambda xs: xs[int(rng.integers(len(xs)))]  # noqa: E731
    ab = pick([W.F32, W.BF16, W.F16])
    M, N, K = (int(rng.integers(1, 420)), int(rng.integers(1, 420)), int(rng.integers(1, 520)))
    if ab != W.F32 and rng.random() < 0.7:
        a_order, b_order = W.ROW, W.COL           # the 16-bit matrix-core layout
    else:
        a_order, b_order = pick([W.ROW, W.COL]), pick([W.ROW, W.COL])
    c_order = W.COL if rng.random() < 0.15 else W.ROW
    # leading dimensions: mostly rounded up to the tiled kernels' 16-byte
    # alignment (8 16-bit or 4 fp32 elements), sometimes padded to an odd
    # size (the generic kernel)
    q = 4 if ab == W.F32 else 8
    aligned = rng.random() < 0.75

    def ld(natural):
        if aligned:
            return -(-natural // q) * q + pick([0, 0, q])
        return natural + pick([0, 3])
    lda = ld(K if a_order == W.ROW else M)
    ldb = ld(N if b_order == W.ROW else K)
    ldc = (N if c_order == W.ROW else M) + pick([0, 0, 5])
    batch = pick([1, 1, 1, 2, 3])
    kw = dict(lda=lda, ldb=ldb, ldc=ldc)
    if batch > 1:
        if rng.random() < 0.25:
            kw["stride_a"] = 0
        if rng.random() < 0.25:
            kw["stride_b"] = 0
    alpha = pick([1.0, 1.0, 1.5, -0.5, 0.0])
    beta = pick([0.0, 0.0, 0.5, -1.0])
    has_bias = rng.random() < 0.5
    act = pick([W.ACT_NONE, W.ACT_NONE, W.ACT_GELU_ERF, W.ACT_GELU_TANH])
    split_k = pick([0, 0, 0, 0, 2, 3, 5]) if alpha != 0.0 else 0
    mfma16_layout = ab != W.F32 and a_order == W.ROW and b_order == W.COL and aligned
    schedule = 2 if (mfma16_layout and split_k == 0 and batch == 1 and rng.random() < 0.5) else 0
    p = W.Problem(name=f"fuzz{i}", M=M, N=N, K=K, batch=batch, a_type=ab, b_type=ab,
                  c_type=pick([W.F32, ab]), a_order=a_order, b_order=b_order, c_order=c_order,
                  alpha=alpha, beta=beta, has_bias=has_bias, bias_type=pick([W.F32, ab]),
                  act=act, split_k=split_k, seed=1000 + i, **kw)
    return p, schedule, bool(rng.random() < 0.5)


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz(i):
    from workloads.device import DeviceProblem
    p, schedule, small_int = _case(i)
    d = dg.make_desc(**dict(W.desc_fields(p), schedule=schedule))
    try:
        dg.dg_gemm_describe(d, 1 << 34)
    except dg.DgError as e:
        # stream-K only where the plan allows it
        assert schedule == 2 and e.status == dg.DG_ERROR_NOT_SUPPORTED
        schedule = 0
    x = W.make_inputs(p, small_int=small_int)
    dp = DeviceProblem(p, x, schedule=schedule)
    print(f"[{p.name}] {p} sched={schedule} int={small_int}: {dp.describe()}", flush=True)
    dp.run()
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, dp.result(), ref, mag, out, exact=small_int and p.act == W.ACT_NONE,
          what=f"{p.name} sched={schedule} int={small_int}")
