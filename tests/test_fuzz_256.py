"""Seeded randomised GPU parity of the 256 x 256 16-bit tile (16 x 16 x 32
MFMA blocks) against the CPU oracle.

The tile is forced on every case (the planner keeps the few with an M- or
N-contiguous operand and K <= 64 on the 128 x 128 tile), so that random
shapes a few tiles wide
(ragged in M, N and K) reach it with every operand order (K-contiguous
staging and the transposing reads of M- or N-contiguous operands), either
output order, a batch with broadcast operands, alpha, beta, bias and
activation, and the data-parallel, split-K and stream-K schedules.  Every
output is checked against the oracle (bit for bit on small-integer inputs
without an activation)."""
import numpy as np
import pytest

import dense_gemm_10_amd as dg
import oracle
import workloads as W
from parity_util import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

N_CASES = 48


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i):
    rng = np.random.default_rng([256, i])
    pick = lambda xs: xs[int(rng.integers(len(xs)))]  # noqa: E731
    ab = pick([W.BF16, W.F16])
    M, N = int(rng.integers(200, 700)), int(rng.integers(200, 700))
    K = int(rng.integers(1, 600))
    a_order, b_order = pick([W.ROW, W.COL]), pick([W.ROW, W.COL])
    c_order = W.COL if rng.random() < 0.2 else W.ROW
    # leading dimensions a multiple of 8 elements (the tiled kernel's
    # alignment), sometimes padded
    ld = lambda natural: -(-natural // 8) * 8 + pick([0, 0, 8, 24])  # noqa: E731
    kw = dict(lda=ld(K if a_order == W.ROW else M), ldb=ld(N if b_order == W.ROW else K),
              ldc=(N if c_order == W.ROW else M) + pick([0, 0, 3]))
    batch = pick([1, 1, 2])
    if batch > 1:
        # batch strides of whole padded matrices (multiples of 8 elements,
        # as the tiled kernel requires), or 0 to broadcast
        kw["stride_a"] = 0 if rng.random() < 0.3 else (M if a_order == W.ROW else K) * kw["lda"]
        kw["stride_b"] = 0 if rng.random() < 0.3 else (K if b_order == W.ROW else N) * kw["ldb"]
    alpha = pick([1.0, 1.0, 1.5, -0.5])
    beta = pick([0.0, 0.0, 0.5])
    act = pick([W.ACT_NONE, W.ACT_NONE, W.ACT_GELU_ERF, W.ACT_GELU_TANH])
    split_k = pick([0, 0, 0, 2, 3]) if batch == 1 else 0
    schedule = 2 if split_k == 0 and batch == 1 and rng.random() < 0.4 else 0
    p = W.Problem(name=f"fuzz256_{i}", M=M, N=N, K=K, batch=batch, a_type=ab, b_type=ab,
                  c_type=pick([W.F32, ab]), a_order=a_order, b_order=b_order, c_order=c_order,
                  alpha=alpha, beta=beta, has_bias=bool(rng.random() < 0.5),
                  bias_type=pick([W.F32, ab]), act=act, split_k=split_k, seed=5000 + i, **kw)
    return p, schedule, bool(rng.random() < 0.5)


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_256(i, monkeypatch):
    from workloads.device import DeviceProblem
    p, schedule, small_int = _case(i)
    tile = f"mfma_{'bf16' if p.a_type == W.BF16 else 'f16'}_256x256x64_w2x2_s2"
    monkeypatch.setenv("DG_FORCE_TILE", tile)
    d = dg.make_desc(**dict(W.desc_fields(p), schedule=schedule))
    try:
        dg.dg_gemm_describe(d, 1 << 34)
    except dg.DgError as e:
        # stream-K only where the plan allows it
        assert schedule == 2 and e.status == dg.DG_ERROR_NOT_SUPPORTED
        schedule = 0
    x = W.make_inputs(p, small_int=small_int)
    dp = DeviceProblem(p, x, schedule=schedule)
    text = dp.describe()
    print(f"[{p.name}] {p} sched={schedule} int={small_int}: {text}", flush=True)
    # (with an M- or N-contiguous operand the planner keeps K <= 64 on the
    # 128 x 128 tile; such a case still checks that tile)
    if (p.a_order == W.ROW and p.b_order == W.COL) or p.K > 64:
        assert f"tile={tile} " in text
    dp.run()
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, dp.result(), ref, mag, out, exact=small_int and p.act == W.ACT_NONE,
          what=f"{p.name} sched={schedule} int={small_int}")
