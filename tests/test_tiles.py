"""GPU parity of every tile configuration of every matrix-core family (the
candidates the offline tuning sweep may put in the planner's table), under
the data-parallel and the stream-K schedule, on ragged shapes with a
partial last K tile, against the CPU oracle."""
import pytest

import dense_gemm_10_amd as dg
import oracle
import workloads as W
from dense_gemm_10_amd.tune import TILES
from parity_util import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _problem(family, epilogue):
    """`epilogue`: "plain" (alpha 1, beta 0); "ragged" (alpha, beta * C, bias
    and GELU with N = 387, so no output row starts on a 16-byte boundary:
    the general row path); "aligned" and "aligned_gelu" (the same terms
    with N = 392 and the family's own output type: interior tiles take the
    whole-tile path, edge tiles the general one)."""
    dt = {"mfma_bf16": W.BF16, "mfma_f16": W.F16, "mfma_f32": W.F32}[family]
    if dt == W.F32:
        base = dict(M=520, N=392, K=300, a_type=dt, b_type=dt, c_type=W.F32)
    else:
        base = dict(M=520, N=392, K=1000, a_type=dt, b_type=dt, a_order=W.ROW, b_order=W.COL,
                    c_type=dt)
    terms = dict(alpha=1.5, beta=0.5, has_bias=True, bias_type=dt)
    if epilogue == "ragged":
        base.update(terms, c_type=W.F32, act=W.ACT_GELU_ERF, N=392 - 5)
        if dt == W.F32:
            base.update(ldb=392)     # row-major B: the fp32 kernels need ldb % 4 == 0
    elif epilogue == "aligned":
        base.update(terms)
    elif epilogue == "aligned_gelu":
        base.update(terms, act=W.ACT_GELU_TANH)
    return W.Problem(name=f"{family}_{epilogue}", seed=61, **base)


CASES = [(f, t, s) for f, tiles in TILES.items() for t in tiles for s in (1, 2)]


@pytest.mark.parametrize("family,tile,schedule", CASES,
                         ids=[f"{t}-{'dp' if s == 1 else 'sk'}" for _, t, s in CASES])
@pytest.mark.parametrize("epilogue", ["plain", "ragged", "aligned", "aligned_gelu"])
def test_every_tile(family, tile, schedule, epilogue, monkeypatch):
    from workloads.device import DeviceProblem
    monkeypatch.setenv("DG_FORCE_TILE", tile)
    p = _problem(family, epilogue)
    d = dg.make_desc(**dict(W.desc_fields(p), schedule=schedule))
    try:
        dg.dg_gemm_describe(d, 1 << 34)
    except dg.DgError as e:
        assert schedule == 2 and e.status == dg.DG_ERROR_NOT_SUPPORTED   # fp32: no stream-K
        pytest.skip("stream-K does not apply to this family")
    for small_int in (True, False):
        x = W.make_inputs(p, small_int=small_int)
        dp = DeviceProblem(p, x, schedule=schedule)
        text = dp.describe()
        print(f"[{p.name}] {text}", flush=True)
        assert f"tile={tile} " in text
        assert ("schedule=stream_k" in text) == (schedule == 2)
        dp.run()
        ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
        check(p, dp.result(), ref, mag, out, exact=small_int and p.act == W.ACT_NONE,
              what=f"{tile} sched={schedule} int={small_int}")


VALU_TILES = ["valu_f32_128x128x16_t8x8", "valu_f32_128x256x16_t8x16"]
ORDERS = [(W.ROW, W.ROW), (W.ROW, W.COL), (W.COL, W.ROW), (W.COL, W.COL)]


@pytest.mark.parametrize("tile", VALU_TILES)
@pytest.mark.parametrize("orders", ORDERS, ids=[f"{a}{b}" for a, b in ORDERS])
@pytest.mark.parametrize("epilogue", ["plain", "ragged"])
def test_every_valu_tile(tile, orders, epilogue, monkeypatch):
    """Both thread tiles of the vector-FMA SGEMM, every operand order, on a
    ragged grid (M = 520 and N = 600 cut the 128-row and 256-column blocks)
    with K = 300 (a partial last K tile), checked in full."""
    from workloads.device import DeviceProblem
    monkeypatch.setenv("DG_FORCE_TILE", tile)
    a_order, b_order = orders
    base = dict(M=520, N=600, K=300, a_order=a_order, b_order=b_order, lda=None, ldb=None)
    # the vector kernel reads 16-byte pieces: leading dimensions a multiple of 4
    base["lda"] = 300 if a_order == W.ROW else 520
    base["ldb"] = 600 if b_order == W.ROW else 300
    if epilogue == "ragged":
        base.update(alpha=1.5, beta=0.5, has_bias=True, act=W.ACT_GELU_ERF)
    p = W.Problem(name=f"valu_{epilogue}", seed=62, **base)
    for small_int in (True, False):
        x = W.make_inputs(p, small_int=small_int)
        dp = DeviceProblem(p, x, algo=dg.DG_ALGO_VALU_F32)
        text = dp.describe()
        print(f"[{p.name}] {text}", flush=True)
        assert f"tile={tile} " in text
        dp.run()
        ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
        check(p, dp.result(), ref, mag, out, exact=small_int and p.act == W.ACT_NONE,
              what=f"{tile} {a_order}{b_order} int={small_int}")


RAGGED_K = [5, 13, 29, 1001]
RAGGED_TILES = ["128x128x32_w2x2_s4", "256x256x64_w2x2_s2", "128x256x32_w2x2_s3"]


@pytest.mark.parametrize("K", RAGGED_K)
@pytest.mark.parametrize("tile", RAGGED_TILES)
@pytest.mark.parametrize("dt", [W.BF16, W.F16])
@pytest.mark.parametrize("schedule", [1, 2])
def test_ragged_k_tail(K, tile, dt, schedule, monkeypatch):
    """K not a multiple of 8 with leading dimensions padded to 8: the 16-bit
    kernels' register-loaded K tail takes its element path for the chunk
    that straddles K (a K multiple of 8 takes the clamped vector path,
    covered by the other tile tests).  Checked in full against the oracle."""
    from workloads.device import DeviceProblem
    fam = "bf16" if dt == W.BF16 else "f16"
    name = f"mfma_{fam}_{tile}"
    monkeypatch.setenv("DG_FORCE_TILE", name)
    up8 = (K + 7) // 8 * 8
    p = W.Problem(name=f"raggedk{K}", M=300, N=520, K=K, a_type=dt, b_type=dt, c_type=W.F32,
                  a_order=W.ROW, b_order=W.COL, lda=up8, ldb=up8, alpha=1.25, beta=0.5,
                  has_bias=True, bias_type=dt, seed=63)
    d = dg.make_desc(**dict(W.desc_fields(p), schedule=schedule))
    try:
        dg.dg_gemm_describe(d, 1 << 34)
    except dg.DgError:
        pytest.skip("no stream-K tail for this shape")
    for small_int in (True, False):
        x = W.make_inputs(p, small_int=small_int)
        dp = DeviceProblem(p, x, schedule=schedule)
        text = dp.describe()
        print(f"[{p.name}] {text}", flush=True)
        assert f"tile={name} " in text
        dp.run()
        ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
        check(p, dp.result(), ref, mag, out, exact=small_int,
              what=f"{name} K={K} sched={schedule} int={small_int}")
