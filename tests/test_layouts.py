"""GPU parity of the 16-bit matrix-core kernel on every order of A and B
("Skill: Write a Triton GEMM Kernel", Inputs the agent should gather first,
item 3: row- or column-major operands).  A column-major A or row-major B
is staged with its M (N) dimension contiguous and transposed by the LDS
reads; these cases cover both tiles it runs on, ragged M, N and K (edges
that cut a 16-byte chunk, a partial last K tile), split-K, stream-K, a
batch with a broadcast operand and every epilogue term, against the CPU
oracle on every output (bit for bit on small-integer inputs)."""
import itertools

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


LAYOUTS = [(W.ROW, W.ROW), (W.COL, W.COL), (W.COL, W.ROW), (W.ROW, W.COL)]


def _run(p, small_int, **kw):
    from workloads.device import DeviceProblem
    x = W.make_inputs(p, small_int=small_int)
    dp = DeviceProblem(p, x, **kw)
    text = dp.describe()
    print(f"[{p.name}] {text}", flush=True)
    dp.run()
    got = dp.result()
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, got, ref, mag, out, exact=small_int and p.act == W.ACT_NONE,
          what=f"{p.name} int={small_int}")
    return text


def _padded(ao, bo, M, N, K):
    """The shape with leading dimensions rounded up to a multiple of 8
    elements (16 bytes), as the matrix-core kernel needs, so that ragged M
    and N stay ragged."""
    up8 = lambda v: -(-v // 8) * 8     # noqa: E731
    return dict(M=M, N=N, K=K, lda=up8(K if ao == W.ROW else M), ldb=up8(N if bo == W.ROW else K))


# shape, expected tile, description
SHAPES = [
    (dict(M=300, N=260, K=200), "128x128", "ragged M and N (edge cuts a chunk), partial K tile"),
    (dict(M=520, N=392, K=1000), "128x128", "several tiles, partial K tile"),
    (dict(M=1030, N=1027, K=256), "256x256", "the large tile, ragged edges, whole K tiles"),
    (dict(M=1024, N=1024, K=320), "256x256", "the large tile, no ragged edge"),
]


@pytest.mark.parametrize("shape,tile,what", SHAPES, ids=[s[2] for s in SHAPES])
@pytest.mark.parametrize("ao,bo", LAYOUTS, ids=[f"A{a}_B{b}" for a, b in LAYOUTS])
@pytest.mark.parametrize("dt", [W.BF16, W.F16])
def test_layout_parity(dt, ao, bo, shape, tile, what, monkeypatch):
    if tile == "256x256":
        # the large tile on a grid below a wave: force it (the planner
        # would pick 128 x 128 there)
        fam = "mfma_bf16" if dt == W.BF16 else "mfma_f16"
        monkeypatch.setenv("DG_FORCE_TILE", f"{fam}_256x256x64_w2x2_s2")
    p = W.Problem(name=f"layout_{dt}_{ao}{bo}", a_type=dt, b_type=dt, c_type=dt, a_order=ao,
                  b_order=bo, alpha=1.0, beta=0.0, dist_a=("normal", 1.0),
                  dist_b=("normal", 1.0), seed=71, **_padded(ao, bo, **shape))
    for small_int in (True, False):
        text = _run(p, small_int)
        assert f"kernel=mfma_{'bf16' if dt == W.BF16 else 'f16'}" in text
        assert f"_{tile}x" in text, text


@pytest.mark.parametrize("ao,bo", LAYOUTS[:3], ids=[f"A{a}_B{b}" for a, b in LAYOUTS[:3]])
def test_layout_epilogue_terms_padding_and_batch(ao, bo):
    # alpha, beta * C, bias, GELU, fp32 output, padded leading dimensions
    # and a batch with B broadcast
    M, N, K = 264, 200, 136
    lda = (K if ao == W.ROW else M) + 8
    ldb = (N if bo == W.ROW else K) + 16
    p = W.Problem(name=f"layout_terms_{ao}{bo}", M=M, N=N, K=K, batch=3, a_type=W.BF16,
                  b_type=W.BF16, c_type=W.F32, a_order=ao, b_order=bo, lda=lda, ldb=ldb,
                  stride_b=0, alpha=1.5, beta=0.5, has_bias=True, bias_type=W.BF16,
                  act=W.ACT_GELU_ERF, dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=72)
    for small_int in (True, False):
        text = _run(p, small_int)
        assert "kernel=mfma_bf16" in text


@pytest.mark.parametrize("ao,bo", LAYOUTS[:3], ids=[f"A{a}_B{b}" for a, b in LAYOUTS[:3]])
@pytest.mark.parametrize("sched", ["split_k", "stream_k"])
def test_layout_split_and_stream_k(ao, bo, sched):
    if sched == "split_k":
        # a ragged K split into slices: the last slice ends at K and, where
        # an edge cuts a chunk, loads its last K tile through registers
        p = W.Problem(name=f"layout_splitk_{ao}{bo}", a_type=W.BF16,
                      b_type=W.BF16, c_type=W.F32, a_order=ao, b_order=bo, split_k=3,
                      **_padded(ao, bo, 134, 131, 4104),
                      dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=73)
        kw = {}
    else:
        p = W.Problem(name=f"layout_streamk_{ao}{bo}", M=1160, N=1160, K=2056, a_type=W.BF16,
                      b_type=W.BF16, c_type=W.BF16, a_order=ao, b_order=bo,
                      dist_a=("normal", 1.0), dist_b=("normal", 1.0), seed=74)
        kw = dict(schedule=dg.DG_SCHED_STREAM_K)
    for small_int in (True, False):
        text = _run(p, small_int, **kw)
        if sched == "split_k":
            assert "splits=3" in text
        else:
            assert "schedule=stream_k" in text


def test_c3_shape_with_row_major_b_sampled():
    """The bf16 4096^3 workload with B stored row-major (PyTorch's default
    layout for both operands), in the launch configuration the library
    picks, on sampled outputs."""
    from workloads.device import DeviceProblem
    p = W.WORKLOADS["c3"].replace(name="gemm_bf16_4096_nn", b_order=W.ROW)
    x = W.make_inputs(p)
    dp = DeviceProblem(p, x)
    text = dp.describe()
    print(f"[{p.name}] {text}", flush=True)
    assert "kernel=mfma_bf16" in text and "tile=mfma_bf16_256x256" in text
    dp.run()
    pts = W.sample_points(p, 3000)
    ref, mag, out = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
    check(p, dp.result(), ref, mag, out, pts=pts, what=p.name)
