"""GPU parity of the stream-K schedule against the CPU oracle.

The tiles of the full waves are computed data-parallel; each tail tile is
cut into K slices whose fp32 partials a second kernel adds in slice order
before the epilogue.  Forced on grids smaller than a wave, every tile is a
tail tile, which keeps the full-matrix oracle checks fast; the automatic
choice is checked on the GELU workload (data-parallel waves plus a tail).
Small-integer inputs make every result exact in fp32, so the sliced sums
must equal the oracle bit for bit."""

import numpy as np
import pytest

import dense_gemm_10_amd as dg
import oracle
import workloads as W
from parity_util import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SK = dg.DG_SCHED_STREAM_K


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16(name, M, N, K, **kw):
    base = dict(name=name, M=M, N=N, K=K, a_type=W.BF16, b_type=W.BF16, c_type=W.BF16,
                a_order=W.ROW, b_order=W.COL, alpha=1.0, beta=0.0, seed=77)
    base.update(kw)
    return W.Problem(**base)


def _run(p, x, **kw):
    from workloads.device import DeviceProblem
    dp = DeviceProblem(p, x, **kw)
    text = dp.describe()
    print(f"[{p.name}] {text}", flush=True)
    dp.run()
    return dp, text


def _check_full(p, small_int, **kw):
    x = W.make_inputs(p, small_int=small_int)
    dp, text = _run(p, x, **kw)
    ref, mag, out = oracle.gemm(p, x.A, x.B, x.C, x.bias)
    check(p, dp.result(), ref, mag, out, exact=small_int and p.act == W.ACT_NONE,
          what=f"{p.name} int={small_int}")
    return text


def _check_sampled(p, small_int, n=3000, **kw):
    x = W.make_inputs(p, small_int=small_int)
    dp, text = _run(p, x, **kw)
    pts = W.sample_points(p, n)
    ref, mag, out = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
    check(p, dp.result(), ref, mag, out, pts=pts, exact=small_int and p.act == W.ACT_NONE,
          what=f"{p.name} sampled int={small_int}")
    return text


def _tail(text):
    kv = dict(t.split("=", 1) for t in text.split() if "=" in t)
    return int(kv["tail_tiles"]), int(kv["tail_splits"])


# 5 x 5 tiles of 128 x 128, all in the tail, K = 1024 in 16 slices (K = 1000:
# the last slice ends in a partial K step)
@pytest.mark.parametrize("K", [1024, 1000])
@pytest.mark.parametrize("small_int", [True, False])
def test_stream_k_128_full(K, small_int):
    p = _bf16(f"sk128_K{K}", 640, 640, K)
    text = _check_full(p, small_int, schedule=SK)
    assert "schedule=stream_k" in text and _tail(text)[1] >= 2


def test_stream_k_epilogue_fp32_out_beta_bias_gelu():
    p = _bf16("sk128_epi", 640 - 7, 640 + 5, 1000, c_type=W.F32, alpha=1.5, beta=0.5,
              has_bias=True, bias_type=W.BF16, act=W.ACT_GELU_ERF)
    text = _check_full(p, False, schedule=SK)
    assert _tail(text)[1] >= 2


# 17 x 17 tiles of 256 x 256 (one wave is 256): 256 data-parallel, 33 in the tail
@pytest.mark.parametrize("small_int", [True, False])
def test_stream_k_256_sampled(small_int, monkeypatch):
    monkeypatch.setenv("DG_FORCE_TILE", "mfma_bf16_256x256x64_w2x2_s2")
    p = _bf16("sk256", 4352, 4352 - 3, 1024)
    text = _check_sampled(p, small_int, schedule=SK)
    assert "bm=256" in text and "dp_tiles=256" in text
    assert _tail(text)[0] == 33 and _tail(text)[1] >= 2


def test_automatic_stream_k_matches_data_parallel():
    # a grid like the GELU workload's with a long K and N = 4352 (17 full
    # tile columns, so no sliver columns): the library's own plan (stream-K,
    # with workspace) and the data-parallel plan agree bit for bit on
    # small-integer inputs
    p = W.WORKLOADS["c4"].replace(name="c4_longk", K=4096, N=4352, act=W.ACT_NONE)
    x = W.make_inputs(p, small_int=True)
    dp1, t1 = _run(p, x)
    dp2, t2 = _run(p, x, schedule=dg.DG_SCHED_DATA_PARALLEL)
    assert "schedule=stream_k" in t1 and "schedule=data_parallel" in t2
    assert np.array_equal(dp1.result().view(np.uint8), dp2.result().view(np.uint8))


def test_stream_k_is_deterministic():
    p = _bf16("sk_det", 1000, 1000, 4096)
    x = W.make_inputs(p)
    dp, _ = _run(p, x, schedule=SK)
    first = dp.result().copy()
    for _ in range(3):
        dp.reset_c()
        dp.run()
        assert np.array_equal(dp.result().view(np.uint8), first.view(np.uint8))


# explicit K-slice counts of the tail tiles (split_k under the stream-K
# schedule), including counts that do not divide K
@pytest.mark.parametrize("slices", [3, 5, 16])
def test_stream_k_explicit_slices(slices):
    p = _bf16(f"sk_slices{slices}", 640, 640 - 3, 1000, split_k=slices)
    text = _check_full(p, True, schedule=SK)
    # slices of ceil(K / S) rounded up to whole K steps: 5 slices of K = 1000
    # in steps of 64 are 256 long, so 4 of them cover K
    bk = int(dict(t.split("=", 1) for t in text.split() if "=" in t)["bk"])
    kps = -(-(-(-1000 // slices)) // bk) * bk
    assert "splits=1 " in text and _tail(text)[1] == -(-1000 // kps)
