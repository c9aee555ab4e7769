"""dg_gemm_noalloc, the entry point for callers that cannot allocate: the
same results as dg_gemm with a caller-provided workspace, for several calls
in a row on one GPU, each smaller than the one before, covering a stream-K
plan, split-K plans and a plan without workspace.  Both paths run the same
plan here, so their outputs must agree bit for bit; each is also held to
the oracle on sampled outputs (the acceptance tolerances)."""
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


# Each call smaller than the one before; the first two use the scratch
# array for stream-K and split-K partials.
CASES = [
    W.WORKLOADS["c4"],                                              # stream-K tail (tuned)
    W.WORKLOADS["c5"],                                              # split-K, 16 MiB
    W.WORKLOADS["c5"].replace(name="c5_small", batch=4, K=8192),    # split-K, 2 MiB
    W.WORKLOADS["c3"].replace(name="c3_small", M=300, N=264, K=200),  # no workspace
]


def test_noalloc_matches_dg_gemm_call_after_call():
    import dense_gemm_10_amd as dg
    from workloads.device import DeviceProblem
    stream = torch.cuda.current_stream().cuda_stream
    for p in CASES:
        x = W.make_inputs(p)
        dp = DeviceProblem(p, x)
        plan = dp.describe()
        print(f"[noalloc] {p.name}: {plan}", flush=True)
        assert dp.ws_bytes <= dg.DG_NOALLOC_SCRATCH_BYTES
        dp.run(stream)
        want = dp.result()
        dp.reset_c()
        torch.cuda.synchronize()
        dg.dg_gemm_noalloc(dp.desc, dp.A.data_ptr(), dp.B.data_ptr(), dp.C.data_ptr(), stream)
        got = dp.result()
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), p.name
        pts = W.sample_points(p, 2000)
        ref, mag, out = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
        check(p, got, ref, mag, out, pts=pts, what=f"noalloc {p.name}")
        del dp
