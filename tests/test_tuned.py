"""GPU parity of every plan in the offline-tuned table at its own full shape
(the exact M, N, K and batch it was tuned for, through the library's own
plan: tile, schedule and slice count from the table), on small-integer
inputs where every result is exact: sampled outputs, corners included, must
equal the oracle bit for bit (GELU workloads within the 16-bit
tolerance)."""
import os
import re

import pytest

import oracle
import workloads as W
from conftest import ROOT
from dense_gemm_10_amd.tune import shapes
from parity_util import check

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

FAM_TYPE = {"KERNEL_MFMA_BF16": "bf16", "KERNEL_MFMA_F16": "f16", "KERNEL_MFMA_F32": "f32"}


def _entries():
    text = open(os.path.join(ROOT, "dense_gemm_10_amd", "csrc", "tuned_table.inc")).read()
    pat = (r'\{(KERNEL_\w+), (\d+), (\d+), (\d+), (\d+), "([\w]+)", (DG_SCHED_\w+), '
           r'(\d+)\},')
    by_shape = {(p.M, p.N, p.K, p.batch, p.a_type): p for p in shapes()}
    out = []
    for k, M, N, K, b, tile, sched, S in re.findall(pat, text):
        out.append((by_shape[(int(M), int(N), int(K), int(b), FAM_TYPE[k])], tile, sched))
    return out


ENTRIES = _entries()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("p,tile,sched", ENTRIES, ids=[e[0].name for e in ENTRIES])
def test_tuned_plan_full_shape(p, tile, sched):
    from workloads.device import DeviceProblem
    x = W.make_inputs(p, small_int=True)
    dp = DeviceProblem(p, x)
    text = dp.describe()
    print(f"[{p.name}] {text}", flush=True)
    assert "tuned=1" in text and f"tile={tile} " in text
    dp.run()
    pts = W.sample_points(p, 600)
    ref, mag, out = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, *pts)
    check(p, dp.result(), ref, mag, out, pts=pts, exact=p.act == W.ACT_NONE,
          what=f"{p.name} tuned {tile} {sched}")
