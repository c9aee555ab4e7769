"""Move seeded host buffers to the GPU and run one problem through the
library's C ABI (dg_gemm).  Marshalling only: no GEMM arithmetic here."""
from __future__ import annotations

import numpy as np

from . import F32, Problem, desc_fields


def to_device(arr, device="cuda"):
    """Host storage array (float32, or uint16 bf16 / fp16 bits) -> device tensor with
    the same bytes."""
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    if t.numel() == 0:
        t = torch.zeros(1, dtype=t.dtype)
    return t.to(device)


def to_host(t, dtype):
    """Device tensor -> host numpy array in storage dtype."""
    a = t.cpu().numpy()
    return a if dtype == F32 else a.view(np.uint16)


class DeviceProblem:
    """Device copies of one problem's operands plus its descriptor."""

    def __init__(self, p: Problem, x, device="cuda", **desc_overrides):
        import dense_gemm_10_amd as dg
        self.p = p
        self.A = to_device(x.A, device)
        self.B = to_device(x.B, device)
        self.C0 = to_device(x.C, device)
        self.C = self.C0.clone()
        self.bias = to_device(x.bias, device) if x.bias is not None else None
        f = desc_fields(p)
        f.update(desc_overrides)
        f["bias"] = self.bias.data_ptr() if self.bias is not None else None
        self.desc = dg.make_desc(**f)
        self.ws_bytes = dg.dg_gemm_workspace_size(self.desc)
        import torch
        self.ws = (torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)
                   if self.ws_bytes else None)

    def reset_c(self):
        self.C.copy_(self.C0)

    def describe(self):
        import dense_gemm_10_amd as dg
        return dg.dg_gemm_describe(self.desc, self.ws_bytes)

    def run(self, stream=None):
        """Enqueue C = act(alpha A B + beta C + bias) on `stream` (default:
        torch's current stream)."""
        import torch
        import dense_gemm_10_amd as dg
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        dg.dg_gemm(self.desc, self.A.data_ptr(), self.B.data_ptr(), self.C.data_ptr(),
                   self.ws.data_ptr() if self.ws is not None else None, self.ws_bytes, stream)

    def result(self):
        import torch
        torch.cuda.synchronize()
        return to_host(self.C, self.p.c_type)


def run_once(p: Problem, x, **desc_overrides):
    """Copy, run once from the given C_in, synchronise, return C (host)."""
    dp = DeviceProblem(p, x, **desc_overrides)
    dp.run()
    return dp.result()
