"""coda_chain_bwd_noalloc (the backward without a workspace, scratch in the
library's static device array) against coda_chain_bwd on the same inputs.

Two calls in a row on one GPU, the second with a smaller input, so the
second runs on scratch the first left behind: each call's five gradients are
bit-identical to coda_chain_bwd's (the products see the same fragments; only
where the weights are read from differs).  The first shape needs nearly all
of the 64 MiB scratch.  Outputs are NaN-poisoned before each call.
"""
import sys

import numpy as np
import pytest
import torch

import coda_inputs as ci
import transformer_gemm_epilogue_gemm1_amd as coda
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

GRADS = ("dA", "dR", "dW1", "dW2", "dg")


def _inputs(shape, dtype, wl_id):
    wl = ci.custom_workload(*shape, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=wl_id)
    x = ci.make_inputs(wl, seed=wl_id, with_dy=True)
    d = {k: dev(v) for k, v in x.items()}
    H, Hg, r, Y, P = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    d["H"], d["r"] = H, r
    return wl, d


def _outputs(wl, d):
    M, K, D, N2 = wl.M, wl.K, wl.D, wl.N2
    t = d["A"].dtype
    nan = float("nan")
    return {"dA": torch.full((M, K), nan, device="cuda", dtype=t), "dR": torch.full((M, D), nan, device="cuda", dtype=t),
            "dW1": torch.full((K, D), nan, device="cuda", dtype=t), "dW2": torch.full((D, N2), nan, device="cuda", dtype=t),
            "dg": torch.full((D,), nan, device="cuda", dtype=torch.float32)}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_backward_matches_workspace_backward(dtype):
    big = (7680, 512, 4096, 1024) if dtype == "bf16" else (3840, 256, 4096, 512)   # near the scratch limit
    small = (300, 256, 512, 1032)
    for i, shape in enumerate((big, small)):
        print(f"[no-alloc] {dtype} call {i + 1}: M, K, D, N2 = {shape}", file=sys.__stderr__, flush=True)
        wl, d = _inputs(shape, dtype, wl_id=950 + i)
        args = (d["dY"], d["A"], d["W1"], d["g"], d["W2"], d["H"], d["r"])
        ref = _outputs(wl, d)
        ws = torch.empty((coda.coda_chain_bwd_workspace_bytes(d["A"].dtype, wl.M, wl.K, wl.D, wl.N2),),
                         device="cuda", dtype=torch.uint8)
        coda.coda_chain_bwd(*args, *(ref[k] for k in GRADS), ws)
        out = _outputs(wl, d)
        coda.coda_chain_bwd_noalloc(*args, *(out[k] for k in GRADS))
        torch.cuda.synchronize()
        for k in GRADS:
            assert torch.isfinite(out[k].float()).all().item(), f"{k}: not every element written"
            assert torch.equal(_bits(out[k]), _bits(ref[k])), f"{k} differs from coda_chain_bwd's"
