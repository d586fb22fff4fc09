"""GPU parity of the backward chain (coda_chain_bwd) through the C ABI.

The GPU forward (coda_gemm_res_prms + coda_rms_combine) produces the stored
H and r that the backward consumes, as in training.  Every gradient (dA, dR,
dW1, dW2, dg) is compared element by element with the fp64 CPU oracle's
reverse-mode backward of the plain chain on the same seeded inputs.  Bars:
max|x - x_ref| / max|x_ref| <= 1e-2 (bf16) or 1e-5 (fp32) per tensor.

Stage-wise checks pin each backward GEMM on the GPU's own intermediates with
host fp64 arithmetic: dA = dH W1^T, dW1 = A^T dH (dH = the returned dR), and
dW2 = X_n^T dY with X_n = round((H r) g) formed on the host from the stored
H and r.
"""
import sys

import numpy as np
import pytest
import torch

import coda_inputs as ci
import oracle
import transformer_gemm_epilogue_gemm1_amd as coda
from tests.gpu_util import dev, host_bits, host_f32, max_rel, round_to, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
    torch.cuda.synchronize()


GRADS = ("dA", "dR", "dW1", "dW2", "dg")


def _forward_backward(wl, seed):
    x = ci.make_inputs(wl, seed=seed, with_dy=True)
    d = {k: dev(v) for k, v in x.items()}
    H, Hg, r, Y, P = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    grads = coda.fused_backward(d["dY"], d["A"], d["W1"], d["g"], d["W2"], H, r)
    torch.cuda.synchronize()
    return x, d, {"H": H, "r": r, "Y": Y}, dict(zip(GRADS, grads))


def _check_oracle(wl, x, out, tol=None):
    orc = oracle.backward(x["dY"].f32, x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps)
    errs = {}
    for k in GRADS:
        errs[k] = max_rel(host_f32(out[k]), orc[k])
        assert errs[k] <= (tol or tolerance(wl.dtype)), f"{k}: error {errs[k]:.3e}"
    return errs


def _check_stages(wl, x, fwd, out):
    """Each backward GEMM against host fp64 products of the GPU's own operands."""
    dH = host_f32(out["dR"]).astype(np.float64)
    H = host_f32(fwd["H"]).astype(np.float32)
    r = fwd["r"].cpu().numpy().astype(np.float32)
    # bf16: one rounding of an fp32 accumulation (half an ulp, 2^-9, with
    # headroom); fp32: the accumulation error itself, within the parity bar
    tol = 2.0 ** -8 if wl.dtype == "bf16" else 1e-5
    dA = dH @ x["W1"].f64().T
    assert max_rel(host_f32(out["dA"]), dA) <= tol
    dW1 = x["A"].f64().T @ dH
    assert max_rel(host_f32(out["dW1"]), dW1) <= tol
    xn = round_to(wl.dtype, (H * r[:, None]).astype(np.float32) * x["g"].f32[None, :]).astype(np.float64)
    dW2 = xn.T @ x["dY"].f64()
    assert max_rel(host_f32(out["dW2"]), dW2) <= tol


def test_tiny_fp32_workload():
    wl = ci.WORKLOADS["tiny-fp32"]
    x, d, fwd, out = _forward_backward(wl, seed=0)
    errs = _check_oracle(wl, x, out)
    _check_stages(wl, x, fwd, out)
    print("tiny-fp32 backward errors", {k: f"{v:.2e}" for k, v in errs.items()})


SHAPES = [
    (1, 64, 256, 256),
    (3, 136, 264, 520),
    (128, 256, 256, 256),
    (257, 256, 512, 768),
    (300, 512, 384, 1032),
    (513, 1024, 1024, 2048),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_matches_oracle(shape, dtype):
    M, K, D, N2 = shape
    wl = ci.custom_workload(M, K, D, N2, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=300)
    x, d, fwd, out = _forward_backward(wl, seed=1)
    _check_oracle(wl, x, out)
    _check_stages(wl, x, fwd, out)


def test_repeatable_and_overwrites_poison():
    wl = ci.custom_workload(300, 256, 512, 768, wl_id=301)
    x, d, fwd, out = _forward_backward(wl, seed=2)
    poisoned = {k: torch.full_like(v, float("nan")) for k, v in out.items()}
    ws = torch.full((coda.coda_chain_bwd_workspace_bytes(torch.bfloat16, wl.M, wl.K, wl.D, wl.N2),), 0xFF,
                    device="cuda", dtype=torch.uint8)
    coda.coda_chain_bwd(d["dY"], d["A"], d["W1"], d["g"], d["W2"], fwd["H"], fwd["r"], poisoned["dA"],
                        poisoned["dR"], poisoned["dW1"], poisoned["dW2"], poisoned["dg"], ws)
    torch.cuda.synchronize()
    for k in GRADS:
        assert np.array_equal(host_bits(poisoned[k]), host_bits(out[k])), k


def test_zero_upstream_gradient():
    wl = ci.custom_workload(200, 256, 256, 512, wl_id=302)
    x, d, fwd, out = _forward_backward(wl, seed=3)
    zero = torch.zeros_like(d["dY"])
    grads = coda.fused_backward(zero, d["A"], d["W1"], d["g"], d["W2"], fwd["H"], fwd["r"])
    torch.cuda.synchronize()
    for k, t in zip(GRADS, grads):
        assert torch.count_nonzero(t).item() == 0, k


def test_empty_batch_writes_zero_weight_gradients():
    K, D, N2 = 64, 256, 512
    wl = ci.custom_workload(8, K, D, N2, wl_id=303)
    x = ci.make_inputs(wl, seed=4, with_dy=True)
    d = {k: dev(v) for k, v in x.items()}
    e = lambda *s, dt=torch.bfloat16: torch.empty(s, device="cuda", dtype=dt)  # noqa: E731
    dW1 = torch.full((K, D), float("nan"), device="cuda", dtype=torch.bfloat16)
    dW2 = torch.full((D, N2), float("nan"), device="cuda", dtype=torch.bfloat16)
    dg = torch.full((D,), float("nan"), device="cuda")
    ws = e(coda.coda_chain_bwd_workspace_bytes(torch.bfloat16, 0, K, D, N2), dt=torch.uint8)
    coda.coda_chain_bwd(e(0, N2), e(0, K), d["W1"], d["g"], d["W2"], e(0, D), e(0, dt=torch.float32),
                        e(0, K), e(0, D), dW1, dW2, dg, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW1).item() == 0 and not torch.isnan(dW1.float()).any().item()
    assert torch.count_nonzero(dW2).item() == 0 and not torch.isnan(dW2.float()).any().item()
    assert torch.count_nonzero(dg).item() == 0 and not torch.isnan(dg).any().item()


@pytest.mark.slow
def test_full_size_7b_backward():
    # the 7B backward workload at full size in the benchmark's launch
    # configuration, against the full fp64 oracle backward
    wl = ci.WORKLOADS["7b-bwd-bf16"]
    x, d, fwd, out = _forward_backward(wl, seed=0)
    errs = _check_oracle(wl, x, out)
    print("7b-bwd-bf16 errors", {k: f"{v:.2e}" for k, v in errs.items()})
