"""Seeded random shapes through the fused forward, the unfused reference
chain and the backward (C ABI), each against the fp64 oracle: the same bars
as the fixed-shape tests (max|x - x_ref| / max|x_ref| <= 1e-2 bf16, 1e-5
fp32; H bit-identical between the fused and the unfused chain).  The shapes
are drawn once from a fixed seed: M in [1, 700], K, D, N2 multiples of 8 in
[8, 1104], so that tiles, k-tiles and slabs end ragged in every combination.
"""
import sys

import numpy as np
import pytest
import torch

import coda_inputs as ci
import oracle
import transformer_gemm_epilogue_gemm1_amd as coda
from tests.gpu_util import dev, host_bits, host_f32, max_rel, tolerance

pytestmark = pytest.mark.gpu


def _shapes(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 701))
        K, D, N2 = (int(8 * rng.integers(1, 139)) for _ in range(3))
        out.append((M, K, D, N2))
    return out


SHAPES = _shapes(12)


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_shape_forward_backward(shape, dtype):
    M, K, D, N2 = shape
    wl = ci.custom_workload(M, K, D, N2, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=900)
    x = ci.make_inputs(wl, seed=sum(shape), with_dy=True)
    d = {k: dev(v) for k, v in x.items()}
    H, Hg, r, Y, P = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    Hr, rr, Yr = coda.ref_chain(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    grads = coda.fused_backward(d["dY"], d["A"], d["W1"], d["g"], d["W2"], H, r)
    torch.cuda.synchronize()
    tol = tolerance(dtype)
    fo = oracle.forward(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps)
    assert max_rel(host_f32(Y), fo["Y"]) <= tol
    assert max_rel(host_f32(Yr), fo["Y"]) <= tol
    assert np.array_equal(host_bits(H), host_bits(Hr))
    bo = oracle.backward(x["dY"].f32, x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps)
    for k, t in zip(("dA", "dR", "dW1", "dW2", "dg"), grads):
        err = max_rel(host_f32(t), bo[k])
        assert err <= tol, f"{k}: error {err:.3e}"
