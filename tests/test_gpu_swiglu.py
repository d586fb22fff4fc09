"""GPU parity of the SwiGLU epilogue (coda_gemm_rowscale_swiglu) and of the
backward through the gate (coda_swiglu_bwd + coda_chain_bwd), through the C ABI.

The chain runs on the GPU up to r and Hg (coda_gemm_res_prms +
coda_rms_combine), then the gated second GEMM writes Z = silu(Y_gate) * Y_up
(and optionally the pre-activation Y).  Z is compared element by element with
the fp64 oracle of the same chain on the same seeded inputs (bars:
max|Z - Z_ref| / max|Z_ref| <= 1e-2 bf16, 1e-5 fp32).  Stage-wise: the kept Y
is bit-identical to the plain row-scale GEMM's output (same accumulation
order, only the column order of the B loads differs), and Z matches host fp64
arithmetic on the GPU's own Hg and r to one rounding.
"""
import sys

import numpy as np
import pytest
import torch

import coda_inputs as ci
import oracle
import transformer_gemm_epilogue_gemm1_amd as coda
from tests.gpu_util import dev, host_bits, host_f32, max_rel, tolerance, whole_max_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
    torch.cuda.synchronize()


def _run(wl, seed, keep_y=True):
    x = ci.make_inputs(wl, seed=seed)
    d = {k: dev(v) for k, v in x.items()}
    H, Hg, r, Z, Y = coda.fused_forward_swiglu(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, keep_y=keep_y)
    torch.cuda.synchronize()
    return x, d, {"H": H, "Hg": Hg, "r": r, "Z": Z, "Y": Y}


def _check(wl, x, o, rows=None):
    orc = oracle.forward_swiglu(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    err = max_rel(host_f32(o["Z"])[sel], orc["Z"])
    assert err <= tolerance(wl.dtype), f"Z error {err:.3e}"
    if o["Y"] is not None:
        yerr = max_rel(host_f32(o["Y"])[sel], orc["Y"])
        assert yerr <= tolerance(wl.dtype), f"Y error {yerr:.3e}"
    return err


def _check_stages(wl, d, o):
    # Y bit-identical to the plain second GEMM on the same Hg and r
    Yp = torch.empty_like(o["Y"])
    coda.coda_gemm_rowscale(o["Hg"], d["W2"], o["r"], Yp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Yp), host_bits(o["Y"])), "gated GEMM's Y differs from the plain GEMM's"
    # Z against host fp64 on the GPU's own operands (one rounding of fp32 work)
    y = host_f32(o["Hg"]).astype(np.float64) @ host_f32(d["W2"]).astype(np.float64)
    y *= o["r"].cpu().numpy().astype(np.float64)[:, None]
    F = y.shape[1] // 2
    z = oracle.silu(y[:, :F]) * y[:, F:]
    tol = 2.0 ** -8 if wl.dtype == "bf16" else 2e-6
    assert max_rel(host_f32(o["Z"]), z) <= tol


SHAPES = [  # M, K, D, F (F a multiple of 32, 2F ragged against 256-column tiles)
    (1, 64, 256, 128),
    (3, 136, 264, 288),
    (257, 256, 512, 384),
    (300, 512, 384, 544),
    (513, 1024, 1024, 1024),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_swiglu_matches_oracle(shape, dtype):
    M, K, D, F = shape
    wl = ci.custom_workload(M, K, D, 2 * F, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=400)
    x, d, o = _run(wl, seed=1)
    _check(wl, x, o)
    _check_stages(wl, d, o)


def test_z_alone_equals_z_with_y_and_repeats():
    wl = ci.custom_workload(300, 256, 512, 1024, wl_id=401)
    x, d, o = _run(wl, seed=2)
    Z2 = torch.full_like(o["Z"], float("nan"))
    coda.coda_gemm_rowscale_swiglu(o["Hg"], d["W2"], o["r"], Z2, None)
    Z3 = torch.full_like(o["Z"], float("nan"))
    coda.coda_gemm_rowscale_swiglu(o["Hg"], d["W2"], o["r"], Z3, None)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Z2), host_bits(o["Z"]))
    assert np.array_equal(host_bits(Z3), host_bits(Z2))


def test_without_row_scale_and_strided():
    # r = NULL: Z = silu(X W_gate) * (X W_up); operands as column slices of wider buffers
    M, D, F = 200, 512, 384
    wl = ci.custom_workload(M, 8, D, 2 * F, wl_id=402)
    x = ci.make_inputs(wl, seed=3)

    def wide(t, extra):
        w = torch.zeros((t.shape[0], t.shape[1] + extra), device=t.device, dtype=t.dtype)
        w[:, :t.shape[1]] = t
        return w[:, :t.shape[1]]

    X = wide(dev(x["R"]), 16)
    W2 = wide(dev(x["W2"]), 40)
    Z = wide(torch.empty((M, F), device="cuda", dtype=torch.bfloat16), 8)
    Y = wide(torch.empty((M, 2 * F), device="cuda", dtype=torch.bfloat16), 24)
    coda.coda_gemm_rowscale_swiglu(X, W2, None, Z, Y)
    torch.cuda.synchronize()
    y = x["R"].f64() @ x["W2"].f64()
    z = oracle.silu(y[:, :F]) * y[:, F:]
    assert max_rel(host_f32(Z.contiguous()), z) <= 4e-3
    assert max_rel(host_f32(Y.contiguous()), y) <= 4e-3


@pytest.mark.slow
def test_full_size_7b_whole_tensor():
    # the 7B shape (F = 14336) in the benchmark's launch configuration, Z
    # against the oracle over every row
    wl = ci.WORKLOADS["7b-bf16"]
    x, d, o = _run(wl, seed=0, keep_y=False)
    W1, g, W2 = x["W1"].f64(), x["g"].f64(), x["W2"].f64()

    def orc(rows):
        return {"Z": oracle.forward_swiglu(x["A"].f32, W1, x["R"].f32, g, W2, wl.eps, rows=rows)["Z"]}

    err = whole_max_rel(orc, {"Z": o["Z"]}, wl.M)["Z"]
    print(f"7b-bf16 SwiGLU whole-tensor Z error {err:.3e}", file=sys.__stderr__, flush=True)
    assert err <= 1e-2


# ---- backward through the gate (coda_swiglu_bwd), then the chain's backward ----
# dZ is the first F columns of the seeded upstream-gradient draw (N(0, 1)).

def _swiglu_train(wl, seed):
    x = ci.make_inputs(wl, seed=seed, with_dy=True)
    F = wl.N2 // 2
    d = {k: dev(v) for k, v in x.items()}
    dZ = d["dY"][:, :F].contiguous()
    H, Hg, r, Z, Y = coda.fused_forward_swiglu(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, keep_y=True)
    grads = coda.fused_backward_swiglu(dZ, Y, d["A"], d["W1"], d["g"], d["W2"], H, r)
    torch.cuda.synchronize()
    return x, dZ, Y, dict(zip(("dA", "dR", "dW1", "dW2", "dg", "dY"), grads))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 136, 264, 288), (257, 256, 512, 384), (513, 512, 1024, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_swiglu_backward_matches_oracle(shape, dtype):
    M, K, D, F = shape
    wl = ci.custom_workload(M, K, D, 2 * F, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=410)
    x, dZ, Y, out = _swiglu_train(wl, seed=5)
    dz = host_f32(dZ).astype(np.float64)
    # stage: dY against host fp64 on the GPU's own dZ and Y (one rounding)
    dy_host = oracle.swiglu_dy(dz, host_f32(Y).astype(np.float64))
    assert max_rel(host_f32(out["dY"]), dy_host) <= (2.0 ** -8 if dtype == "bf16" else 2e-6)
    # end to end: every gradient against the oracle's backward of <dZ, Z>
    orc = oracle.backward_swiglu(dz, x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps)
    for k in ("dY", "dA", "dR", "dW1", "dW2", "dg"):
        err = max_rel(host_f32(out[k]), orc[k])
        assert err <= tolerance(dtype), f"{k}: error {err:.3e}"


@pytest.mark.slow
def test_swiglu_bwd_full_size_whole_tensor():
    # the gate's backward at the 7B shape (M = 16384, F = 14336), every row;
    # Y and dZ drawn on the host (seeded) and uploaded
    wl = ci.WORKLOADS["7b-bf16"]
    F = wl.N2 // 2
    rng = np.random.default_rng(11)
    y_bits = ci.bf16_bits((rng.standard_normal((wl.M, 2 * F), dtype=np.float32) * 2.0).astype(np.float32))
    dz_bits = ci.bf16_bits(rng.standard_normal((wl.M, F), dtype=np.float32))
    Y = torch.from_numpy(y_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dZ = torch.from_numpy(dz_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dY = torch.full_like(Y, float("nan"))
    coda.coda_swiglu_bwd(dZ, Y, dY)
    torch.cuda.synchronize()

    def orc(rows):
        return {"dY": oracle.swiglu_dy(ci.bf16_bits_to_f32(dz_bits[rows]), ci.bf16_bits_to_f32(y_bits[rows]))}

    err = whole_max_rel(orc, {"dY": dY}, wl.M, block=1024)["dY"]
    print(f"7b SwiGLU gate backward whole-tensor dY error {err:.3e}", file=sys.__stderr__, flush=True)
    assert err <= 2.0 ** -8