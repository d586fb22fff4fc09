"""GPU parity of the fused forward chain and the unfused reference chain.

Every case runs libcoda's kernels through the C ABI on seeded inputs and
compares element by element with the fp64 CPU oracle (the plain
GEMM-residual-RMSNorm-GEMM definition from the CODA news article by Synced,
epilogue section).  Bars: max|Y - Y_ref| / max|Y_ref| <= 1e-2 for bf16 and
<= 1e-5 for fp32; H within one rounding of the exact value; H bit-identical
between the fused and the unfused chain; repeated calls bit-identical.
Stage-wise checks of the fused path use host arithmetic on the GPU's own
intermediates: Hg = round(float(H) * g) exactly, the partial sums of squares
add up to sum(float(H)^2), and r = 1/sqrt(mean + eps) of them.
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


def _run(wl, seed=0, ref=True):
    x = ci.make_inputs(wl, seed=seed)
    d = {k: dev(v) for k, v in x.items()}
    H, Hg, r, Y, P = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    out = {"x": x, "d": d, "H": H, "Hg": Hg, "r": r, "Y": Y, "P": P}
    if ref:
        out["ref"] = coda.ref_chain(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    torch.cuda.synchronize()
    return out


def _check_against_oracle(wl, o, rows=None):
    x = o["x"]
    orc = oracle.forward(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    H = host_f32(o["H"])[sel]
    Y = host_f32(o["Y"])[sel]
    r = o["r"].cpu().numpy()[sel]
    # H: one rounding of an fp32 accumulation of the exact value
    rt = 2.0 ** -8 if wl.dtype == "bf16" else 1e-6
    np.testing.assert_allclose(H, orc["H"], rtol=rt * 1.01, atol=1e-5)
    np.testing.assert_allclose(r, orc["r"], rtol=2e-3 if wl.dtype == "bf16" else 1e-5)
    err = max_rel(Y, orc["Y"])
    assert err <= tolerance(wl.dtype), f"fused Y error {err:.3e}"
    ref_err = None
    if "ref" in o:
        Hr, rr, Yr = o["ref"]
        assert np.array_equal(host_bits(Hr), host_bits(o["H"])), "fused H differs from the unfused chain's H"
        ref_err = max_rel(host_f32(Yr)[sel], orc["Y"])
        assert ref_err <= tolerance(wl.dtype), f"unfused Y error {ref_err:.3e}"
        _comparable(err, ref_err, wl.dtype)
    return err, ref_err


def _comparable(err, ref_err, dtype):
    """The fused chain is as accurate as the operator-by-operator chain (the
    CODA news article, results section: error comparable to the PyTorch
    reference, sometimes smaller): its error against the oracle is at most
    1.25x the unfused chain's, up to 5% of the tolerance (both chains round
    Y and one operand of the second product to the storage dtype, in
    different places)."""
    assert err <= 1.25 * ref_err + 0.05 * tolerance(dtype), f"fused error {err:.3e} vs unfused {ref_err:.3e}"
    print(f"Y error against the oracle: fused {err:.3e}, unfused {ref_err:.3e}", file=sys.__stderr__, flush=True)


def _check_stages(wl, o):
    """The fused path's intermediates against host arithmetic on the GPU's own H."""
    x = o["x"]
    H = host_f32(o["H"]).astype(np.float32)
    g = x["g"].f32
    hg = (H * g[None, :]).astype(np.float32)
    want = ci.bf16_bits(hg) if wl.dtype == "bf16" else hg.view(np.uint32)
    np.testing.assert_array_equal(host_bits(o["Hg"]), want)
    P = o["P"].cpu().numpy().astype(np.float64)
    T = coda.coda_prms_num_partials(o["H"].dtype, wl.D)
    assert P.shape == (T, wl.M)
    H64 = H.astype(np.float64)
    ss = np.sum(H64 * H64, axis=1)
    np.testing.assert_allclose(P.sum(0), ss, rtol=2e-6, atol=1e-6)
    # each partial covers its own 64 columns
    for t in range(T):
        cols = slice(64 * t, min(64 * t + 64, wl.D))
        np.testing.assert_allclose(P[t], np.sum(H64[:, cols] ** 2, axis=1), rtol=2e-6, atol=1e-6)
    r_host = 1.0 / np.sqrt(P.sum(0) / wl.D + wl.eps)
    np.testing.assert_allclose(o["r"].cpu().numpy(), r_host, rtol=1e-6)


def test_tiny_fp32_workload():
    wl = ci.WORKLOADS["tiny-fp32"]
    o = _run(wl)
    err, ref_err = _check_against_oracle(wl, o)
    _check_stages(wl, o)
    print(f"tiny-fp32: fused {err:.2e}, unfused {ref_err:.2e}")


SHAPES = [
    (1, 64, 256, 256),
    (3, 136, 264, 520),
    (257, 256, 512, 768),
    (300, 512, 384, 1032),
    (513, 1024, 1024, 2048),
    (1000, 2048, 768, 1536),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_and_unfused_match_oracle(shape, dtype):
    M, K, D, N2 = shape
    wl = ci.custom_workload(M, K, D, N2, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=200)
    o = _run(wl, seed=1)
    _check_against_oracle(wl, o)
    _check_stages(wl, o)


def test_repeatable_and_overwrites_poison():
    wl = ci.custom_workload(300, 512, 512, 1024, wl_id=201)
    o = _run(wl, seed=2, ref=False)
    d = o["d"]
    H = torch.full_like(o["H"], float("nan"))
    Hg = torch.full_like(o["Hg"], float("nan"))
    P = torch.full_like(o["P"], float("nan"))
    r = torch.full_like(o["r"], float("nan"))
    Y = torch.full_like(o["Y"], float("nan"))
    coda.coda_gemm_res_prms(d["A"], d["W1"], d["R"], d["g"], H, Hg, P)
    coda.coda_rms_combine(P, r, wl.D, wl.eps)
    coda.coda_gemm_rowscale(Hg, d["W2"], r, Y)
    torch.cuda.synchronize()
    for a, b in ((H, o["H"]), (Hg, o["Hg"]), (Y, o["Y"])):
        assert np.array_equal(host_bits(a), host_bits(b))
    assert torch.equal(P, o["P"]) and torch.equal(r, o["r"])


def test_zero_rows_and_constant_rows():
    # rows of A and R set to zero give H = 0, r = 1/sqrt(eps), Y = 0;
    # A = 0 with constant R rows gives the oracle's closed form
    wl = ci.custom_workload(64, 256, 256, 512, wl_id=202)
    x = ci.make_inputs(wl, seed=3)
    x["A"].bits[5] = 0
    x["R"].bits[5] = 0
    x["A"].bits[9] = 0
    x["R"].bits[9] = ci.bf16_bits(np.full(256, 1.5, np.float32))
    for k in ("A", "R"):
        x[k].f32 = ci.bf16_bits_to_f32(x[k].bits)
    d = {k: dev(v) for k, v in x.items()}
    H, Hg, r, Y, P = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    torch.cuda.synchronize()
    rr = r.cpu().numpy()
    assert rr[5] == pytest.approx(1.0 / np.sqrt(wl.eps), rel=1e-6)
    assert np.all(host_f32(Y)[5] == 0.0)
    assert rr[9] == pytest.approx(1.0 / np.sqrt(1.5 ** 2 + wl.eps), rel=1e-6)
    orc = oracle.forward(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps)
    assert max_rel(host_f32(Y), orc["Y"]) <= 1e-2


def test_strided_leading_dimensions():
    # every matrix a column slice of a wider allocation (ld > width)
    M, K, D, N2 = 260, 256, 384, 640
    wl = ci.custom_workload(M, K, D, N2, wl_id=203)
    x = ci.make_inputs(wl, seed=4)
    d = {k: dev(v) for k, v in x.items()}

    def wide(t, extra=24):
        w = torch.zeros((t.shape[0], t.shape[1] + extra), device=t.device, dtype=t.dtype)
        w[:, :t.shape[1]] = t
        return w[:, :t.shape[1]]

    A, W1, R, W2 = wide(d["A"]), wide(d["W1"]), wide(d["R"]), wide(d["W2"])
    H = wide(torch.empty((M, D), device="cuda", dtype=torch.bfloat16), 8)
    Hg = wide(torch.empty((M, D), device="cuda", dtype=torch.bfloat16), 16)
    Y = wide(torch.empty((M, N2), device="cuda", dtype=torch.bfloat16), 40)
    P = torch.empty((coda.coda_prms_num_partials(torch.bfloat16, D), M), device="cuda")
    r = torch.empty((M,), device="cuda")
    coda.coda_gemm_res_prms(A, W1, R, d["g"], H, Hg, P)
    coda.coda_rms_combine(P, r, D, wl.eps)
    coda.coda_gemm_rowscale(Hg, W2, r, Y)
    H0, Hg0, r0, Y0, P0 = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(H.contiguous()), host_bits(H0))
    assert np.array_equal(host_bits(Y.contiguous()), host_bits(Y0))
    assert torch.equal(r, r0)


def test_rowscale_without_r_is_plain_gemm():
    M, D, N2 = 200, 512, 768
    wl = ci.custom_workload(M, 8, D, N2, wl_id=204)
    x = ci.make_inputs(wl, seed=5)
    X = dev(x["R"])
    W2 = dev(x["W2"])
    Y = torch.empty((M, N2), device="cuda", dtype=torch.bfloat16)
    coda.coda_gemm_rowscale(X, W2, None, Y)
    torch.cuda.synchronize()
    ref = x["R"].f64() @ x["W2"].f64()
    assert max_rel(host_f32(Y), ref) <= 4e-3


FULL = ["1b-bf16", "7b-bf16", "70b-bf16"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_tensor(name):
    # the full workloads in the benchmark's launch configuration, fused and
    # unfused, against the oracle over every row (computed in row blocks)
    wl = ci.WORKLOADS[name]
    o = _run(wl, seed=0, ref=True)
    x = o["x"]
    Hr, rr, Yr = o["ref"]
    assert torch.equal(Hr.view(torch.int16), o["H"].view(torch.int16)), "fused H differs from the unfused chain's H"

    W1, g, W2 = x["W1"].f64(), x["g"].f64(), x["W2"].f64()   # converted once, not per block

    def orc(rows):
        ref = oracle.forward(x["A"].f32, W1, x["R"].f32, g, W2, wl.eps, rows=rows)
        # the unfused chain's Y is compared with the same reference Y; r as a column
        return {"Y": ref["Y"], "Yref": ref["Y"], "H": ref["H"], "r": ref["r"][:, None]}

    def check(rows, ref, host):
        np.testing.assert_allclose(host["H"], ref["H"], rtol=2.0 ** -8 * 1.01, atol=1e-5)
        np.testing.assert_allclose(host["r"], ref["r"], rtol=2e-3)

    errs = whole_max_rel(orc, {"Y": o["Y"], "Yref": Yr, "H": o["H"], "r": o["r"][:, None]}, wl.M, check=check)
    print(f"{name}: whole-tensor Y error fused {errs['Y']:.3e}, unfused {errs['Yref']:.3e}",
          file=sys.__stderr__, flush=True)
    assert errs["Y"] <= 1e-2 and errs["Yref"] <= 1e-2
    _comparable(errs["Y"], errs["Yref"], wl.dtype)
    # whole-tensor property: r * RMS(H_stored) == 1 up to eps
    H = o["H"].float()
    ms = (H * H).mean(dim=1)
    rrms = o["r"] * torch.sqrt(ms)
    expect = torch.sqrt(ms / (ms + wl.eps))
    assert torch.max(torch.abs(rrms - expect)).item() < 1e-5


@pytest.mark.slow
def test_largest_matrix_spans():
    # A [32768, 32760] and Y [32768, 32760] each span 2,146,959,360 bytes, just
    # under the 2 GiB - 256 limit of one matrix: the direct loads address A
    # with 32-bit offsets up to the top of that range, and the contraction
    # (32760 = 1023 k-tiles + 24) and Y's columns (127 tiles + 248) both end
    # ragged.  Every row against the oracle.
    M, K, D, N2 = 32768, 32760, 256, 32760
    wl = ci.custom_workload(M, K, D, N2, wl_id=130)
    assert M * K * 2 <= 2 ** 31 - 256 and M * N2 * 2 <= 2 ** 31 - 256
    o = _run(wl, seed=3, ref=False)
    x = o["x"]
    W1, g, W2 = x["W1"].f64(), x["g"].f64(), x["W2"].f64()

    def orc(rows):
        ref = oracle.forward(x["A"].f32, W1, x["R"].f32, g, W2, wl.eps, rows=rows)
        return {"Y": ref["Y"], "H": ref["H"]}

    errs = whole_max_rel(orc, {"Y": o["Y"], "H": o["H"]}, M)
    print(f"largest spans: whole-tensor Y error {errs['Y']:.3e}, H error {errs['H']:.3e}", file=sys.__stderr__,
          flush=True)
    assert errs["Y"] <= 1e-2 and errs["H"] <= 2.0 ** -8
