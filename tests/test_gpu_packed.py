"""GPU parity of the forward pair with the Hg intermediate tile-packed
(coda_gemm_res_prms_packed + coda_rms_combine + coda_gemm_rowscale_packed).

The packed pair computes exactly what the row-major pair computes: H,
partials, r and Y must be bit-identical to coda_gemm_res_prms +
coda_gemm_rowscale on the same inputs, and the packed Hg must hold exactly
the row-major Hg, permuted (element (i, 8c + e) at bfloat16 index
((i/16 * D/8 + c) * 16 + i%16) * 8 + e).  Y is also checked against the fp64
oracle (the plain chain of the CODA news article by Synced, epilogue
section) with the bf16 bar of 1e-2.  Shapes include ragged M (padding rows
in the last block), D not a multiple of the 32-column k-tile, and the full
7B workload in the benchmark's launch configuration (every row against the
oracle).  The same bit-identity holds for the other second GEMMs on the
packed Hg (SwiGLU, the LM head with the cross-entropy statistics and its
backward, the QKV projection with RoPE) and for the fp8 chain with both
second-GEMM operands packed; each is also checked against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import coda_inputs as ci
import oracle
import transformer_gemm_epilogue_gemm1_amd as coda
from tests.gpu_util import dev, host_bits, host_f32, max_rel, whole_max_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
    torch.cuda.synchronize()


def _both(wl, seed):
    x = ci.make_inputs(wl, seed=seed)
    d = {k: dev(v) for k, v in x.items()}
    row = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    pk = coda.fused_forward_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    torch.cuda.synchronize()
    return x, row, pk


def _same(a, b, what):
    assert np.array_equal(host_bits(a) if a.dtype == torch.bfloat16 else a.cpu().numpy().view(np.uint32),
                          host_bits(b) if b.dtype == torch.bfloat16 else b.cpu().numpy().view(np.uint32)), \
        f"{what} differs between the packed and the row-major pair"


def _index_check(Hgp, Hg, M, D):
    # the documented index formula, element by element on the host
    flat = host_bits(Hgp).reshape(-1)
    ref = host_bits(Hg)
    i = np.arange(M)[:, None]
    col = np.arange(D)[None, :]
    idx = ((i // 16 * (D // 8) + col // 8) * 16 + i % 16) * 8 + col % 8
    np.testing.assert_array_equal(flat[idx], ref)


SHAPES = [(256, 256, 256, 512), (300, 256, 512, 768), (1, 64, 72, 40), (33, 96, 40, 264), (513, 320, 328, 600)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_packed_pair_matches_row_major_and_oracle(shape):
    M, K, D, N2 = shape
    wl = ci.custom_workload(M, K, D, N2, eps=1e-5, dtype="bf16", wl_id=700 + M % 97)
    x, (H, Hg, r, Y, P), (Hp, Hgp, rp, Yp, Pp) = _both(wl, seed=5)
    _same(H, Hp, "H")
    _same(P, Pp, "partials")
    _same(r, rp, "r")
    _same(Y, Yp, "Y")
    assert tuple(Hgp.shape) == ((M + 15) // 16, D // 8, 16, 8)
    _index_check(Hgp, Hg, M, D)
    assert torch.equal(coda.unpack(Hgp, M).view(torch.int16), Hg.view(torch.int16))
    orc = oracle.forward(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps)
    err = max_rel(host_f32(Yp), orc["Y"])
    print(f"{shape}: packed Y error {err:.3e}")
    assert err <= 1e-2


def test_packed_rowscale_without_r_and_strided_y():
    # r = NULL (plain GEMM) and a Y with ldy > N2, against the row-major kernel
    M, D, N2 = 200, 256, 304
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    X = torch.randn((M, D), device="cuda", generator=g).to(torch.bfloat16)
    W2 = (torch.randn((D, N2), device="cuda", generator=g) * D ** -0.5).to(torch.bfloat16)
    Xp = coda.packed_empty(M, D, "cuda")
    Xp.copy_(torch.nn.functional.pad(X, (0, 0, 0, (-M) % 16)).reshape(-1, 16, D // 8, 8).permute(0, 2, 1, 3))
    assert torch.equal(coda.unpack(Xp, M), X)
    Yb = torch.full((M, N2 + 40), float("nan"), device="cuda", dtype=torch.bfloat16)
    Yp = Yb[:, :N2]
    Yr = torch.empty((M, N2), device="cuda", dtype=torch.bfloat16)
    coda.coda_gemm_rowscale(X, W2, None, Yr)
    lib = coda._lib.load()
    st = lib.coda_gemm_rowscale_packed(M, D, N2, Xp.data_ptr(), W2.data_ptr(), N2, None, Yp.data_ptr(), N2 + 40,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(Yp.view(torch.int16), Yr.view(torch.int16))
    assert torch.isnan(Yb[:, N2:].float()).all()  # the padding columns are not written


def test_packed_repeatable():
    wl = ci.custom_workload(300, 256, 512, 768, eps=1e-5, dtype="bf16", wl_id=790)
    x = ci.make_inputs(wl, seed=2)
    d = {k: dev(v) for k, v in x.items()}
    a = coda.fused_forward_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    b = coda.fused_forward_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    torch.cuda.synchronize()
    # the packed Hg is compared on its M rows: the last block's padding rows
    # are never written
    a = list(a)
    b = list(b)
    a[1], b[1] = coda.unpack(a[1], wl.M), coda.unpack(b[1], wl.M)
    for t, u in zip(a, b):
        assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t,
                           u.view(torch.int16) if u.dtype == torch.bfloat16 else u)


@pytest.mark.slow
def test_full_size_7b_packed_whole_tensor():
    # the benchmark's workload and launch configuration; Y bit-identical to
    # the row-major pair, and every row against the oracle
    wl = ci.WORKLOADS["7b-bf16"]
    x, (H, Hg, r, Y, P), (Hp, Hgp, rp, Yp, Pp) = _both(wl, seed=0)
    _same(H, Hp, "H")
    _same(r, rp, "r")
    _same(Y, Yp, "Y")
    assert torch.equal(coda.unpack(Hgp, wl.M).view(torch.int16), Hg.view(torch.int16))
    W1, g, W2 = x["W1"].f64(), x["g"].f64(), x["W2"].f64()

    def orc(rows):
        return {"Y": oracle.forward(x["A"].f32, W1, x["R"].f32, g, W2, wl.eps, rows=rows)["Y"]}

    err = whole_max_rel(orc, {"Y": Yp}, wl.M)["Y"]
    print(f"7b packed whole-tensor Y error {err:.3e}", file=sys.__stderr__, flush=True)
    assert err <= 1e-2


# ---- fp8: Hg8 and W2t8 tile-packed ----
def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


FP8_SHAPES = [(1, 64, 256, 256), (3, 144, 272, 528), (300, 512, 384, 1040), (513, 1024, 1024, 2048)]


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_packed_chain_matches_row_major_and_oracle(shape):
    M, K, D, N2 = shape
    wl = ci.custom_workload(M, K, D, N2, dtype="fp8", wl_id=520)
    x = ci.make_inputs_fp8(wl, seed=3)
    d = {"A8": _u8(x["A8"]), "sa": _f32(x["sa"]), "W1t8": _u8(x["W1t8"]), "sw1": _f32(x["sw1"]),
         "W2t8": _u8(x["W2t8"]), "sw2": _f32(x["sw2"]), "R": dev(x["R"]), "g": dev(x["g"])}
    H, Hg8, E, r, Y, P = coda.fused_forward_fp8(d["A8"], d["sa"], d["W1t8"], d["sw1"], d["R"], d["g"], d["W2t8"],
                                                d["sw2"], wl.eps)
    # the packed weight codes: the row-major codes permuted
    W2p = coda.packed_empty_e4m3(N2, D, "cuda")
    W2p.copy_(torch.nn.functional.pad(d["W2t8"], (0, 0, 0, (-N2) % 16)).reshape(-1, 16, D // 16, 16)
              .permute(0, 2, 1, 3))
    Hp, Hg8p, Ep, rp, Yp, Pp = coda.fused_forward_fp8_packed(d["A8"], d["sa"], d["W1t8"], d["sw1"], d["R"], d["g"],
                                                             W2p, d["sw2"], wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(coda.unpack_e4m3(Hg8p, M), Hg8)
    assert torch.equal(Ep, E)
    _same(H, Hp, "H")
    _same(P, Pp, "partials")
    _same(r, rp, "r")
    _same(Y, Yp, "Y")
    orc = oracle.forward_fp8(x["A8"], x["sa"], x["W1t8"], x["sw1"], x["R"].f32, x["g"].f32, x["W2t8"], x["sw2"],
                             wl.eps)
    err = max_rel(host_f32(Yp), orc["Y"])
    print(f"{shape}: fp8 packed Y error {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("KN", [(256, 512), (4096, 272), (64, 16)], ids=lambda s: "x".join(map(str, s)))
def test_quantize_weight_packed_is_the_row_major_codes_permuted(KN):
    K, N = KN
    g = torch.Generator(device="cuda")
    g.manual_seed(K + N)
    W = (torch.randn((K, N), device="cuda", generator=g) * K ** -0.5).to(torch.bfloat16)
    Wt8, s = coda.quantize_weight_e4m3(W)
    Wt8p, sp = coda.quantize_weight_e4m3_packed(W)
    torch.cuda.synchronize()
    assert torch.equal(s, sp)
    assert torch.equal(coda.unpack_e4m3(Wt8p, N), Wt8)


@pytest.mark.slow
def test_full_size_7b_fp8_packed():
    # the 7B fp8 workload in the benchmark's configuration: quantised on the
    # device, packed and row-major chains bit-identical
    M, K, D, N2 = 16384, 4096, 4096, 28672
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    A = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    W1 = (torch.randn((K, D), device="cuda", generator=g) * K ** -0.5).to(torch.bfloat16)
    W2 = (torch.randn((D, N2), device="cuda", generator=g) * D ** -0.5).to(torch.bfloat16)
    R = torch.randn((M, D), device="cuda", generator=g).to(torch.bfloat16)
    gg = (1.0 + 0.1 * torch.randn((D,), device="cuda", generator=g)).to(torch.bfloat16)
    A8, sa = coda.quantize_rows_e4m3(A)
    W1t8, sw1 = coda.quantize_weight_e4m3(W1)
    W2t8, sw2 = coda.quantize_weight_e4m3(W2)
    W2t8p, sw2p = coda.quantize_weight_e4m3_packed(W2)
    H, Hg8, E, r, Y, P = coda.fused_forward_fp8(A8, sa, W1t8, sw1, R, gg, W2t8, sw2, 1e-5)
    Hp, Hg8p, Ep, rp, Yp, Pp = coda.fused_forward_fp8_packed(A8, sa, W1t8, sw1, R, gg, W2t8p, sw2p, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(coda.unpack_e4m3(W2t8p, N2), W2t8)
    assert torch.equal(coda.unpack_e4m3(Hg8p, M), Hg8)
    assert torch.equal(Ep, E)
    _same(Y, Yp, "Y")


# ---- SwiGLU second GEMM on the tile-packed Hg ----
@pytest.mark.parametrize("shape", [(300, 256, 512, 768), (33, 96, 40, 320), (513, 320, 328, 640)],
                         ids=lambda s: "x".join(map(str, s)))
def test_swiglu_packed_matches_row_major(shape):
    M, K, D, N2 = shape
    wl = ci.custom_workload(M, K, D, N2, eps=1e-5, dtype="bf16", wl_id=740)
    x = ci.make_inputs(wl, seed=9)
    d = {k: dev(v) for k, v in x.items()}
    H, Hg, r, Z, Y = coda.fused_forward_swiglu(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, keep_y=True)
    Hp, Hgp, rp, Zp, Yp = coda.fused_forward_swiglu_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps,
                                                           keep_y=True)
    _, _, _, Zn, _ = coda.fused_forward_swiglu_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
    torch.cuda.synchronize()
    _same(r, rp, "r")
    _same(Z, Zp, "Z")
    _same(Y, Yp, "Y (pre-activation)")
    _same(Z, Zn, "Z without Y")
    # Z against the oracle of the gated chain
    orc = oracle.forward_swiglu(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps)
    err = max_rel(host_f32(Zp), orc["Z"])
    print(f"{shape}: packed SwiGLU Z error {err:.3e}")
    assert err <= 1e-2


# ---- the LM-head (cross-entropy) and QKV (RoPE) second GEMMs on the packed Hg ----
CE_SHAPES = [(3, 136, 264, 520), (257, 256, 512, 1000), (300, 512, 384, 2056)]  # M, K, D, V


def _ce_pair(wl, seed):
    x = ci.make_inputs(wl, seed=seed)
    t = ci.make_targets(wl, seed=seed)
    d = {k: dev(v) for k, v in x.items()}
    tt = torch.from_numpy(t).cuda()
    row = coda.fused_forward_ce(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tt)
    pk = coda.fused_forward_ce_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tt)
    torch.cuda.synchronize()
    return x, d, t, tt, row, pk


@pytest.mark.parametrize("shape", CE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ce_packed_matches_row_major_and_oracle(shape):
    wl = ci.custom_workload(*shape, eps=1e-5, dtype="bf16", wl_id=750)
    x, d, t, tt, (H, Hg, r, lse, loss), (Hp, Hgp, rp, lsep, lossp) = _ce_pair(wl, seed=3)
    _same(lse, lsep, "lse")
    _same(loss, lossp, "loss")
    orc = oracle.forward_ce(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, t)
    err = max_rel(lossp.cpu().numpy(), orc["loss"])
    print(f"{shape}: packed CE loss error {err:.3e}")
    assert err <= 1e-2
    # backward: dY from the packed Hg equals the row-major one bit for bit,
    # and every gradient meets the oracle's bar
    dl = np.random.default_rng(5).standard_normal(wl.M).astype(np.float32)
    tdl = torch.from_numpy(dl).cuda()
    g_row = coda.fused_backward_ce(d["A"], d["W1"], d["g"], d["W2"], H, Hg, r, tt, lse, tdl)
    g_pk = coda.fused_backward_ce_packed(d["A"], d["W1"], d["g"], d["W2"], Hp, Hgp, rp, tt, lsep, tdl)
    torch.cuda.synchronize()
    _same(g_row[-1], g_pk[-1], "dY")
    orc_b = oracle.backward_ce(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, t, dl)
    for k, v in zip(("dA", "dR", "dW1", "dW2", "dg", "dY"), g_pk):
        err = max_rel(host_f32(v), orc_b[k])
        assert err <= 1e-2, f"{k}: error {err:.3e}"


ROPE_SHAPES = [  # M, K, D, N2, n_q, n_k, d_head
    (3, 136, 264, 520, 256, 128, 64),
    (300, 512, 384, 1040, 512, 256, 64),
    (130, 128, 256, 264, 128, 64, 8),
]


def _positions(M, max_pos, seed):
    p = np.random.default_rng(seed).integers(0, max_pos, size=M).astype(np.int32)
    p[: min(M, 3)] = [0, max_pos - 1, max_pos // 2][: min(M, 3)]
    return p


@pytest.mark.parametrize("shape", ROPE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_rope_packed_matches_row_major_and_oracle(shape):
    M, K, D, N2, nq, nk, dh = shape
    wl = ci.custom_workload(M, K, D, N2, eps=1e-5, dtype="bf16", wl_id=760)
    x = ci.make_inputs(wl, seed=6)
    d = {k: dev(v) for k, v in x.items()}
    pos = _positions(M, 4096, 6)
    tp = torch.from_numpy(pos).cuda()
    cs = coda.rope_cache(4096, dh, 10000.0)
    _, _, r, Y = coda.fused_forward_rope(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tp, cs, nq, nk, dh)
    _, _, rp, Yp = coda.fused_forward_rope_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tp, cs, nq, nk,
                                                  dh)
    torch.cuda.synchronize()
    _same(Y, Yp, "Y")
    orc = oracle.forward_rope(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, pos, nq, nk, dh,
                              10000.0)
    err = max_rel(host_f32(Yp), orc["Yr"])
    print(f"{shape}: packed RoPE Y error {err:.3e}")
    assert err <= 1e-2


@pytest.mark.slow
def test_full_size_7b_ce_and_qkv_packed():
    # the LM-head and QKV workloads at full size: the packed calls equal the
    # row-major ones bit for bit (loss, lse, dY; rotated Y)
    wl = ci.WORKLOADS["7b-ce-bf16"]
    x, d, t, tt, (H, Hg, r, lse, loss), (Hp, Hgp, rp, lsep, lossp) = _ce_pair(wl, seed=0)
    _same(lse, lsep, "lse")
    _same(loss, lossp, "loss")
    assert torch.isfinite(lossp).all().item()
    tdl = torch.full((wl.M,), 1.0 / wl.M, device="cuda", dtype=torch.float32)
    dY = torch.empty((wl.M, wl.N2), device="cuda", dtype=torch.bfloat16)
    dYp = torch.empty_like(dY)
    coda.coda_gemm_rowscale_ce_bwd(Hg, d["W2"], r, tt, lse, tdl, dY)
    coda.coda_gemm_rowscale_ce_bwd_packed(Hgp, d["W2"], rp, tt, lsep, tdl, dYp)
    torch.cuda.synchronize()
    _same(dY, dYp, "dY")
    del dY, dYp, d, x
    wl = ci.WORKLOADS["7b-rope-bf16"]
    x = ci.make_inputs(wl, seed=0)
    d = {k: dev(v) for k, v in x.items()}
    tp = torch.from_numpy(ci.make_positions(wl)).cuda()
    cs = coda.rope_cache(2048, 128, 10000.0)
    _, _, _, Y = coda.fused_forward_rope(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tp, cs, 4096, 4096, 128)
    _, _, _, Yp = coda.fused_forward_rope_packed(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tp, cs, 4096,
                                                 4096, 128)
    torch.cuda.synchronize()
    _same(Y, Yp, "Y")
