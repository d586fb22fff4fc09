"""GPU parity of the chain whose second GEMM is the QKV projection with the
rotary embedding in its epilogue (coda_rope_cache, coda_gemm_rowscale_rope,
coda_rope_bwd) through the C ABI.

Compared with the fp64 oracle (oracle/rope.py) on the same seeded inputs:
  * the table: within one float32 ulp of the fp64 cos / sin;
  * Y (rotated [Q | K | V]): max|Y - Y_ref| / max|Y_ref| <= 1e-2 (bf16) or
    1e-5 (fp32);
  * stage-wise (fp32): the epilogue against the host rotation, with the GPU's
    own table, of coda_gemm_rowscale's output (the same y), to a few float32
    roundings; V columns bit-identical;
  * invalid positions: NaN in that row's Q and K columns only;
  * backward: against the oracle's transpose rotation, and the rotation undone.
"""
import sys

import numpy as np
import pytest
import torch

import coda_inputs as ci
import oracle
import transformer_gemm_epilogue_gemm1_amd as coda
from tests.gpu_util import dev, host_f32, max_rel, tolerance, whole_max_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
    torch.cuda.synchronize()


def _positions(M, max_pos, seed):
    rng = np.random.default_rng(seed)
    p = rng.integers(0, max_pos, size=M).astype(np.int32)
    p[: min(M, 4)] = [0, 1, max_pos - 1, max_pos // 2][: min(M, 4)]
    return p


@pytest.mark.parametrize("d_head,base,max_pos", [(128, 10000.0, 4096), (64, 500000.0, 1000), (8, 10000.0, 33)])
def test_rope_cache_matches_fp64(d_head, base, max_pos):
    cs = coda.rope_cache(max_pos, d_head, base)
    torch.cuda.synchronize()
    got = cs.cpu().numpy().astype(np.float64)
    ang = oracle.rope_angles(np.arange(max_pos), d_head, base)
    for k, ref in ((0, np.cos(ang)), (1, np.sin(ang))):
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got[:, :, k] - ref) <= ulp), f"component {k} off by more than an ulp"


def _run(wl, seed, nq, nk, d_head, base, max_pos, positions=None):
    x = ci.make_inputs(wl, seed=seed)
    d = {k: dev(v) for k, v in x.items()}
    pos = _positions(wl.M, max_pos, seed) if positions is None else np.asarray(positions, dtype=np.int32)
    tp = torch.from_numpy(pos).cuda()
    cs = coda.rope_cache(max_pos, d_head, base)
    H, Hg, r, Y = coda.fused_forward_rope(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tp, cs, nq, nk, d_head)
    torch.cuda.synchronize()
    return x, d, pos, tp, cs, {"H": H, "Hg": Hg, "r": r, "Y": Y}


SHAPES = [  # M, K, D, N2, n_q, n_k, d_head
    (1, 64, 256, 384, 128, 128, 128),
    (3, 136, 264, 520, 256, 128, 64),        # ragged N2 with a ragged V part
    (257, 256, 512, 768, 256, 256, 128),
    (300, 512, 384, 1040, 512, 256, 64),     # grouped keys (fewer K heads)
    (513, 1024, 1024, 1536, 1024, 256, 128),
    (130, 128, 256, 264, 128, 64, 8),        # the smallest head width
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_rope_chain_matches_oracle(shape, dtype):
    M, K, D, N2, nq, nk, dh = shape
    wl = ci.custom_workload(M, K, D, N2, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=700)
    x, d, pos, tp, cs, o = _run(wl, 1, nq, nk, dh, 10000.0, 4096)
    orc = oracle.forward_rope(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, pos, nq, nk, dh,
                              10000.0)
    err = max_rel(host_f32(o["Y"]), orc["Yr"])
    assert err <= tolerance(dtype), f"Y error {err:.3e}"


def test_epilogue_against_host_rotation_fp32():
    M, K, D, N2, nq, nk, dh = 300, 256, 384, 1040, 512, 256, 64
    wl = ci.custom_workload(M, K, D, N2, eps=1e-6, dtype="f32", wl_id=701)
    x, d, pos, tp, cs, o = _run(wl, 2, nq, nk, dh, 10000.0, 2048)
    Y0 = torch.empty((M, N2), device="cuda")
    coda.coda_gemm_rowscale(o["Hg"], d["W2"], o["r"], Y0)
    torch.cuda.synchronize()
    y = host_f32(Y0)
    t = cs.cpu().numpy()[pos]  # [M, dh/2, 2]
    got = host_f32(o["Y"])
    np.testing.assert_array_equal(got[:, nq + nk:], y[:, nq + nk:])
    for h in range(0, nq + nk, dh):
        e, od = y[:, h:h + dh:2], y[:, h + 1:h + dh:2]
        c, s = t[:, :, 0], t[:, :, 1]
        # a few float32 roundings of the two products' magnitudes (the kernel
        # may fuse one product into the add)
        for k, ref, scale in ((0, e * c - od * s, np.abs(e * c) + np.abs(od * s)),
                              (1, e * s + od * c, np.abs(e * s) + np.abs(od * c))):
            np.testing.assert_array_less(np.abs(got[:, h + k:h + dh:2] - ref), 4e-7 * scale + 1e-30)


def test_invalid_positions_give_nan_in_q_and_k_only():
    M, K, D, N2, nq, nk, dh = 64, 128, 256, 768, 256, 256, 128
    wl = ci.custom_workload(M, K, D, N2, wl_id=702)
    pos = _positions(M, 512, 3)
    pos[5], pos[9] = -1, 512
    x, d, pos, tp, cs, o = _run(wl, 3, nq, nk, dh, 10000.0, 512, positions=pos)
    y = host_f32(o["Y"])
    assert np.isnan(y[[5, 9], : nq + nk]).all()
    assert np.isfinite(y[[5, 9], nq + nk:]).all()
    ok = np.ones(M, bool)
    ok[[5, 9]] = False
    assert np.isfinite(y[ok]).all()
    orc = oracle.forward_rope(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps,
                              np.where(ok, pos, 0), nq, nk, dh, 10000.0)
    assert max_rel(y[ok], orc["Yr"][ok]) <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_bwd_matches_oracle(dtype):
    M, N2, nq, nk, dh, max_pos = 300, 1040, 512, 256, 64, 2048
    rng = np.random.default_rng(4)
    G = rng.standard_normal((M, N2)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.from_numpy(G).cuda().to(tdt)
    pos = _positions(M, max_pos, 4)
    tp = torch.from_numpy(pos).cuda()
    cs = coda.rope_cache(max_pos, dh, 10000.0)
    dY = torch.full_like(g, float("nan"))
    coda.coda_rope_bwd(g, tp, cs, nq, nk, dh, dY)
    torch.cuda.synchronize()
    ref = oracle.rope_backward(host_f32(g), pos, nq, nk, dh, 10000.0)
    assert max_rel(host_f32(dY), ref) <= tolerance(dtype)
    assert torch.equal(dY[:, nq + nk:], g[:, nq + nk:])
    if dtype == "f32":
        # the backward undoes the forward rotation of the epilogue
        wl = ci.custom_workload(M, 256, 384, N2, eps=1e-6, dtype="f32", wl_id=703)
        x, d, pos2, tp2, cs2, o = _run(wl, 5, nq, nk, dh, 10000.0, max_pos, positions=pos)
        back = torch.empty_like(o["Y"])
        coda.coda_rope_bwd(o["Y"], tp, cs, nq, nk, dh, back)
        Y0 = torch.empty_like(o["Y"])
        coda.coda_gemm_rowscale(o["Hg"], d["W2"], o["r"], Y0)
        torch.cuda.synchronize()
        assert max_rel(host_f32(back), host_f32(Y0).astype(np.float64)) <= 1e-6


@pytest.mark.slow
def test_full_size_7b_qkv_whole_tensor():
    # the rotated QKV projection of every row against the oracle
    wl = ci.WORKLOADS["7b-rope-bf16"]
    nq = nk = 4096
    pos = ci.make_positions(wl)
    x, d, pos, tp, cs, o = _run(wl, 0, nq, nk, 128, 10000.0, 2048, positions=pos)
    W1, g, W2 = x["W1"].f64(), x["g"].f64(), x["W2"].f64()

    def orc(rows):
        return {"Y": oracle.forward_rope(x["A"].f32, W1, x["R"].f32, g, W2, wl.eps, pos, nq, nk, 128, 10000.0,
                                         rows=rows)["Yr"]}

    err = whole_max_rel(orc, {"Y": o["Y"]}, wl.M)["Y"]
    print(f"7b-qkv whole-tensor Y error {err:.3e}", file=sys.__stderr__, flush=True)
    assert err <= 1e-2