"""GPU parity of the chain ending in the LM head and the per-token
cross-entropy (coda_gemm_rowscale_lse + coda_ce_combine) and of its backward
(coda_gemm_rowscale_ce_bwd, then coda_chain_bwd) through the C ABI.

The logits are never written: the second GEMM's epilogue keeps per-tile
max / sum-exp statistics and the target logit, a combine turns them into
lse and loss.  Compared with the fp64 oracle (oracle/ce.py) on the same
seeded inputs and targets: max|x - x_ref| / max|x_ref| <= 1e-2 (bf16) or
1e-5 (fp32) for lse and loss.  Stage-wise (fp32, where the LM-head GEMM with
a row scale stores exactly the y the statistics see): pmax and the target
logit bit-exact against the host on coda_gemm_rowscale's output, psum to
fp32 rounding.  Backward: dY and every chain gradient against the oracle
(same bars); in fp32 dY against the host formula on the same logits and lse.
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


def _run(wl, seed, targets=None):
    x = ci.make_inputs(wl, seed=seed)
    t = ci.make_targets(wl, seed=seed) if targets is None else np.asarray(targets, dtype=np.int32)
    d = {k: dev(v) for k, v in x.items()}
    tt = torch.from_numpy(t).cuda()
    H, Hg, r, lse, loss = coda.fused_forward_ce(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps, tt)
    torch.cuda.synchronize()
    return x, d, t, tt, {"H": H, "Hg": Hg, "r": r, "lse": lse, "loss": loss}


def _check(wl, x, t, o, rows=None):
    orc = oracle.forward_ce(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, t, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    for k in ("lse", "loss"):
        err = max_rel(o[k].cpu().numpy()[sel], orc[k])
        assert err <= tolerance(wl.dtype), f"{k} error {err:.3e}"
    return max_rel(o["loss"].cpu().numpy()[sel], orc["loss"])


SHAPES = [  # M, K, D, V (V ragged against the 256-column tiles)
    (1, 64, 256, 256),
    (3, 136, 264, 520),
    (257, 256, 512, 1000),
    (300, 512, 384, 2056),
    (513, 1024, 1024, 4096),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ce_chain_matches_oracle(shape, dtype):
    wl = ci.custom_workload(*shape, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=600)
    x, d, t, tt, o = _run(wl, seed=1)
    _check(wl, x, t, o)


def test_statistics_against_the_logits_fp32():
    M, K, D, V = 300, 256, 384, 1000
    wl = ci.custom_workload(M, K, D, V, eps=1e-6, dtype="f32", wl_id=601)
    # targets on tile and chunk edges
    t = (np.arange(M) * 37) % V
    t[:6] = [0, 7, 8, 63, 64, V - 1]
    x, d, t, tt, o = _run(wl, seed=2, targets=t)
    Hg = torch.empty((M, D), device="cuda")
    P = torch.empty((coda.coda_prms_num_partials(torch.float32, D), M), device="cuda")
    H = torch.empty_like(Hg)
    r = torch.empty((M,), device="cuda")
    coda.coda_gemm_res_prms(d["A"], d["W1"], d["R"], d["g"], H, Hg, P)
    coda.coda_rms_combine(P, r, D, wl.eps)
    Y = torch.empty((M, V), device="cuda")
    coda.coda_gemm_rowscale(Hg, d["W2"], r, Y)
    T = coda.coda_prms_num_partials(torch.float32, V)
    pmax = torch.full((T, M), float("nan"), device="cuda")
    psum = torch.full_like(pmax, float("nan"))
    tgt = torch.full((M,), float("nan"), device="cuda")
    coda.coda_gemm_rowscale_lse(Hg, d["W2"], r, tt, pmax, psum, tgt)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    pm, ps = pmax.cpu().numpy(), psum.cpu().numpy()
    for ti in range(T):
        cols = slice(64 * ti, min(64 * ti + 64, V))
        if 64 * ti >= V:
            assert np.all(pm[ti] == -np.inf) and np.all(ps[ti] == 0.0)
            continue
        np.testing.assert_array_equal(pm[ti], y[:, cols].max(axis=1))
        ref = np.sum(np.exp(y[:, cols].astype(np.float64) - pm[ti][:, None]), axis=1)
        np.testing.assert_allclose(ps[ti], ref, rtol=2e-6)
    np.testing.assert_array_equal(tgt.cpu().numpy(), y[np.arange(M), t])


def test_invalid_target_gives_nan_only_there():
    wl = ci.custom_workload(64, 128, 256, 512, wl_id=602)
    t = ci.make_targets(wl, seed=3)
    t[5] = -1
    t[9] = 512
    x, d, t, tt, o = _run(wl, seed=3, targets=t)
    loss = o["loss"].cpu().numpy()
    assert np.isnan(loss[5]) and np.isnan(loss[9])
    ok = np.ones(64, bool)
    ok[[5, 9]] = False
    assert np.isfinite(loss[ok]).all()
    orc = oracle.forward_ce(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps,
                            np.where(ok, t, 0))
    assert max_rel(loss[ok], orc["loss"][ok]) <= 1e-2


@pytest.mark.slow
def test_full_size_7b_lm_head_whole_tensor():
    # lse and the per-token loss of every row against the oracle
    wl = ci.WORKLOADS["7b-ce-bf16"]
    x, d, t, tt, o = _run(wl, seed=0)
    W1, g, W2 = x["W1"].f64(), x["g"].f64(), x["W2"].f64()

    def orc(rows):
        ref = oracle.forward_ce(x["A"].f32, W1, x["R"].f32, g, W2, wl.eps, t, rows=rows)
        return {"lse": ref["lse"], "loss": ref["loss"]}

    errs = whole_max_rel(orc, {"lse": o["lse"], "loss": o["loss"]}, wl.M)
    print(f"7b-ce whole-tensor lse error {errs['lse']:.3e}, loss error {errs['loss']:.3e}", file=sys.__stderr__,
          flush=True)
    assert errs["lse"] <= 1e-2 and errs["loss"] <= 1e-2


GRADS = ("dA", "dR", "dW1", "dW2", "dg")


def _dloss(M, seed):
    return np.random.default_rng(seed + 1000).standard_normal(M).astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES[1:], ids=lambda s: "x".join(map(str, s)))
def test_ce_backward_matches_oracle(shape, dtype):
    wl = ci.custom_workload(*shape, eps=1e-5 if dtype == "bf16" else 1e-6, dtype=dtype, wl_id=610)
    x, d, t, tt, o = _run(wl, seed=4)
    dl = _dloss(wl.M, 4)
    tdl = torch.from_numpy(dl).cuda()
    grads = coda.fused_backward_ce(d["A"], d["W1"], d["g"], d["W2"], o["H"], o["Hg"], o["r"], tt, o["lse"], tdl)
    torch.cuda.synchronize()
    out = dict(zip(GRADS + ("dY",), grads))
    orc = oracle.backward_ce(x["A"].f32, x["W1"].f32, x["R"].f32, x["g"].f32, x["W2"].f32, wl.eps, t, dl)
    for k in GRADS + ("dY",):
        err = max_rel(host_f32(out[k]), orc[k])
        assert err <= tolerance(dtype), f"{k}: error {err:.3e}"


def test_ce_grad_against_the_logits_fp32():
    M, K, D, V = 300, 256, 384, 1000
    wl = ci.custom_workload(M, K, D, V, eps=1e-6, dtype="f32", wl_id=611)
    t = (np.arange(M) * 37) % V
    t[:6] = [0, 7, 8, 63, 64, V - 1]
    x, d, t, tt, o = _run(wl, seed=5, targets=t)
    dl = _dloss(M, 5)
    dY = torch.full((M, V), float("nan"), device="cuda")
    coda.coda_gemm_rowscale_ce_bwd(o["Hg"], d["W2"], o["r"], tt, o["lse"], torch.from_numpy(dl).cuda(), dY)
    Y = torch.empty((M, V), device="cuda")
    coda.coda_gemm_rowscale(o["Hg"], d["W2"], o["r"], Y)
    torch.cuda.synchronize()
    y = host_f32(Y).astype(np.float64)
    lse = o["lse"].cpu().numpy().astype(np.float64)
    ref = np.exp(y - lse[:, None])
    ref[np.arange(M), t] -= 1.0
    ref *= dl[:, None]
    got = host_f32(dY)
    # the exponential of the same y, in fp32 with the hardware exp2: a few
    # float32 roundings of |dloss| (e^(y - lse) + 1)
    bound = 4e-6 * np.abs(dl)[:, None] * (np.exp(y - lse[:, None]) + 1.0)
    assert np.all(np.abs(got - ref) <= bound)
    np.testing.assert_allclose(got.sum(axis=1), 0.0, atol=1e-5 * np.abs(dl).max())


def test_ce_grad_invalid_target_gives_nan_row():
    wl = ci.custom_workload(64, 128, 256, 512, wl_id=612)
    t = ci.make_targets(wl, seed=6)
    t[3], t[40] = -5, 512
    x, d, t, tt, o = _run(wl, seed=6, targets=t)
    dY = torch.empty((64, 512), device="cuda", dtype=torch.bfloat16)
    coda.coda_gemm_rowscale_ce_bwd(o["Hg"], d["W2"], o["r"], tt, o["lse"], torch.ones(64, device="cuda"), dY)
    torch.cuda.synchronize()
    g = host_f32(dY)
    assert np.isnan(g[[3, 40]]).all()
    ok = np.ones(64, bool)
    ok[[3, 40]] = False
    assert np.isfinite(g[ok]).all()


@pytest.mark.slow
def test_full_size_7b_lm_head_grad_whole_tensor():
    # the logits' gradient dY = dloss (softmax - onehot) of every row
    wl = ci.WORKLOADS["7b-ce-bf16"]
    x, d, t, tt, o = _run(wl, seed=0)
    dl = np.full(wl.M, 1.0 / wl.M, dtype=np.float32)
    dY = torch.empty((wl.M, wl.N2), device="cuda", dtype=torch.bfloat16)
    coda.coda_gemm_rowscale_ce_bwd(o["Hg"], d["W2"], o["r"], tt, o["lse"], torch.from_numpy(dl).cuda(), dY)
    torch.cuda.synchronize()
    W1, g, W2 = x["W1"].f64(), x["g"].f64(), x["W2"].f64()

    def orc(rows):
        Yo = oracle.forward(x["A"].f32, W1, x["R"].f32, g, W2, wl.eps, rows=rows)["Y"]
        return {"dY": oracle.cross_entropy_grad(Yo, t[rows], dl[rows])}

    def check(rows, ref, host):   # each row of the gradient sums to zero
        assert np.all(np.abs(host["dY"].sum(axis=1)) <= 1e-2 / wl.M)

    err = whole_max_rel(orc, {"dY": dY}, wl.M, check=check)["dY"]
    print(f"7b-ce whole-tensor dY error {err:.3e}", file=sys.__stderr__, flush=True)
    assert err <= 1e-2
