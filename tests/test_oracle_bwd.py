"""Pins for the fp64 CPU oracle of the chain's backward (CPU only).

The pages state that the RMSNorm re-parameterisation carries over to the
backward pass (CODA news article by Synced, epilogue section) but print no
formula; the oracle differentiates the plain forward step by step.  It is
pinned by torch's own autograd in float64 (a library routine), by central
finite differences of the pinned forward, and by Euler identities that follow
from the homogeneity of the chain.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(seed, M, K, D, N2):
    rng = np.random.default_rng(seed)
    return dict(
        A=rng.standard_normal((M, K)), W1=rng.standard_normal((K, D)) / np.sqrt(K),
        R=rng.standard_normal((M, D)), g=1.0 + 0.1 * rng.standard_normal(D),
        W2=rng.standard_normal((D, N2)) / np.sqrt(D), dY=rng.standard_normal((M, N2)))


def _loss(c, eps):
    return float(np.sum(c["dY"] * oracle.forward(c["A"], c["W1"], c["R"], c["g"], c["W2"], eps)["Y"]))


@pytest.mark.parametrize("shape", [(1, 4, 4, 6), (5, 8, 4, 6), (7, 6, 16, 9), (33, 16, 24, 40)])
@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.3])
def test_matches_torch_autograd(shape, eps):
    c = _case(sum(shape), *shape)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dY")) for k, v in c.items()}
    H = t["A"] @ t["W1"] + t["R"]
    Xn = torch.nn.functional.rms_norm(H, (H.shape[1],), t["g"], eps)
    Y = Xn @ t["W2"]
    (Y * t["dY"]).sum().backward()
    out = oracle.backward(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], eps)
    for name, key in (("dA", "A"), ("dR", "R"), ("dW1", "W1"), ("dW2", "W2"), ("dg", "g")):
        np.testing.assert_allclose(out[name], t[key].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("eps", [1e-5, 0.5])
def test_central_differences(eps):
    c = _case(4, 3, 5, 6, 4)
    out = oracle.backward(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], eps)
    rng = np.random.default_rng(0)
    h = 1e-6
    for name, key in (("dA", "A"), ("dR", "R"), ("dW1", "W1"), ("dW2", "W2"), ("dg", "g")):
        for _ in range(6):
            idx = tuple(rng.integers(0, n) for n in c[key].shape)
            cp = {k: v.copy() for k, v in c.items()}
            cm = {k: v.copy() for k, v in c.items()}
            cp[key][idx] += h
            cm[key][idx] -= h
            fd = (_loss(cp, eps) - _loss(cm, eps)) / (2 * h)
            assert out[name][idx] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, idx)


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.2])
def test_euler_identities(eps):
    c = _case(21, 9, 12, 16, 10)
    out = oracle.backward(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], eps)
    Y = oracle.forward(c["A"], c["W1"], c["R"], c["g"], c["W2"], eps)["Y"]
    L = np.sum(c["dY"] * Y)
    # Y is linear in W2 and in g
    assert np.sum(out["dW2"] * c["W2"]) == pytest.approx(L, rel=1e-12)
    assert np.sum(out["dg"] * c["g"]) == pytest.approx(L, rel=1e-12)
    # H depends on W1 only through the linear term A W1
    assert np.sum(out["dW1"] * c["W1"]) == pytest.approx(np.sum(out["dH"] * (c["A"] @ c["W1"])), rel=1e-12)
    # dR is dH exactly
    np.testing.assert_array_equal(out["dR"], out["dH"])
    # row-wise <dH_i, H_i> = eps r_i^3 s_i (zero at eps = 0: degree-0 homogeneity)
    H = c["A"] @ c["W1"] + c["R"]
    lhs = np.sum(out["dH"] * H, axis=1)
    np.testing.assert_allclose(lhs, eps * out["r"] ** 3 * out["s"], rtol=1e-9, atol=1e-12)
    if eps == 0.0:
        tot = np.sum(out["dA"] * c["A"]) + np.sum(out["dR"] * c["R"])
        assert abs(tot) <= 1e-12 * np.sum(np.abs(out["dR"] * c["R"]))
