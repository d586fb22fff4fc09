"""Pins for the fp64 CPU oracle of the chain with a SwiGLU epilogue (CPU only).

The pages name SwiGLU among the epilogue compositions the re-parameterisation
covers (CODA news article by Synced, epilogue and results sections) without
writing it out; the oracle takes the LLaMA gate Z = silu(Y_gate) * Y_up over
W2 = [W_gate | W_up].  Pins: an independent pure-Python brute force, torch's
own silu and autograd in float64 (library routines), closed forms of silu,
central differences, and planted mistakes that the brute force rejects.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import brute_force


def _case(seed, M, K, D, F):
    rng = np.random.default_rng(seed)
    return dict(A=rng.standard_normal((M, K)), W1=rng.standard_normal((K, D)) / np.sqrt(K),
                R=rng.standard_normal((M, D)), g=1.0 + 0.1 * rng.standard_normal(D),
                W2=rng.standard_normal((D, 2 * F)) / np.sqrt(D), dZ=rng.standard_normal((M, F)))


def _brute_swiglu(A, W1, R, g, W2, eps):
    _, _, Y = brute_force.chain(A.tolist(), W1.tolist(), R.tolist(), g.tolist(), W2.tolist(), eps)
    F = len(Y[0]) // 2
    return [[Y[i][j] / (1.0 + math.exp(-Y[i][j])) * Y[i][F + j] for j in range(F)] for i in range(len(Y))]


@pytest.mark.parametrize("shape", [(1, 4, 4, 3), (3, 8, 4, 5), (5, 4, 8, 2)])
@pytest.mark.parametrize("eps", [1e-5, 0.25])
def test_brute_force(shape, eps):
    c = _case(sum(shape), *shape)
    out = oracle.forward_swiglu(c["A"], c["W1"], c["R"], c["g"], c["W2"], eps)
    ref = np.array(_brute_swiglu(c["A"], c["W1"], c["R"], c["g"], c["W2"], eps))
    np.testing.assert_allclose(out["Z"], ref, rtol=1e-12, atol=1e-14)


def test_silu_is_torch_silu_and_its_closed_forms():
    x = np.concatenate([np.linspace(-40, 40, 801), [0.0, -745.0, 745.0, 1e-300]])
    s = oracle.silu(x)
    np.testing.assert_allclose(s, torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(s - oracle.silu(-x), x, rtol=1e-13, atol=1e-13)   # silu(x) - silu(-x) = x
    assert s[801] == 0.0 and np.isfinite(s).all()
    assert s[802] == pytest.approx(0.0, abs=1e-300) and s[803] == 745.0


def test_zero_gate_or_up_columns_give_zero():
    c = _case(3, 6, 8, 16, 5)
    W2 = c["W2"].copy()
    W2[:, :5] = 0.0        # gate columns
    z = oracle.forward_swiglu(c["A"], c["W1"], c["R"], c["g"], W2, 1e-5)["Z"]
    assert np.all(z == 0.0)
    W2 = c["W2"].copy()
    W2[:, 5:] = 0.0        # up columns
    z = oracle.forward_swiglu(c["A"], c["W1"], c["R"], c["g"], W2, 1e-5)["Z"]
    assert np.all(z == 0.0)


def test_large_gate_is_linear():
    # silu(x) = x (1 - e^-x / (1 + e^-x)) = x exactly in float64 for x > 40:
    # gate columns scaled up so that rows with Y_gate > 50 give Z = Y_gate * Y_up
    c = _case(4, 8, 8, 8, 3)
    W2 = c["W2"].copy()
    W2[:, :3] *= 1e3
    out = oracle.forward_swiglu(c["A"], c["W1"], c["R"], c["g"], W2, 1e-5)
    yg, yu = out["Y"][:, :3], out["Y"][:, 3:]
    big = yg > 50.0
    assert big.sum() >= 3
    np.testing.assert_array_equal(out["Z"][big], (yg * yu)[big])
    small = yg < -50.0   # and silu(x) -> 0 for x << 0
    assert small.sum() >= 3
    np.testing.assert_allclose(out["Z"][small], 0.0, atol=1e-18 * np.abs(yu).max())


@pytest.mark.parametrize("shape", [(1, 4, 4, 3), (5, 8, 4, 6), (9, 6, 16, 4)])
@pytest.mark.parametrize("eps", [1e-5, 0.3])
def test_backward_matches_torch_autograd(shape, eps):
    c = _case(10 + sum(shape), *shape)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dZ")) for k, v in c.items()}
    H = t["A"] @ t["W1"] + t["R"]
    Y = torch.nn.functional.rms_norm(H, (H.shape[1],), t["g"], eps) @ t["W2"]
    F = Y.shape[1] // 2
    Z = torch.nn.functional.silu(Y[:, :F]) * Y[:, F:]
    (Z * t["dZ"]).sum().backward()
    out = oracle.backward_swiglu(c["dZ"], c["A"], c["W1"], c["R"], c["g"], c["W2"], eps)
    for name, key in (("dA", "A"), ("dR", "R"), ("dW1", "W1"), ("dW2", "W2"), ("dg", "g")):
        np.testing.assert_allclose(out[name], t[key].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_dy_by_central_differences():
    # dL/dY of L = <dZ, Z(Y)> elementwise, by central differences in Y
    rng = np.random.default_rng(12)
    Y = rng.standard_normal((3, 8)) * 2.0
    dZ = rng.standard_normal((3, 4))

    def L(Yv):
        F = Yv.shape[1] // 2
        return float(np.sum(dZ * oracle.silu(Yv[:, :F]) * Yv[:, F:]))

    dY = oracle.swiglu_dy(dZ, Y)
    h = 1e-6
    for i in range(3):
        for j in range(8):
            e = np.zeros_like(Y)
            e[i, j] = h
            assert (L(Y + e) - L(Y - e)) / (2 * h) == pytest.approx(dY[i, j], rel=1e-7, abs=1e-9)


def _mutant(kind, Y):
    F = Y.shape[1] // 2
    yg, yu = Y[:, :F], Y[:, F:]
    if kind == "gate_up_swapped":
        return oracle.silu(yu) * yg
    if kind == "sigmoid_not_silu":
        return 1.0 / (1.0 + np.exp(-yg)) * yu
    if kind == "no_gate":
        return yg * yu
    if kind == "interleaved_halves":
        return oracle.silu(Y[:, 0::2]) * Y[:, 1::2]
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["gate_up_swapped", "sigmoid_not_silu", "no_gate", "interleaved_halves"])
def test_brute_force_rejects_planted_mistakes(kind):
    c = _case(7, 3, 8, 4, 5)
    Y = oracle.forward(c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5)["Y"]
    ref = np.array(_brute_swiglu(c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5))
    assert np.max(np.abs(_mutant(kind, Y) - ref)) > 1e-3
