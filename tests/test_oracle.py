"""Pins for the fp64 CPU oracle of the forward chain (CPU only).

The oracle is the plain definition of the GEMM-RMSNorm-GEMM pattern (CODA news
article by Synced, epilogue section): H = A W1 + R, r = 1/sqrt(mean(H^2)+eps),
Y = diag(r) H diag(g) W2.  The pages print no worked numbers, so the pins are:
a hand-worked example with exact rationals, an independent pure-Python brute
force, closed forms, invariants and library special cases.  The last test
plants plausible mistakes into copies of the chain and shows that the pins
reject every one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac(x):
    return float(Fraction(x))


def _golden():
    with open(os.path.join(GOLDEN, "fwd_hand_example.json")) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _case(rng, M, K, D, N2):
    return (_rand(rng, M, K), _rand(rng, K, D) / np.sqrt(K), _rand(rng, M, D),
            1.0 + 0.1 * _rand(rng, D), _rand(rng, D, N2) / np.sqrt(D))


def test_hand_worked_example():
    gd = _golden()
    out = oracle.forward(gd["A"], gd["W1"], gd["R"], gd["g"], gd["W2"], gd["eps"])
    np.testing.assert_allclose(out["H"], [[_frac(v) for v in row] for row in gd["H"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["r"], [_frac(v) for v in gd["r"]], rtol=1e-15, atol=0)
    np.testing.assert_allclose(out["Y"], [[_frac(v) for v in row] for row in gd["Y"]], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("M", [1, 3, 5])
@pytest.mark.parametrize("K,D", [(4, 4), (4, 8), (8, 4)])
@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.7])
def test_brute_force(M, K, D, eps):
    rng = np.random.default_rng(1000 * M + 10 * K + D)
    A, W1, R, g, W2 = _case(rng, M, K, D, 6)
    H, r, Y = brute_force.chain(A.tolist(), W1.tolist(), R.tolist(), g.tolist(), W2.tolist(), eps)
    out = oracle.forward(A, W1, R, g, W2, eps)
    np.testing.assert_allclose(out["H"], H, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out["r"], r, rtol=1e-13)
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.25])
def test_constant_rows_closed_form(eps):
    # A = 0 and R_i = c_i * 1: H_i = c_i * 1, mean square c_i^2,
    # r_i = 1/sqrt(c_i^2 + eps), Y_i = c_i r_i (g @ W2).
    rng = np.random.default_rng(7)
    M, K, D, N2 = 6, 5, 12, 7
    c = np.array([1.0, -2.0, 0.5, 3.0, -0.25, 7.0])
    g = 1.0 + 0.1 * rng.standard_normal(D)
    W2 = rng.standard_normal((D, N2))
    out = oracle.forward(np.zeros((M, K)), rng.standard_normal((K, D)),
                         c[:, None] * np.ones((M, D)), g, W2, eps)
    r_exp = 1.0 / np.sqrt(c * c + eps)
    np.testing.assert_allclose(out["r"], r_exp, rtol=1e-15)
    np.testing.assert_allclose(out["Y"], (c * r_exp)[:, None] * (g @ W2)[None, :], rtol=1e-13, atol=1e-14)
    if eps == 0.0:  # g = 1: Y_i = sign(c_i) * colsum(W2)
        out1 = oracle.forward(np.zeros((M, K)), np.eye(K, D), c[:, None] * np.ones((M, D)), np.ones(D), W2, 0.0)
        np.testing.assert_allclose(out1["Y"], np.sign(c)[:, None] * W2.sum(0)[None, :], rtol=1e-13, atol=1e-13)


def test_zero_rows():
    # an all-zero row of H gives r = 1/sqrt(eps) (finite) and a zero row of Y
    rng = np.random.default_rng(3)
    A, W1, R, g, W2 = _case(rng, 4, 8, 8, 5)
    A[2] = 0.0
    R[2] = 0.0
    out = oracle.forward(A, W1, R, g, W2, 1e-5)
    assert out["r"][2] == pytest.approx(1.0 / np.sqrt(1e-5), rel=1e-15)
    assert np.all(out["Y"][2] == 0.0)


def test_r_times_rms():
    rng = np.random.default_rng(11)
    A, W1, R, g, W2 = _case(rng, 9, 16, 24, 8)
    for eps in (0.0, 1e-5, 0.3):
        out = oracle.forward(A, W1, R, g, W2, eps)
        rms = np.sqrt(np.mean(out["H"] ** 2, axis=1))
        ms = rms ** 2
        np.testing.assert_allclose(out["r"] * rms, np.sqrt(ms / (ms + eps)), rtol=1e-14)
        if eps == 0.0:
            np.testing.assert_allclose(out["r"] * rms, 1.0, rtol=1e-14)


def test_deferred_row_scale_equals_normalise_then_multiply():
    # the re-association the fused path relies on (epilogue section of the
    # article): scaling the rows of (H diag(g)) W2 by r afterwards gives the
    # normalise-then-multiply result; brute-force sums in exact rationals on
    # a tiny case, so neither side shares the oracle's matmul
    rng = np.random.default_rng(21)
    A, W1, R, g, W2 = _case(rng, 3, 4, 5, 2)
    eps = 0.25
    out = oracle.forward(A, W1, R, g, W2, eps)
    H = [[Fraction(v) for v in row] for row in out["H"]]
    r = [Fraction(v) for v in out["r"]]
    gq = [Fraction(v) for v in g]
    W2q = [[Fraction(v) for v in row] for row in W2]
    for i in range(3):
        for k in range(2):
            deferred = r[i] * sum(H[i][j] * gq[j] * W2q[j][k] for j in range(5))
            normalised = sum((r[i] * H[i][j] * gq[j]) * W2q[j][k] for j in range(5))
            assert deferred == normalised
            assert float(deferred) == pytest.approx(out["Y"][i, k], rel=1e-13, abs=1e-15)


def test_constant_rows_with_unit_weight():
    # g = 1 and a row of H constant c: r = 1/sqrt(c^2 + eps) and the
    # normalised row is c r (1, ..., 1), so Y_i = c r (column sums of W2)
    rng = np.random.default_rng(22)
    M, K, D, N2 = 4, 8, 16, 6
    A = np.zeros((M, K))
    W1 = rng.standard_normal((K, D))
    R = np.repeat(np.array([[2.0], [-0.5], [0.0], [7.0]]), D, axis=1)
    W2 = rng.standard_normal((D, N2))
    eps = 1e-3
    out = oracle.forward(A, W1, R, np.ones(D), W2, eps)
    c = R[:, 0]
    r = 1.0 / np.sqrt(c * c + eps)
    np.testing.assert_allclose(out["r"], r, rtol=1e-15)
    np.testing.assert_allclose(out["Y"], (c * r)[:, None] * W2.sum(axis=0)[None, :], rtol=1e-13, atol=1e-15)


def test_scale_invariance_and_row_permutation():
    rng = np.random.default_rng(5)
    A, W1, R, g, W2 = _case(rng, 7, 8, 16, 9)
    base = oracle.forward(A, W1, R, g, W2, 0.0)
    for alpha in (0.01, 3.0, 1e4):
        s = oracle.forward(alpha * A, W1, alpha * R, g, W2, 0.0)
        np.testing.assert_allclose(s["Y"], base["Y"], rtol=1e-12, atol=1e-13)
    perm = rng.permutation(7)
    p = oracle.forward(A[perm], W1, R[perm], g, W2, 0.0)
    np.testing.assert_allclose(p["Y"], base["Y"][perm], rtol=1e-14, atol=1e-15)


def test_row_subset_is_exact():
    rng = np.random.default_rng(6)
    A, W1, R, g, W2 = _case(rng, 40, 8, 16, 9)
    full = oracle.forward(A, W1, R, g, W2, 1e-5, block_rows=7)
    rows = [39, 0, 17, 17, 5]
    sub = oracle.forward(A, W1, R, g, W2, 1e-5, rows=rows, block_rows=2)
    # identical up to BLAS blocking order (a few ulp), never a different row
    for name in ("H", "r", "Y"):
        np.testing.assert_allclose(sub[name], full[name][rows], rtol=1e-13, atol=1e-15)


def test_identity_weights_reduce_to_torch_rms_norm():
    # W1 = I, W2 = I: Y = RMSNorm(A + R; g, eps) by torch's own rms_norm
    rng = np.random.default_rng(8)
    M, D = 11, 32
    A = rng.standard_normal((M, D))
    R = rng.standard_normal((M, D))
    g = 1.0 + 0.1 * rng.standard_normal(D)
    for eps in (1e-6, 1e-5, 0.5):
        out = oracle.forward(A, np.eye(D), R, g, np.eye(D), eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(A + R), (D,), torch.from_numpy(g), eps).numpy()
        np.testing.assert_allclose(out["Y"], ref, rtol=1e-13, atol=1e-14)


def test_unit_rms_rows_reduce_to_plain_matmuls():
    # R = 0, eps = 0 and A W1 with rows of mean square exactly 1 (A of +-1,
    # W1 a signed permutation): r = 1, so Y = (A W1) diag(g) W2 by numpy.matmul.
    rng = np.random.default_rng(9)
    M, D, N2 = 6, 16, 10
    A = rng.choice([-1.0, 1.0], size=(M, D))
    W1 = np.eye(D)[rng.permutation(D)] * rng.choice([-1.0, 1.0], size=(D, 1))
    g = 1.0 + 0.1 * rng.standard_normal(D)
    W2 = rng.standard_normal((D, N2))
    out = oracle.forward(A, W1, np.zeros((M, D)), g, W2, 0.0)
    np.testing.assert_allclose(out["r"], 1.0, rtol=1e-15)
    np.testing.assert_allclose(out["Y"], np.matmul(np.matmul(A, W1) * g, W2), rtol=1e-13, atol=1e-14)


# ---- the pins have power: plausible mistakes planted in copies of the chain ----

def _mutant(kind, A, W1, R, g, W2, eps):
    A, W1, R, g, W2 = (np.asarray(x, dtype=np.float64) for x in (A, W1, R, g, W2))
    D = W1.shape[1]
    H = A @ W1 + (0.0 if kind == "drop_residual" else R)
    if kind == "residual_sign":
        H = A @ W1 - R
    ms = np.sum(H * H, 1) if kind == "sum_not_mean" else np.mean(H * H, 1)
    if kind == "mean_over_wrong_axis":
        ms = np.mean(H * H, 0)[: H.shape[0]] if H.shape[0] <= D else np.resize(np.mean(H * H, 0), H.shape[0])
    r = 1.0 / (np.sqrt(ms) + eps) if kind == "eps_outside_sqrt" else 1.0 / np.sqrt(ms + eps)
    if kind == "rms_not_inverse":
        r = np.sqrt(ms + eps)
    gg = 1.0 + g if kind == "one_plus_g" else g
    if kind == "drop_g":
        gg = np.ones_like(g)
    Xn = H * r[:, None] * gg[None, :]
    if kind == "w2_transposed_view":
        # reading W2 with the wrong leading dimension (a flat reinterpretation)
        Y = Xn @ W2.reshape(-1)[: D * W2.shape[1]].reshape(W2.shape[1], D).T
    else:
        Y = Xn @ W2
    if kind == "scale_columns":
        Y = Xn @ (W2 * np.resize(r, W2.shape[1])[None, :])
    return H, r, Y


MUTATIONS = ["drop_residual", "residual_sign", "sum_not_mean", "mean_over_wrong_axis",
             "eps_outside_sqrt", "rms_not_inverse", "one_plus_g", "drop_g",
             "w2_transposed_view", "scale_columns"]


@pytest.mark.parametrize("kind", MUTATIONS)
def test_pins_reject_planted_mistakes(kind):
    gd = _golden()
    H, r, Y = _mutant(kind, gd["A"], gd["W1"], gd["R"], gd["g"], gd["W2"], gd["eps"])
    y_ref = np.array([[_frac(v) for v in row] for row in gd["Y"]])
    golden_ok = np.allclose(Y, y_ref, rtol=1e-12, atol=1e-12)
    rng = np.random.default_rng(2)
    A, W1, R, g, W2 = _case(rng, 3, 4, 8, 6)
    _, _, Yb = brute_force.chain(A.tolist(), W1.tolist(), R.tolist(), g.tolist(), W2.tolist(), 1e-5)
    _, _, Ym = _mutant(kind, A, W1, R, g, W2, 1e-5)
    brute_ok = np.allclose(Ym, Yb, rtol=1e-10, atol=1e-12)
    assert not (golden_ok and brute_ok), f"mutation {kind} slipped through both pins"
