"""Pins for the fp64 CPU oracle of the chain ending in a per-token
cross-entropy (CPU only).

The pages name the cross-entropy loss among the operations the
re-parameterisation covers and the tile log-sum-exp and online max/sum-exp
statistics among the epilogue building blocks (CODA news article by Synced,
epilogue and building-block sections); they do not write the loss out.  The
oracle takes the standard per-token loss lse(Y_i) - Y_i,t_i.  Pins: scipy's
logsumexp and torch's cross_entropy (library routines), a pure-Python brute
force, closed forms and invariances, and planted mistakes.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import coda_inputs as ci
import oracle


def _case(seed, M, K, D, V):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, K)), rng.standard_normal((K, D)) / np.sqrt(K), rng.standard_normal((M, D)),
            1.0 + 0.1 * rng.standard_normal(D), rng.standard_normal((D, V)) / np.sqrt(D),
            rng.integers(0, V, size=M))


@pytest.mark.parametrize("shape", [(1, 4, 8, 5), (6, 8, 16, 33), (17, 16, 8, 300)])
def test_matches_scipy_and_torch(shape):
    A, W1, R, g, Wv, t = _case(sum(shape), *shape)
    out = oracle.forward_ce(A, W1, R, g, Wv, 1e-5, t)
    np.testing.assert_allclose(out["lse"], scipy.special.logsumexp(out["Y"], axis=1), rtol=1e-14)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(out["Y"]), torch.from_numpy(t), reduction="none")
    np.testing.assert_allclose(out["loss"], ref.numpy(), rtol=1e-13, atol=1e-14)


def test_brute_force():
    A, W1, R, g, Wv, t = _case(3, 3, 4, 8, 6)
    out = oracle.forward_ce(A, W1, R, g, Wv, 0.25, t)
    for i in range(3):
        row = [float(v) for v in out["Y"][i]]
        lse = math.log(math.fsum(math.exp(v) for v in row))
        assert out["loss"][i] == pytest.approx(lse - row[int(t[i])], rel=1e-13, abs=1e-14)


def test_closed_forms_and_invariances():
    V = 37
    Y = np.zeros((3, V))
    t = np.array([0, 5, 36])
    out = oracle.cross_entropy_rows(Y, t)                      # equal logits: loss = log V
    np.testing.assert_allclose(out["loss"], np.log(V), rtol=1e-15)
    rng = np.random.default_rng(4)
    Y = rng.standard_normal((5, V)) * 3
    t = rng.integers(0, V, size=5)
    base = oracle.cross_entropy_rows(Y, t)["loss"]
    c = rng.standard_normal((5, 1)) * 50                         # a per-row shift leaves the loss unchanged
    np.testing.assert_allclose(oracle.cross_entropy_rows(Y + c, t)["loss"], base, rtol=1e-12, atol=1e-12)
    perm = rng.permutation(V)                                    # relabelling classes consistently
    inv = np.argsort(perm)
    np.testing.assert_allclose(oracle.cross_entropy_rows(Y[:, perm], inv[t])["loss"], base, rtol=1e-13)
    big = np.array([[1000.0, 0.0, -1000.0]])                     # no overflow: the max is factored out
    assert oracle.cross_entropy_rows(big, [0])["loss"][0] == pytest.approx(0.0, abs=1e-300)
    assert np.all(base > 0)


def test_targets_in_range_and_seeded():
    wl = ci.custom_workload(1000, 8, 16, 300, wl_id=9)
    t = ci.make_targets(wl, seed=1)
    assert t.dtype == np.int32 and t.min() >= 0 and t.max() < 300
    assert np.array_equal(t, ci.make_targets(wl, seed=1)) and not np.array_equal(t, ci.make_targets(wl, seed=2))
    with pytest.raises(ValueError):
        oracle.cross_entropy_rows(np.zeros((2, 3)), [0, 3])


@pytest.mark.parametrize("kind", ["no_max_factor", "mean_not_sum", "wrong_target_index", "sign"])
def test_pins_reject_planted_mistakes(kind):
    rng = np.random.default_rng(6)
    Y = rng.standard_normal((4, 9)) * 2
    t = rng.integers(0, 9, size=4)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(Y), torch.from_numpy(t), reduction="none").numpy()
    m = Y.max(axis=1)
    if kind == "no_max_factor":
        bad = np.log(np.sum(np.exp(Y - m[:, None]), axis=1)) - Y[np.arange(4), t]   # forgot to add m back
    elif kind == "mean_not_sum":
        bad = m + np.log(np.mean(np.exp(Y - m[:, None]), axis=1)) - Y[np.arange(4), t]
    elif kind == "wrong_target_index":
        bad = oracle.logsumexp_rows(Y) - Y[np.arange(4), (t + 1) % 9]
    else:
        bad = Y[np.arange(4), t] - oracle.logsumexp_rows(Y)
    assert np.max(np.abs(bad - ref)) > 1e-3


def test_grad_matches_torch_autograd_and_sums_to_zero():
    rng = np.random.default_rng(7)
    Y = rng.standard_normal((6, 40)) * 3
    t = rng.integers(0, 40, size=6)
    dl = rng.standard_normal(6)
    got = oracle.cross_entropy_grad(Y, t, dl)
    y = torch.from_numpy(Y).requires_grad_(True)
    loss = torch.nn.functional.cross_entropy(y, torch.from_numpy(t), reduction="none")
    (loss * torch.from_numpy(dl)).sum().backward()
    np.testing.assert_allclose(got, y.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(got.sum(axis=1), 0.0, atol=1e-14)          # softmax and one-hot both sum to 1
    big = np.array([[1000.0, 0.0, -1000.0]])                              # no overflow
    np.testing.assert_allclose(oracle.cross_entropy_grad(big, [0], [1.0]), [[0.0, 0.0, 0.0]], atol=1e-300)


def test_chain_backward_against_finite_differences():
    # d(sum_i dloss_i loss_i) / dW, through the whole chain, by central
    # differences of the forward oracle on a tiny case
    A, W1, R, g, Wv, t = _case(8, 3, 4, 8, 7)
    dl = np.array([0.5, -1.0, 2.0])
    out = oracle.backward_ce(A, W1, R, g, Wv, 1e-5, t, dl)

    def f(**kw):
        args = dict(A=A, W1=W1, R=R, g=g, Wv=Wv)
        args.update(kw)
        o = oracle.forward_ce(args["A"], args["W1"], args["R"], args["g"], args["Wv"], 1e-5, t)
        return float(np.sum(dl * o["loss"]))

    h = 1e-6
    for name, arr, grad in (("Wv", Wv, out["dW2"]), ("W1", W1, out["dW1"]), ("A", A, out["dA"]),
                            ("R", R, out["dR"]), ("g", g, out["dg"])):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            up, dn = arr.copy(), arr.copy()
            up[idx] += h
            dn[idx] -= h
            num[idx] = (f(**{name: up}) - f(**{name: dn})) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("kind", ["no_onehot", "sign", "unscaled", "softmax_over_rows"])
def test_grad_pins_reject_planted_mistakes(kind):
    rng = np.random.default_rng(9)
    Y = rng.standard_normal((5, 8)) * 2
    t = rng.integers(0, 8, size=5)
    dl = rng.standard_normal(5) + 2.0
    y = torch.from_numpy(Y).requires_grad_(True)
    (torch.nn.functional.cross_entropy(y, torch.from_numpy(t), reduction="none") * torch.from_numpy(dl)).sum().backward()
    ref = y.grad.numpy()
    p = np.exp(Y - oracle.logsumexp_rows(Y)[:, None])
    if kind == "softmax_over_rows":
        p = np.exp(Y) / np.exp(Y).sum(axis=0, keepdims=True)
    bad = p.copy()
    if kind != "no_onehot":
        bad[np.arange(5), t] -= 1.0
    bad = -bad if kind == "sign" else bad
    if kind != "unscaled":
        bad = bad * dl[:, None]
    assert np.max(np.abs(bad - ref)) > 1e-3
