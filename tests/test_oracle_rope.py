"""Pins for the fp64 CPU oracle of the QKV projection with RoPE (CPU only).

The pages name RoPE among the element-wise epilogue transforms the
re-parameterisation covers (CODA news article by Synced, epilogue and
building-block sections) without writing it out; the oracle takes the
rotary embedding in its interleaved form (oracle/rope.py).  Pins: numpy's
complex multiplication (the rotation as (y_2i + i y_2i+1) e^(i p theta_i)),
closed forms (position 0 is the identity, pair norms are kept, V untouched),
the relative-position identity <R(q, m), R(k, n)> = <R(q, m - n), k>, a
pure-Python brute force, and planted mistakes.
"""
import math

import numpy as np
import pytest

import coda_inputs as ci
import oracle


def _y(seed, M, N):
    return np.random.default_rng(seed).standard_normal((M, N))


def test_complex_form():
    d, nq, nk = 16, 32, 16
    Y = _y(1, 5, nq + nk + 16)
    pos = np.array([0, 1, 7, 1000, 4095])
    out = oracle.rope_rotate(Y, pos, nq, nk, d, 10000.0)
    theta = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    for h in range(0, nq + nk, d):
        z = Y[:, h:h + d:2] + 1j * Y[:, h + 1:h + d:2]
        z = z * np.exp(1j * pos[:, None] * theta[None, :])
        np.testing.assert_allclose(out[:, h:h + d:2], z.real, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(out[:, h + 1:h + d:2], z.imag, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(out[:, nq + nk:], Y[:, nq + nk:])


def test_identity_at_zero_and_norms_kept():
    Y = _y(2, 4, 64)
    out = oracle.rope_rotate(Y, np.zeros(4), 32, 16, 8, 500000.0)
    np.testing.assert_array_equal(out, Y)
    out = oracle.rope_rotate(Y, np.array([3, 9, 27, 81]), 32, 16, 8, 500000.0)
    np.testing.assert_allclose(out[:, 0:48:2] ** 2 + out[:, 1:48:2] ** 2, Y[:, 0:48:2] ** 2 + Y[:, 1:48:2] ** 2,
                               rtol=1e-13)


def test_relative_position_identity():
    d = 32
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    for m, n in ((5, 2), (100, 37), (2047, 0)):
        lhs = np.sum(oracle.rope_rotate(q, [m], d, 0, d, 10000.0) * oracle.rope_rotate(k, [n], d, 0, d, 10000.0))
        rhs = np.sum(oracle.rope_rotate(q, [m - n], d, 0, d, 10000.0) * k)
        assert lhs == pytest.approx(rhs, rel=1e-11, abs=1e-11)


def test_brute_force_chain():
    rng = np.random.default_rng(4)
    M, K, D, d = 3, 8, 8, 4
    nq, nk, nv = 8, 4, 4
    A, W1, R = rng.standard_normal((M, K)), rng.standard_normal((K, D)) / 3, rng.standard_normal((M, D))
    g, W = 1 + 0.1 * rng.standard_normal(D), rng.standard_normal((D, nq + nk + nv)) / 3
    pos = [0, 5, 11]
    out = oracle.forward_rope(A, W1, R, g, W, 1e-5, pos, nq, nk, d, 10000.0)
    for i in range(M):
        y = [float(v) for v in out["Y"][i]]
        for h in range(0, nq + nk, d):
            for j in range(d // 2):
                a = pos[i] * 10000.0 ** (-2.0 * j / d)
                e, o = y[h + 2 * j], y[h + 2 * j + 1]
                assert out["Yr"][i, h + 2 * j] == pytest.approx(e * math.cos(a) - o * math.sin(a), abs=1e-12)
                assert out["Yr"][i, h + 2 * j + 1] == pytest.approx(e * math.sin(a) + o * math.cos(a), abs=1e-12)


def test_inputs_and_shapes():
    wl = ci.WORKLOADS["7b-rope-bf16"]
    p = ci.make_positions(wl)
    assert p.dtype == np.int32 and p[0] == 0 and p[2047] == 2047 and p[2048] == 0 and p.shape == (wl.M,)
    with pytest.raises(ValueError):
        oracle.forward_rope(*([np.zeros((1, 8))] * 3), np.ones(8), np.zeros((8, 24)), 1e-5, [0], 12, 8, 8, 1e4)


def test_backward_is_the_adjoint():
    # <rotate(y), G> = <y, rope_backward(G)> for all y, G (the gradient of a
    # linear map), checked on the unit basis of a small case; and the backward
    # inverts the rotation
    d, nq, nk, nv = 8, 8, 8, 8
    N = nq + nk + nv
    pos = np.array([0, 3, 700])
    G = _y(6, 3, N)
    back = oracle.rope_backward(G, pos, nq, nk, d, 10000.0)
    for i in range(3):
        for j in range(N):
            e = np.zeros((3, N))
            e[i, j] = 1.0
            fwd = oracle.rope_rotate(e, pos, nq, nk, d, 10000.0)
            assert np.sum(fwd * G) == pytest.approx(back[i, j], abs=1e-13)
    Y = _y(7, 3, N)
    np.testing.assert_allclose(oracle.rope_backward(oracle.rope_rotate(Y, pos, nq, nk, d, 10000.0), pos, nq, nk, d,
                                                    10000.0), Y, atol=1e-13)
    np.testing.assert_array_equal(back[:, nq + nk:], G[:, nq + nk:])


@pytest.mark.parametrize("kind", ["rotate_half_pairs", "theta_without_2", "sin_sign", "rotate_v"])
def test_pins_reject_planted_mistakes(kind):
    d, nq, nk = 8, 16, 8
    Y = _y(5, 3, nq + nk + 8)
    pos = np.array([1, 3, 10])
    ref = oracle.rope_rotate(Y, pos, nq, nk, d, 10000.0)
    bad = np.array(Y)
    i = np.arange(d // 2)
    theta = 10000.0 ** ((-1.0 if kind == "theta_without_2" else -2.0) * i / d)
    ang = pos[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    if kind == "sin_sign":
        s = -s
    heads = range(0, nq + nk + (8 if kind == "rotate_v" else 0), d)
    for h in heads:
        if kind == "rotate_half_pairs":
            a, b = Y[:, h:h + d // 2], Y[:, h + d // 2:h + d]
            bad[:, h:h + d // 2], bad[:, h + d // 2:h + d] = a * c - b * s, a * s + b * c
        else:
            e, o = Y[:, h:h + d:2], Y[:, h + 1:h + d:2]
            bad[:, h:h + d:2], bad[:, h + 1:h + d:2] = e * c - o * s, e * s + o * c
    assert np.max(np.abs(bad - ref)) > 1e-3
