"""Pins for the fp64 CPU oracle of the fp8 chain (CPU only).

The pages give no fp8 recipe (the CODA news article by Synced names FP8 only
as making matrix products faster); the readings are in oracle/fp8.py.  Pins:
the e4m3 code table against values the OCP format definition fixes, the
encoder's round trip, ties and saturation, two independent encoders agreeing,
bf16 rounding against torch's cast, a pure-Python brute force of the whole
fp8 chain, a lossless special case that reduces to the plain chain's oracle,
a hand-worked case for the quantisation of the stored bf16 H, and planted
mistakes that the brute force or the hand-worked case rejects.
"""
import math

import numpy as np
import pytest
import torch

import coda_inputs as ci
import oracle


def test_code_table_fixed_values():
    dec = oracle.e4m3_decode
    assert dec(0x38) == 1.0 and dec(0xB8) == -1.0
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0          # largest finite
    assert dec(0x08) == 2.0 ** -6 and dec(0x01) == 2.0 ** -9      # smallest normal / subnormal
    assert dec(0x07) == 7 * 2.0 ** -9
    assert dec(0x40) == 2.0 and dec(0x3C) == 1.5 and dec(0x39) == 1.125
    assert dec(0x00) == 0.0 and np.signbit(dec(0x80))
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    pos = dec(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                               # increasing, 127 distinct


def test_encoder_round_trip_ties_and_saturation():
    codes = np.arange(0x7F)
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(-vals[1:]), codes[1:] | 0x80)
    mids = (vals[:-1] + vals[1:]) / 2
    got = oracle.e4m3_encode(mids)
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])   # halfway: the even code
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mids, 0)), codes[:-1])
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mids, 1e9)), codes[1:])
    np.testing.assert_array_equal(oracle.e4m3_encode([448.0, 464.0, 1e6, -1e30]), [0x7E, 0x7E, 0x7E, 0xFE])
    assert oracle.e4m3_encode([np.nan])[0] == 0x7F


def test_two_independent_encoders_agree():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * 40, rng.standard_normal(20000) * 1e-3,
                        oracle.e4m3_decode(np.arange(0x7F))]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(x), ci.e4m3_codes(x))


def test_bf16_round_is_torch_cast():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000) * 10, [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)]])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)


def _case(seed, M, K, D, N2):
    wl = ci.custom_workload(M, K, D, N2, dtype="fp8", wl_id=seed)
    x = ci.make_inputs_fp8(wl, seed=seed)
    return wl, x


def _args(x):
    return (x["A8"], x["sa"], x["W1t8"], x["sw1"], x["R"].f32, x["g"].f32, x["W2t8"], x["sw2"])


def _brute(A8, sa, W1t8, sw1, R, g, W2t8, sw2, eps):
    """Pure-Python fp8 chain: the code table from the format definition,
    math.fsum sums, float32 product, the block exponent by direct search and
    nearest-even e4m3 by direct search."""
    def val(c):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        return s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    pos = [val(c) for c in range(0x7F)]

    def enc(x):
        a = min(abs(x), 448.0)
        best = min(range(0x7F), key=lambda c: (abs(pos[c] - a), c % 2))
        return best | (0x80 if math.copysign(1.0, x) < 0 else 0)

    def block_exp(vals):   # smallest E in [-127, 127] with max |v| <= 448 * 2^E; 0 for a zero block
        amax = max(abs(v) for v in vals)
        if amax == 0:
            return 0
        return next((E for E in range(-127, 128) if amax <= math.ldexp(448.0, E)), 127)

    M, K = len(A8), len(A8[0])
    D, N2 = len(W1t8), len(W2t8)
    H = [[math.fsum([val(A8[i][k]) * float(sa[i]) * val(W1t8[j][k]) * float(sw1[j]) for k in range(K)]
                    + [float(R[i][j])]) for j in range(D)] for i in range(M)]
    Hb = [[float(torch.tensor(h, dtype=torch.float64).to(torch.bfloat16)) for h in row] for row in H]
    x = [[float(np.float32(np.float32(Hb[i][j]) * np.float32(g[j]))) for j in range(D)] for i in range(M)]
    E = [[block_exp(x[i][b:b + 32]) for b in range(0, D, 32)] for i in range(M)]
    Hg8 = [[enc(math.ldexp(x[i][j], -E[i][j // 32])) for j in range(D)] for i in range(M)]
    r = [1.0 / math.sqrt(math.fsum(h * h for h in H[i]) / D + eps) for i in range(M)]
    Y = [[r[i] * math.fsum(math.ldexp(val(Hg8[i][j]), E[i][j // 32]) * val(W2t8[n][j]) * float(sw2[n])
                           for j in range(D)) for n in range(N2)] for i in range(M)]
    return np.array(H), np.array(Hg8, dtype=np.uint8), np.array(E), np.array(r), np.array(Y)


@pytest.mark.parametrize("shape", [(1, 16, 8, 8), (3, 32, 16, 8), (5, 16, 24, 16), (3, 16, 80, 8)])
def test_brute_force(shape):
    wl, x = _case(40 + sum(shape), *shape)
    out = oracle.forward_fp8(*_args(x), wl.eps)
    H, Hg8, E, r, Y = _brute(*(np.asarray(a).tolist() if np.asarray(a).ndim == 2 else np.asarray(a)
                               for a in _args(x)), wl.eps)
    np.testing.assert_allclose(out["H"], H, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(out["Hg8_exp"], E)
    np.testing.assert_array_equal(out["Hg8"], Hg8)
    np.testing.assert_allclose(out["r"], r, rtol=1e-13)
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-12, atol=1e-13)


def test_lossless_case_reduces_to_the_plain_chain():
    # small-integer codes, unit scales, g = 1 and integer R: every H g is an
    # integer of magnitude < 16, exactly representable in e4m3, so the fp8
    # chain equals the plain oracle on the dequantised operands
    rng = np.random.default_rng(5)
    M, K, D, N2 = 4, 8, 16, 12
    enc = {v: int(oracle.e4m3_encode([float(v)])[0]) for v in range(-2, 3)}
    A = rng.integers(-1, 2, size=(M, K))
    W1t = rng.integers(-1, 2, size=(D, K))
    W2t = rng.integers(-2, 3, size=(N2, D))
    R = rng.integers(-3, 4, size=(M, D)).astype(np.float64)
    to8 = np.vectorize(lambda v: enc[int(v)])
    out = oracle.forward_fp8(to8(A).astype(np.uint8), np.ones(M), to8(W1t).astype(np.uint8), np.ones(D), R,
                             np.ones(D), to8(W2t).astype(np.uint8), np.ones(N2), 1e-5)
    ref = oracle.forward(A.astype(float), W1t.T.astype(float), R, np.ones(D), W2t.T.astype(float), 1e-5)
    assert np.all(np.abs(out["H"]) < 16)
    np.testing.assert_array_equal(out["Hb"], ref["H"])
    np.testing.assert_allclose(out["Y"], ref["Y"], rtol=1e-13, atol=1e-13)


def _hand_case():
    # K = 1: A = 1.0 (code 0x38, sa 1), W1 = 2^-9 (code 0x01) with sw1 0.5,
    # R = 1.0625, g = 1: H = 1.0625 + 2^-10.  The stored bf16 H is 1.0625
    # (spacing 2^-7 near 1).  Its one-column block has max 1.0625, so the
    # block exponent is -8 (448 * 2^-9 = 0.875 < 1.0625 <= 1.75); scaled,
    # 1.0625 * 2^8 = 272 lies halfway between e4m3 256 and 288, so the even
    # code 0x78 (256, i.e. 1.0 after the scale); the unrounded H would give
    # 272.25, code 0x79 (288, i.e. 1.125).
    return (np.array([[0x38]], np.uint8), np.array([1.0], np.float32), np.array([[0x01]], np.uint8),
            np.array([0.5], np.float32), np.array([[1.0625]]), np.array([1.0]),
            np.array([[0x38]], np.uint8), np.array([1.0], np.float32))


def test_quantises_the_stored_bf16_h():
    out = oracle.forward_fp8(*_hand_case(), 0.0)
    assert out["H"][0, 0] == 1.0625 + 2.0 ** -10
    assert out["Hb"][0, 0] == 1.0625
    assert out["Hg8_exp"][0, 0] == -8
    assert out["Hg8"][0, 0] == 0x78
    assert out["Y"][0, 0] == pytest.approx(1.0 / (1.0625 + 2.0 ** -10), rel=1e-15)   # r * 1.0 * 1.0


def _mutant_codes(kind, a, eps):
    A8, sa, W1t8, sw1, R, g, W2t8, sw2 = a
    W1 = (oracle.e4m3_decode(W1t8) * sw1[:, None]).T
    A = oracle.e4m3_decode(A8) * sa[:, None]
    if kind == "scale_columns_of_A":
        A = oracle.e4m3_decode(A8) * np.resize(sa, A8.shape[1])[None, :]
    if kind == "weights_not_transposed":
        W1 = (oracle.e4m3_decode(W1t8) * sw1[:, None]).reshape(W1.shape)
    H = A @ W1 + R
    prod = H if kind == "no_bf16_before_quantising" else oracle.bf16_round(H)
    prod = (np.asarray(prod, dtype=np.float32) * np.asarray(g, np.float32)).astype(np.float32)
    E = oracle.mx_exponents(prod, block=64 if kind == "blocks_of_64" else 32)
    if kind == "exponent_rounded_down":     # saturating: max |x| * 2^-E may exceed 448
        E = np.where(E != 0, E - 1, E)
    Ecol = np.repeat(E, 64 if kind == "blocks_of_64" else 32, axis=1)[:, :prod.shape[1]]
    scaled = np.ldexp(prod.astype(np.float64), -Ecol)
    codes = oracle.e4m3_encode(scaled)
    if kind == "round_down":
        v = oracle.e4m3_decode(codes)
        codes = np.where(np.abs(v) > np.abs(scaled), np.where(codes & 0x7F, codes - 1, codes), codes).astype(np.uint8)
    r = 1.0 / np.sqrt(np.mean(H * H, axis=1) + eps)
    return codes, r[:, None] * (np.ldexp(oracle.e4m3_decode(codes), Ecol) @ (oracle.e4m3_decode(W2t8) * sw2[:, None]).T)


@pytest.mark.parametrize("kind", ["no_bf16_before_quantising", "scale_columns_of_A", "weights_not_transposed",
                                  "round_down", "blocks_of_64", "exponent_rounded_down"])
def test_pins_reject_planted_mistakes(kind):
    if kind == "no_bf16_before_quantising":
        codes, _ = _mutant_codes(kind, _hand_case(), 0.0)
        assert codes[0, 0] != oracle.forward_fp8(*_hand_case(), 0.0)["Hg8"][0, 0] == 0x78
        return
    if kind == "blocks_of_64":
        # one row, A = 0 so H = R: columns 0..31 around 0.01, columns 32..63
        # around 10.  Their 32-column blocks get exponents -15 and -5; a
        # shared 64-column block would quantise the small half with -5 and
        # lose most of its bits.
        R = np.concatenate([np.linspace(0.004, 0.011, 32), np.linspace(3.0, 10.0, 32)])[None, :]
        a = (np.zeros((1, 16), np.uint8), np.ones(1, np.float32), np.zeros((64, 16), np.uint8), np.ones(64, np.float32),
             R, np.ones(64), np.full((8, 64), 0x38, np.uint8), np.ones(8, np.float32))
        out = oracle.forward_fp8(*a, 1e-5)
        assert list(out["Hg8_exp"][0]) == [-15, -5]
        codes, _ = _mutant_codes(kind, a, 1e-5)
        assert not np.array_equal(codes, out["Hg8"])
        return
    wl, x = _case(77, 3, 16, 80, 8)
    a = _args(x)
    _, Hg8, _, _, Y = _brute(*(np.asarray(v).tolist() if np.asarray(v).ndim == 2 else np.asarray(v) for v in a),
                             wl.eps)
    codes, Ym = _mutant_codes(kind, a, wl.eps)
    assert (not np.array_equal(codes, Hg8)) or np.max(np.abs(Ym - Y)) > 1e-9


def test_mx_exponents_closed_forms():
    x = np.array([[448.0, 0, 0, 0], [449.0, 1, 0, 0], [1.0, 0.5, 0, 0], [1.75, -1.0, 0, 0], [0, 0, 0, 0],
                  [-2.0 ** -140, 0, 0, 0], [3e38, 0, 0, 0], [-0.875, 0, 0, 0]], dtype=np.float32)
    E = oracle.mx_exponents(x, block=4)[:, 0]
    # 448 <= 448 * 2^0; 449 needs 2^1; 1.0 and 1.75 fit 448 * 2^-8 = 1.75; 0.875 = 448 * 2^-9
    np.testing.assert_array_equal(E, [0, 1, -8, -8, 0, -127, 120, -9])
    # the definition on random magnitudes: 448 * 2^(E-1) < amax <= 448 * 2^E
    rng = np.random.default_rng(3)
    a = np.exp(rng.uniform(-60, 60, size=(500, 32))).astype(np.float32) * rng.choice([-1, 1], size=(500, 32))
    E = oracle.mx_exponents(a)[:, 0].astype(np.float64)
    amax = np.max(np.abs(a.astype(np.float64)), axis=1)
    assert np.all(amax <= np.ldexp(448.0, E.astype(int))) and np.all(amax > np.ldexp(448.0, E.astype(int) - 1))


def test_large_residual_does_not_saturate():
    # a residual stream 1000x larger than the recipe's N(0, 1): H g reaches
    # ~4e3, far past e4m3's 448.  With the block exponents the fp8 chain's Y
    # stays within the e4m3 rounding of the exact chain on the dequantised
    # operands; the unscaled recipe (codes of clamp(H g, 448)) would be off
    # by most of Y.
    wl, x = _case(91, 64, 64, 128, 64)
    R = x["R"].f32 * 1000.0
    A8, sa, W1t8, sw1, _, g, W2t8, sw2 = _args(x)
    out = oracle.forward_fp8(A8, sa, W1t8, sw1, R, g, W2t8, sw2, wl.eps)
    W1 = (oracle.e4m3_decode(W1t8) * sw1[:, None]).T
    W2 = (oracle.e4m3_decode(W2t8) * sw2[:, None]).T
    exact = oracle.forward(oracle.e4m3_decode(A8) * sa[:, None], W1, R, g, W2, wl.eps)
    assert np.max(np.abs(out["Hb"] * g[None, :])) > 2000
    rel = np.max(np.abs(out["Y"] - exact["Y"])) / np.max(np.abs(exact["Y"]))
    assert rel < 0.05, rel
    prod = (out["Hb"].astype(np.float32) * g.astype(np.float32)[None, :]).astype(np.float32)
    Yclamp = out["r"][:, None] * (oracle.e4m3_decode(oracle.e4m3_encode(prod)) @ W2)
    assert np.max(np.abs(Yclamp - exact["Y"])) / np.max(np.abs(exact["Y"])) > 0.5


def test_quantize_rows_pins():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((6, 200)) * np.array([[1e-3], [1.0], [30.0], [1e4], [0.0], [2.0]])).astype(np.float32)
    x[5, 17] = -9.0                                  # a row whose largest magnitude is negative
    codes, scale = oracle.quantize_rows(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[4] == 1.0 and np.all(codes[4] & 0x7F == 0)          # zero row (signed zeros kept)
    # the largest magnitude of each row maps to the largest code, 448
    for i in (0, 1, 2, 3, 5):
        j = np.argmax(np.abs(x[i]))
        assert oracle.e4m3_decode(codes[i, j]) == np.sign(x[i, j]) * 448.0
    assert codes[5, 17] == 0xFE                                       # -448
    # round trip within half an e4m3 step (3 mantissa bits: relative 2^-4
    # for normals; absolute 2^-10 scale for subnormals)
    back = oracle.e4m3_decode(codes) * scale[:, None].astype(np.float64)
    err = np.abs(back - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None])
    assert np.all(err <= bound * 1.0000001)
    # brute force: each code is the nearest representable value of x / scale
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for i in (1, 2):
        for j in range(0, 200, 13):
            q = np.float32(x[i, j]) / scale[i]
            d = np.abs(np.abs(np.float64(q)) - vals)
            assert abs(oracle.e4m3_decode(codes[i, j])) in vals[d == d.min()]


def test_quantize_matches_the_input_generators_recipe():
    # two independent implementations of the same recipe agree bit for bit
    rng = np.random.default_rng(22)
    x = rng.standard_normal((64, 96)).astype(np.float32) * 3
    c1, s1 = oracle.quantize_rows(x)
    c2, s2 = ci._quantize_rows(x)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)
    ct, st = oracle.quantize_cols_transposed(x)
    np.testing.assert_array_equal(ct, oracle.quantize_rows(x.T)[0])
    assert ct.shape == (96, 64) and st.shape == (96,)


def _bwd_case(seed, M=24, K=32, D=48, N2=64):
    rng = np.random.default_rng(seed)
    return dict(dY=rng.standard_normal((M, N2)).astype(np.float32),
                A=rng.standard_normal((M, K)).astype(np.float32),
                W1=(rng.standard_normal((K, D)) / np.sqrt(K)).astype(np.float32),
                R=rng.standard_normal((M, D)).astype(np.float32),
                g=(1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
                W2=(rng.standard_normal((D, N2)) / np.sqrt(D)).astype(np.float32))


def test_fp8_backward_without_quantisation_is_the_chain_backward():
    c = _bwd_case(31)
    got = oracle.backward_fp8(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5, quantise=False,
                              store_bf16=False)
    ref = oracle.backward(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5)
    for k in ("dA", "dR", "dW1", "dW2", "dg"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-10, atol=1e-12, err_msg=k)


def test_fp8_backward_close_to_exact():
    c = _bwd_case(32, M=256, K=128, D=128, N2=256)
    got = oracle.backward_fp8(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5)
    ref = oracle.backward(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5)
    for k in ("dA", "dW1", "dW2", "dg"):
        rel = np.max(np.abs(got[k] - ref[k])) / np.max(np.abs(ref[k]))
        assert 1e-4 < rel < 0.08, (k, rel)     # quantised, but within a few e4m3 steps


@pytest.mark.parametrize("which", ["dY_row", "W2_row", "dY_col", "W1_row", "A_col"])
def test_fp8_backward_quantisation_axes(which):
    # quantisation commutes with a power-of-two scaling of the vector its
    # scale covers: scaling row i of dY by 8 scales row i of G exactly and
    # leaves the other rows alone (per-row quantisation of dY); likewise for
    # W2's rows (G's columns), dY's columns (dW2's columns), W1's rows (dA's
    # columns) and A's columns (dW1's rows).  A quantiser on the wrong axis
    # would change the other rows or columns too.
    c = _bwd_case(33)
    # fix H and r so that only the backward products see the change
    H = c["A"].astype(np.float64) @ c["W1"].astype(np.float64) + c["R"]
    r = 1.0 / np.sqrt(np.mean(H * H, axis=1) + 1e-5)
    base = oracle.backward_fp8(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5, H=H, r=r)
    c2 = {k: v.copy() for k, v in c.items()}
    if which == "dY_row":
        c2["dY"][5] *= 8
        out, key, sel, axis = "G", "G", 5, 0
    elif which == "W2_row":
        c2["W2"][7] *= 8
        out, key, sel, axis = "G", "G", 7, 1
    elif which == "dY_col":
        c2["dY"][:, 9] *= 8
        out, key, sel, axis = "dW2", "dW2", 9, 1
    elif which == "W1_row":
        c2["W1"][3] *= 8
        out, key, sel, axis = "dA", "dA", 3, 1
    else:
        c2["A"][:, 4] *= 8
        out, key, sel, axis = "dW1", "dW1", 4, 0
    new = oracle.backward_fp8(c2["dY"], c2["A"], c2["W1"], c2["R"], c2["g"], c2["W2"], 1e-5, H=H, r=r)
    a, b = base[key], new[key]
    if axis == 0:
        np.testing.assert_array_equal(b[sel], 8 * a[sel])
        np.testing.assert_array_equal(np.delete(b, sel, axis=0), np.delete(a, sel, axis=0))
    else:
        np.testing.assert_array_equal(b[:, sel], 8 * a[:, sel])
        np.testing.assert_array_equal(np.delete(b, sel, axis=1), np.delete(a, sel, axis=1))


# ---- the backward's bf16 storage (P, X_n, dH), pinned independently -------
from tests import fp8_backward_brute as bb  # noqa: E402


def _bwd_pin_case(seed, M=40, K=16, D=48, N2=72):
    # every contraction spans more than one block of 32 and ends in a short
    # block (N2 = 72, D = 48, M = 40): per-vector scales would not match
    # the backward's inputs, with H and r as the forward stores them (H in
    # bf16, r in float32)
    c = _bwd_case(seed, M, K, D, N2)
    H = oracle.bf16_round(c["A"].astype(np.float64) @ c["W1"].astype(np.float64) + c["R"])
    r = (1.0 / np.sqrt(np.mean(H * H, axis=1) + 1e-5)).astype(np.float32).astype(np.float64)
    return c, H, r


def _listed(*arrays):
    return [np.asarray(a, dtype=np.float64).tolist() for a in arrays]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_backward_matches_brute_force(seed):
    c, H, r = _bwd_pin_case(seed)
    got = oracle.backward_fp8(c["dY"], c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5, H=H, r=r)
    ref = bb.backward(*_listed(c["dY"], c["A"], c["W1"], c["g"], c["W2"], H, r))
    for k in ("dA", "dR", "dW1", "dW2", "dg"):
        np.testing.assert_allclose(got[k], np.array(ref[k]), rtol=1e-12, atol=1e-13, err_msg=k)


def _bwd_fp8_mutant(kind, c, H, r):
    """oracle.backward_fp8's steps with one planted mistake in where a value is
    stored in bf16."""
    from oracle.fp8 import _deq_cols, _deq_rows
    rnd = oracle.bf16_round
    g = np.asarray(c["g"], np.float64)
    D = c["W1"].shape[1]
    G = _deq_rows(c["dY"], True) @ _deq_rows(c["W2"], True).T
    P = G * g[None, :]
    s = np.sum((rnd(P) if kind == "s_from_stored_P" else P) * H, axis=1)
    if kind == "Xn_not_stored":
        Xn = (H * r[:, None]) * g[None, :]
    elif kind == "Xn_rounded_before_g":
        Xn = rnd(rnd(H * r[:, None]) * g[None, :])
    else:
        Xn = rnd((H * r[:, None]) * g[None, :])
    cc = (r ** 3 * s / D)[:, None]
    Pu = P if kind == "dH_from_unrounded_P" else rnd(P)
    if kind == "dH_terms_rounded_first":
        dH = rnd(rnd(r[:, None] * Pu) - rnd(cc * H))
    elif kind == "dH_not_stored":
        dH = r[:, None] * Pu - cc * H
    else:
        dH = rnd(r[:, None] * Pu - cc * H)
    return {"dW2": _deq_cols(Xn, True).T @ _deq_cols(c["dY"], True),
            "dA": _deq_rows(dH, True) @ _deq_rows(c["W1"], True).T,
            "dW1": _deq_cols(c["A"], True).T @ _deq_cols(dH, True)}


@pytest.mark.parametrize("kind", ["dH_from_unrounded_P", "dH_terms_rounded_first", "dH_not_stored",
                                  "Xn_not_stored", "Xn_rounded_before_g", "s_from_stored_P"])
def test_fp8_backward_storage_pin_rejects_planted_mistakes(kind):
    # each misplaced bf16 rounding moves some stored value by an ulp, which
    # flips e4m3 codes (or a row / column scale) of a quantised product: the
    # products through those codes leave the brute force by far more than
    # the brute force and the oracle differ (3e-16)
    c, H, r = _bwd_pin_case(0)
    ref = bb.backward(*_listed(c["dY"], c["A"], c["W1"], c["g"], c["W2"], H, r))
    m = _bwd_fp8_mutant(kind, c, H, r)
    worst = max(np.max(np.abs(m[k] - np.array(ref[k]))) / np.max(np.abs(np.array(ref[k]))) for k in m)
    assert worst > 1e-3, f"{kind} not rejected ({worst:.1e})"


def test_fp8_backward_quantises_the_stored_bf16_xn():
    # Hand-worked: M = 2, K = D = N2 = 1, g = 1, dY = 1, H = (256, 1),
    # r = (1, r1) with r1 = float32(1.0627) = 1.06270003...  X_n = H r g is
    # (256, r1); stored in bf16 the second is 1.0625 (spacing 2^-7), exactly
    # halfway between the e4m3 values 1.0 and 1.125, so its code is the even
    # one, 1.0 -- while the unrounded r1 is past the midpoint: 1.125.
    # X_n's column is one block with largest magnitude 256: exponent 0
    # (224 < 256 <= 448), codes 256 and 1.0.  dY's column (1, 1) has exponent
    # -8 (1 <= 448 / 256 = 1.75) and codes 256, i.e. exactly 1.  So
    # dW2 = 256 + 1.0 = 257, not 257.125.
    r1 = float(np.float32(1.0627))
    assert oracle.bf16_round(np.array([r1]))[0] == 1.0625
    one = np.ones((2, 1), np.float32)
    out = oracle.backward_fp8(one, one, np.ones((1, 1), np.float32), np.zeros((2, 1)), np.ones(1, np.float32),
                              np.ones((1, 1), np.float32), 0.0, H=np.array([[256.0], [1.0]]), r=np.array([1.0, r1]))
    assert out["Xn"][1, 0] == 1.0625
    assert out["dW2"][0, 0] == 257.0


def test_mx_quantize_hand_values():
    # one row, blocks of 32 (the second one short):
    #   block 0: 448 and 1.0 -> E = 0, codes exact (448 = 0x7E, 1.0 = 0x38);
    #   block 1: 449 -> E = 1: 224.5 lies between the e4m3 values 224 and 240,
    #   nearer 224 (0x76), which stands for 448; 3.0 -> 1.5 (0x3C), i.e. 3.0.
    x = np.zeros((1, 40), np.float32)
    x[0, 0], x[0, 1], x[0, 32], x[0, 33] = 448.0, 1.0, 449.0, 3.0
    codes, E = oracle.mx_quantize(x)
    assert E.tolist() == [[0, 1]]
    assert codes[0, :2].tolist() == [0x7E, 0x38] and codes[0, 32:34].tolist() == [0x76, 0x3C]
    assert np.all(codes[0, 2:32] == 0) and np.all(codes[0, 34:] == 0)
    deq = oracle.mx_dequantize(codes, E)
    assert deq[0, 0] == 448.0 and deq[0, 1] == 1.0 and deq[0, 32] == 448.0 and deq[0, 33] == 3.0


def test_fp8_backward_blocks_are_independent():
    # MX quantisation is block-local: scaling the 32 contraction elements of
    # one block by 8 multiplies that block's dequantised values by 8 exactly
    # and leaves every other block's alone.  So scaling dY[i, 32:64] by 8 adds
    # exactly 7 times that block's contribution to row i of G (the contribution
    # computed from dY with everything else zeroed), and changes no other row.
    # With one scale per row (or blocks of 64) the rest of row i would move.
    c = _bwd_case(34, M=8, K=16, D=16, N2=96)
    H = c["A"].astype(np.float64) @ c["W1"].astype(np.float64) + c["R"]
    r = 1.0 / np.sqrt(np.mean(H * H, axis=1) + 1e-5)
    args = (c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5)
    base = oracle.backward_fp8(c["dY"], *args, H=H, r=r)["G"]
    dY2 = c["dY"].copy()
    dY2[3, 32:64] *= 8
    new = oracle.backward_fp8(dY2, *args, H=H, r=r)["G"]
    only = np.zeros_like(c["dY"])
    only[3, 32:64] = c["dY"][3, 32:64]
    part = oracle.backward_fp8(only, *args, H=H, r=r)["G"]
    np.testing.assert_allclose(new[3], base[3] + 7 * part[3], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.delete(new, 3, axis=0), np.delete(base, 3, axis=0))
    # the same along the contraction over M: dW2 with a block of dY's column 5
    # (rows 32..63 of that column) scaled
    c = _bwd_case(35, M=96, K=16, D=16, N2=24)
    H = c["A"].astype(np.float64) @ c["W1"].astype(np.float64) + c["R"]
    r = 1.0 / np.sqrt(np.mean(H * H, axis=1) + 1e-5)
    args = (c["A"], c["W1"], c["R"], c["g"], c["W2"], 1e-5)
    base = oracle.backward_fp8(c["dY"], *args, H=H, r=r)["dW2"]
    dY2 = c["dY"].copy()
    dY2[32:64, 5] *= 8
    new = oracle.backward_fp8(dY2, *args, H=H, r=r)["dW2"]
    only = np.zeros_like(c["dY"])
    only[32:64, 5] = c["dY"][32:64, 5]
    part = oracle.backward_fp8(only, *args, H=H, r=r)["dW2"]
    np.testing.assert_allclose(new[:, 5], base[:, 5] + 7 * part[:, 5], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.delete(new, 5, axis=1), np.delete(base, 5, axis=1))


def _deq_per_row_scale(x, on):
    codes, scale = oracle.quantize_rows(x)
    return oracle.e4m3_decode(codes) * scale[:, None].astype(np.float64)


def _deq_blocks_of_64(x, on):
    from oracle.fp8 import mx_exponents
    x = np.asarray(x, np.float32)
    E = np.repeat(mx_exponents(x, 64), 64, axis=1)[:, :x.shape[1]]
    return np.ldexp(oracle.e4m3_decode(oracle.e4m3_encode(np.ldexp(x.astype(np.float64), -E))), E)


@pytest.mark.parametrize("mutant", [_deq_per_row_scale, _deq_blocks_of_64], ids=["per_row_scale", "blocks_of_64"])
def test_block_pin_rejects_planted_granularity(mutant, monkeypatch):
    # the backward's quantiser replaced by one with the wrong granularity (the
    # brute force alone cannot tell blocks of 64 from blocks of 32 on Gaussian
    # data: their exponents nearly always agree); the block-independence pin
    # must fail
    import oracle.fp8 as f
    monkeypatch.setattr(f, "_deq_rows", mutant)
    with pytest.raises(AssertionError):
        test_fp8_backward_blocks_are_independent()
