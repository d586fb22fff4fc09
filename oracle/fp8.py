"""Plain fp64 CPU oracle of the chain with fp8 (e4m3) GEMM operands.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the test-suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP path and imports nothing from it.

Sources (the CODA news article by Synced / 机器之心, mirrored by KuCoin News):
  the opening section says FP8 and FP4 make the matrix products faster while
  the memory-bound operations around them do not shrink, so fusion matters
  more at low precision; it gives no fp8 recipe.  Readings taken:
  * operands are OCP e4m3 codes (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; largest finite 448; no infinities; S.1111.111 is NaN)
    with float32 scales: A per row (sa), the weights per output channel
    (sw1, sw2), the weights stored transposed, [N, K];
  * the first GEMM's epilogue keeps H in bf16 and quantises x = H g for
    the second GEMM with one power-of-two scale per row and block of 32
    columns (the block scaling of the OCP microscaling formats, which
    gfx950's scaled fp8 matrix products apply per 32 contraction elements):
    x is the float32 product float(H_bf16) * g, the block's exponent E is
    the smallest integer with max |x| over the block <= 448 * 2^E (clamped
    to [-127, 127]; 0 for an all-zero block), so no value saturates, and
    the codes are the nearest-even e4m3 of x * 2^-E;
  * r comes from the exact H, as in the bf16 chain;
  * quantising a bf16 operand (quantize_rows): per row, scale = amax / 448
    in float32 (1 for an all-zero row), codes = e4m3(float32(x) / scale),
    the division correctly rounded in float32; a column-wise variant gives
    the transposed weight codes with per-output-channel scales;
  * backward (backward_fp8): every product of the chain's backward takes
    e4m3 operands with MX block exponents along its contraction (mx_quantize:
    one exponent per 32 contraction elements, chosen as for H g above, so
    no value saturates): G = dY W2^T with dY and W2 [D, N2] in blocks along
    their rows; dW2 = Xn^T dY with Xn and dY in blocks along their columns
    (their contraction runs over the M rows); dA = dH W1^T with dH and
    W1 [K, D] along their rows; dW1 = A^T dH with A and dH along their
    columns.  The quantisers are treated as the identity when
    differentiating (straight-through); the rest is the bf16 chain's
    backward: P = g G, s = sum_j P H, dg = sum_i r H G, Xn = (H r) g,
    dH = r P - (r^3 s / D) H, dR = dH.

    A   = e4m3(A8) * sa[:, None]            W1 = (e4m3(W1t8) * sw1[:, None])^T
    H   = A W1 + R                          Hb = bf16(H)
    x   = f32(Hb) * f32(g)                  E_ib = block exponent of x over block b
    Hg8 = e4m3_code(x * 2^-E)               r  = 1 / sqrt(mean_j H_ij^2 + eps)
    Y   = diag(r) (e4m3(Hg8) * 2^E) (e4m3(W2t8) * sw2[:, None])^T
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


def _e4m3_table() -> np.ndarray:
    """Value of every code, from the format's definition."""
    vals = np.empty(256)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


_TABLE = _e4m3_table()
_POS = _TABLE[:0x7F]          # codes 0x00 .. 0x7E: 0 .. 448, increasing


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each value, ties to the even code, magnitudes
    clamped to 448 first (NaN maps to 0x7F)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_POS, a, side="left")             # first code >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS[hi], hi, code)
    code = np.where(np.isnan(x), 0x7F, code | (np.signbit(x).astype(np.int64) << 7))
    return code.astype(np.uint8)


def quantize_rows(x):
    """Per-row e4m3 codes and float32 scales of a float32 matrix: the row's
    largest magnitude maps to 448 (scale = amax / 448, taken in float32; an
    all-zero row gets scale 1)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return e4m3_encode(x / scale[:, None]), scale


def quantize_cols_transposed(w):
    """Codes of w^T [N, K] with one scale per column of w [K, N] (the weight
    stored transposed with per-output-channel scales)."""
    return quantize_rows(np.ascontiguousarray(np.asarray(w, dtype=np.float32).T))


def bf16_round(x) -> np.ndarray:
    """Round to nearest-even bfloat16, returned as float64 (via float32)."""
    f = np.asarray(x, dtype=np.float32)
    m, e = np.frexp(f.astype(np.float64))          # f = m 2^e, 0.5 <= |m| < 1
    # bfloat16 keeps 8 significant bits: scale m to [128, 256) and round half to even
    return (np.round(m * 256.0) / 256.0) * np.exp2(e)


MX_BLOCK = 32


def mx_exponents(x, block: int = MX_BLOCK) -> np.ndarray:
    """Per row and block of `block` columns of x (the last block may be
    short): the smallest integer E with max |x| over the block <= 448 * 2^E,
    clamped to [-127, 127], and 0 for an all-zero block.  int32 [rows,
    ceil(cols / block)]."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    rows, cols = a.shape
    nb = -(-cols // block)
    amax = np.zeros((rows, nb))
    for b in range(nb):
        amax[:, b] = np.max(a[:, b * block:(b + 1) * block], axis=1)
    pos = amax > 0
    E = np.zeros(amax.shape, dtype=np.int64)
    E[pos] = np.ceil(np.log2(amax[pos] / 448.0)).astype(np.int64)
    # settle the rounding of log2 exactly: 448 * 2^(E-1) < amax <= 448 * 2^E
    E = np.where(pos & (amax > np.ldexp(448.0, E)), E + 1, E)
    E = np.where(pos & (amax <= np.ldexp(448.0, E - 1)), E - 1, E)
    return np.clip(E, -127, 127).astype(np.int32)


def mx_quantize(x):
    """MX e4m3 quantisation of a float32 matrix along its rows: per row and
    block of 32 columns the exponent E of mx_exponents, and the codes
    e4m3(x 2^-E) (nearest, ties to the even code).  Returns (codes uint8
    [rows, cols], E int32 [rows, ceil(cols / 32)])."""
    x = np.asarray(x, dtype=np.float32)
    E = mx_exponents(x)
    Ecol = np.repeat(E, MX_BLOCK, axis=1)[:, :x.shape[1]]
    return e4m3_encode(np.ldexp(x.astype(np.float64), -Ecol)), E


def mx_dequantize(codes, E) -> np.ndarray:
    """The values MX codes and their block exponents stand for (float64)."""
    codes = np.asarray(codes)
    Ecol = np.repeat(np.asarray(E, dtype=np.int64), MX_BLOCK, axis=1)[:, :codes.shape[1]]
    return np.ldexp(e4m3_decode(codes), Ecol)


def forward_fp8(A8, sa, W1t8, sw1, R, g, W2t8, sw2, eps: float,
                rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Returns float64 H (exact), Hb (bf16-rounded H), r, Y, the uint8 Hg8
    codes and their int32 block exponents Hg8_exp [rows, ceil(D/32)]."""
    sa = np.asarray(sa, dtype=np.float64)
    W1 = (e4m3_decode(W1t8) * np.asarray(sw1, dtype=np.float64)[:, None]).T
    W2 = (e4m3_decode(W2t8) * np.asarray(sw2, dtype=np.float64)[:, None]).T
    idx = np.arange(np.asarray(A8).shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    A = e4m3_decode(np.asarray(A8)[idx]) * sa[idx, None]
    H = A @ W1 + np.asarray(R, dtype=np.float64)[idx]
    Hb = bf16_round(H)
    prod = (Hb.astype(np.float32) * np.asarray(g, dtype=np.float32)[None, :]).astype(np.float32)
    E = mx_exponents(prod)
    Ecol = np.repeat(E, MX_BLOCK, axis=1)[:, :prod.shape[1]]
    Hg8 = e4m3_encode(np.ldexp(prod.astype(np.float64), -Ecol))
    ms = np.mean(H * H, axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    Y = r[:, None] * (np.ldexp(e4m3_decode(Hg8), Ecol) @ W2)
    return {"H": H, "Hb": Hb, "Hg8": Hg8, "Hg8_exp": E, "r": r, "Y": Y}


def _deq_rows(x, on: bool) -> np.ndarray:
    """x (float32) after MX quantisation along its rows and dequantisation
    (x itself when off)."""
    if not on:
        return np.asarray(x, dtype=np.float64)
    return mx_dequantize(*mx_quantize(x))


def _deq_cols(x, on: bool) -> np.ndarray:
    """x after MX quantisation along its columns (blocks of 32 rows) and
    dequantisation."""
    if not on:
        return np.asarray(x, dtype=np.float64)
    return _deq_rows(np.ascontiguousarray(np.asarray(x, dtype=np.float32).T), True).T


def backward_fp8(dY, A, W1, R, g, W2, eps: float, H=None, r=None, quantise: bool = True,
                 store_bf16: bool = True) -> Dict[str, np.ndarray]:
    """Gradients of <dY, Y> with e4m3 operands in every backward product.

    dY[M,N2], A[M,K], W1[K,D], R[M,D], g[D], W2[D,N2] as float32 values;
    H[M,D] and r[M] are the forward's (recomputed exactly from A, W1, R when
    not given).  store_bf16: the intermediates the recipe keeps in bf16
    (P, X_n and dH, whose stored values the quantisers see) are rounded to
    bf16, so that the quantisation decisions are taken on the values the
    kernels store; s and dg use the unrounded products.  With
    quantise=False and store_bf16=False this is the plain chain's backward.
    Returns float64 dA, dR, dW1, dW2, dg and the intermediates G, dH, Xn.
    """
    A = np.asarray(A, dtype=np.float32)
    W1 = np.asarray(W1, dtype=np.float32)
    W2 = np.asarray(W2, dtype=np.float32)
    dY = np.asarray(dY, dtype=np.float32)
    g = np.asarray(g, dtype=np.float64)
    D = W1.shape[1]
    if H is None:
        H = A.astype(np.float64) @ W1.astype(np.float64) + np.asarray(R, dtype=np.float64)
        r = 1.0 / np.sqrt(np.mean(H * H, axis=1) + eps)
    H = np.asarray(H, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    q = quantise
    rnd = bf16_round if store_bf16 else (lambda v: v)
    G = _deq_rows(dY, q) @ _deq_rows(W2, q).T          # contraction over N2
    P = G * g[None, :]
    s = np.sum(P * H, axis=1)
    dg = np.sum(r[:, None] * H * G, axis=0)
    Xn = rnd((H * r[:, None]) * g[None, :])
    dH = rnd(r[:, None] * rnd(P) - (r ** 3 * s / D)[:, None] * H)
    dW2 = _deq_cols(Xn, q).T @ _deq_cols(dY, q)        # contraction over M
    dA = _deq_rows(dH, q) @ _deq_rows(W1, q).T          # contraction over D
    dW1 = _deq_cols(A, q).T @ _deq_cols(dH, q)          # contraction over M
    return {"dA": dA, "dR": dH.copy(), "dW1": dW1, "dW2": dW2, "dg": dg, "G": G, "dH": dH, "Xn": Xn}
