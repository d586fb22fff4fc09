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
  * the first GEMM's epilogue keeps H in bf16 and quantises H g for the
    second GEMM without a scale: Hg8 = e4m3(clamp(float(H_bf16) * g, +-448)),
    the product taken in float32 and rounded to nearest-even, which is the
    precision the kernel takes that decision in;
  * r comes from the exact H, as in the bf16 chain;
  * quantising a bf16 operand (quantize_rows): per row, scale = amax / 448
    in float32 (1 for an all-zero row), codes = e4m3(float32(x) / scale),
    the division correctly rounded in float32; a column-wise variant gives
    the transposed weight codes with per-output-channel scales.

    A   = e4m3(A8) * sa[:, None]            W1 = (e4m3(W1t8) * sw1[:, None])^T
    H   = A W1 + R                          Hb = bf16(H)
    Hg8 = e4m3_code(f32(Hb) * f32(g))       r  = 1 / sqrt(mean_j H_ij^2 + eps)
    Y   = diag(r) e4m3(Hg8) (e4m3(W2t8) * sw2[:, None])^T
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


def forward_fp8(A8, sa, W1t8, sw1, R, g, W2t8, sw2, eps: float,
                rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Returns float64 H (exact), Hb (bf16-rounded H), r, Y and the uint8 Hg8 codes."""
    sa = np.asarray(sa, dtype=np.float64)
    W1 = (e4m3_decode(W1t8) * np.asarray(sw1, dtype=np.float64)[:, None]).T
    W2 = (e4m3_decode(W2t8) * np.asarray(sw2, dtype=np.float64)[:, None]).T
    idx = np.arange(np.asarray(A8).shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    A = e4m3_decode(np.asarray(A8)[idx]) * sa[idx, None]
    H = A @ W1 + np.asarray(R, dtype=np.float64)[idx]
    Hb = bf16_round(H)
    prod = (Hb.astype(np.float32) * np.asarray(g, dtype=np.float32)[None, :]).astype(np.float32)
    Hg8 = e4m3_encode(prod)
    ms = np.mean(H * H, axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    Y = r[:, None] * (e4m3_decode(Hg8) @ W2)
    return {"H": H, "Hb": Hb, "Hg8": Hg8, "r": r, "Y": Y}
