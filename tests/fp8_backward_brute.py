"""Pure-Python brute force of the fp8 chain's backward (tiny inputs only).

A second, independent implementation of the reading that oracle/fp8.py
documents for the backward: every product takes e4m3 operands quantised along
its contraction with MX block exponents (per row or per column, in blocks of
32 contraction elements, the last one short: E the smallest integer with the
block's largest float32 magnitude <= 448 2^E, clamped to [-127, 127], 0 for
an all-zero block; codes the nearest-even e4m3 of x 2^-E), the quantisers
count as the identity when differentiating, and the three values
the recipe keeps in bf16 -- P = g G, X_n = (H r) g and dH = r P - (r^3 s / D) H
-- are rounded to bf16 at the point they are stored, from their float32 value
(a value the kernels hold in float32 is stored as bf16), with dH taking the
stored P.  s and dg use the unrounded products.

Nothing here comes from the oracle: the e4m3 values come from the format's
definition, nearest codes from a direct search, bf16 rounding from the
float32 bit pattern (round half to even on the low 16 bits), sums from
math.fsum, and float32 rounding from struct.
"""
import math
import struct


def f32(x: float) -> float:
    """x rounded to float32 (round to nearest even), as a Python float."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf16(x: float) -> float:
    """x rounded to float32, then to bfloat16 (round to nearest even)."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", u))[0]


def e4m3_value(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 15, c & 7
    return s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


_POS = [e4m3_value(c) for c in range(0x7F)]   # 0 .. 448


def e4m3_nearest(x: float) -> int:
    a = min(abs(x), 448.0)
    best = min(range(0x7F), key=lambda c: (abs(_POS[c] - a), c % 2))
    return best | (0x80 if math.copysign(1.0, x) < 0 else 0)


def block_exponent(amax: float) -> int:
    """The smallest integer E in [-127, 127] with amax <= 448 2^E, found by
    counting up (127 if none; 0 for an all-zero block)."""
    if amax == 0:
        return 0
    E = -127
    while E < 127 and amax > 448.0 * 2.0 ** E:
        E += 1
    return E


def quant_vec(v, block=32):
    """Dequantised values of one vector quantised in blocks of `block`."""
    out = []
    for b0 in range(0, len(v), block):
        blk = [f32(x) for x in v[b0:b0 + block]]
        E = block_exponent(max(abs(x) for x in blk))
        out += [e4m3_value(e4m3_nearest(x * 2.0 ** -E)) * 2.0 ** E for x in blk]
    return out


def quant_rows(X):
    return [quant_vec(row) for row in X]


def quant_cols(X):
    cols = quant_rows([list(c) for c in zip(*X)])
    return [list(r) for r in zip(*cols)]


def backward(dY, A, W1, g, W2, H, r, rounding=("P", "Xn", "dH")):
    """Gradients of <dY, Y> for the chain with fp8 backward products.

    Lists of lists of floats; H and r are the forward's.  `rounding` names the
    stored-in-bf16 values (all three for the reading)."""
    M, N2, K, D = len(dY), len(dY[0]), len(A[0]), len(W1[0])
    rb = lambda name, v: bf16(v) if name in rounding else v
    qdY_r, qW2_r = quant_rows(dY), quant_rows(W2)
    G = [[math.fsum(qdY_r[i][n] * qW2_r[j][n] for n in range(N2)) for j in range(D)] for i in range(M)]
    P = [[g[j] * G[i][j] for j in range(D)] for i in range(M)]
    s = [math.fsum(P[i][j] * H[i][j] for j in range(D)) for i in range(M)]
    dg = [math.fsum(r[i] * H[i][j] * G[i][j] for i in range(M)) for j in range(D)]
    Xn = [[rb("Xn", (H[i][j] * r[i]) * g[j]) for j in range(D)] for i in range(M)]
    c = [r[i] ** 3 * s[i] / D for i in range(M)]
    dH = [[rb("dH", r[i] * rb("P", P[i][j]) - c[i] * H[i][j]) for j in range(D)] for i in range(M)]
    qXn_c, qdY_c = quant_cols(Xn), quant_cols(dY)
    dW2 = [[math.fsum(qXn_c[i][j] * qdY_c[i][n] for i in range(M)) for n in range(N2)] for j in range(D)]
    qdH_r, qW1_r = quant_rows(dH), quant_rows(W1)
    dA = [[math.fsum(qdH_r[i][j] * qW1_r[k][j] for j in range(D)) for k in range(K)] for i in range(M)]
    qA_c, qdH_c = quant_cols(A), quant_cols(dH)
    dW1 = [[math.fsum(qA_c[i][k] * qdH_c[i][j] for i in range(M)) for j in range(D)] for k in range(K)]
    return {"dA": dA, "dR": dH, "dW1": dW1, "dW2": dW2, "dg": dg}
