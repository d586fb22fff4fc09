"""Plain fp64 CPU oracle of the chain's second GEMM as a QKV projection with
rotary position embedding (RoPE) on the query and key columns.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the test-suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP path and imports nothing from it.

Sources (the CODA news article by Synced / 机器之心, mirrored by KuCoin News):
  [EPI]  section "CODA：「尾声」里藏着宝藏": the re-parameterisation applies to
         RoPE as well;
  [PRIM] section "五种「积木」和一套「乐高语言」": RoPE is one of the
         element-wise epilogue transforms.
The pages do not write RoPE out.  Reading taken (the rotary embedding in its
original interleaved form, as in the LLaMA reference code): the output
columns are [Q | K | V], n_q and n_k columns of heads of width d (V is not
rotated); inside each Q or K head the column pairs (2i, 2i + 1),
i = 0 .. d/2 - 1, are rotated by the angle p theta_i, p the row's position,
theta_i = base^(-2i / d):

    y'_2i   = y_2i cos(p theta_i) - y_2i+1 sin(p theta_i)
    y'_2i+1 = y_2i sin(p theta_i) + y_2i+1 cos(p theta_i)

The backward of this linear map is its transpose, the rotation by -p theta_i.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .chain import forward


def rope_angles(positions, d_head: int, base: float) -> np.ndarray:
    """angle[row, i] = p_row * base^(-2i / d_head), float64."""
    i = np.arange(d_head // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d_head)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def rope_rotate(Y, positions, n_q: int, n_k: int, d_head: int, base: float) -> np.ndarray:
    """Y with its first n_q + n_k columns rotated head by head."""
    Y = np.array(Y, dtype=np.float64)
    ang = rope_angles(positions, d_head, base)
    c, s = np.cos(ang), np.sin(ang)
    for start in range(0, n_q + n_k, d_head):
        head = Y[:, start:start + d_head]
        even, odd = head[:, 0::2].copy(), head[:, 1::2].copy()
        head[:, 0::2] = even * c - odd * s
        head[:, 1::2] = even * s + odd * c
    return Y


def rope_backward(G, positions, n_q: int, n_k: int, d_head: int, base: float) -> np.ndarray:
    """Gradient of the unrotated values from the gradient G of the rotated
    ones: each pair turned back by its angle (the rotation's transpose)."""
    return rope_rotate(G, -np.asarray(positions, dtype=np.float64), n_q, n_k, d_head, base)


def forward_rope(A, W1, R, g, Wqkv, eps: float, positions, n_q: int, n_k: int, d_head: int, base: float,
                 rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """The chain [EPI] with the QKV projection as second GEMM, then RoPE:
    float64 H, r, Y (before RoPE) and Yr (after)."""
    if n_q % d_head or n_k % d_head or d_head % 2:
        raise ValueError("Q and K widths must be whole heads of even width")
    out = forward(A, W1, R, g, Wqkv, eps, rows=rows)
    p = np.asarray(positions)
    if rows is not None:
        p = p[np.asarray(rows, dtype=np.int64)]
    out["Yr"] = rope_rotate(out["Y"], p, n_q, n_k, d_head, base)
    return out
