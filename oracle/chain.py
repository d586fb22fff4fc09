"""Plain fp64 CPU oracle of the GEMM-Residual-RMSNorm-GEMM chain and its backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the test-suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP path and imports nothing from it.

Sources (a web news article on CODA, "Rewriting Transformer Blocks as
GEMM-Epilogue Programs", published by Synced / 机器之心 and mirrored by
KuCoin News):
  [EPI]  section "CODA：「尾声」里藏着宝藏" (the epilogue section): the
         GEMM-RMSNorm-GEMM pattern is a GEMM, a residual add, an RMS
         normalisation and a second GEMM, run as separate operators; the
         RMSNorm row scale r is one scalar per row.  The same section says the
         backward pass admits the same re-parameterisation.
  [PRIM] section "五种「积木」和一套「乐高语言」": the RMSNorm weight is a
         broadcast vector.
The fused method reaches the same result as the plain chain (it only moves
where r is applied), so this oracle is the plain, unfused definition, written
step by step in float64:

    C  = A @ W1
    H  = C + R
    ms = mean_j H_ij^2               (mean over the true width D)
    r  = 1 / sqrt(ms + eps)
    Xn = diag(r) @ H @ diag(g)       (multiplicative weight, no bias)
    Y  = Xn @ W2

The backward is reverse-mode differentiation of those same steps, one step at
a time, in reverse order.

Every function accepts any real dtype and computes in float64.  Rows are
independent in every forward step, so `forward(..., rows=idx)` computes the
exact result for a subset of rows.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def forward(A, W1, R, g, W2, eps: float, rows: Optional[Sequence[int]] = None,
            block_rows: int = 1024) -> Dict[str, np.ndarray]:
    """Unfused forward chain [EPI]: returns float64 H[m,D], r[m], Y[m,N2].

    A[M,K], W1[K,D], R[M,D], g[D], W2[D,N2].  `rows` restricts the result to
    those rows (exact: no step mixes rows); blocks of `block_rows` rows bound
    host memory for large M.
    """
    W1 = _f64(W1)
    W2 = _f64(W2)
    g = _f64(g)
    A = np.asarray(A)
    R = np.asarray(R)
    M = A.shape[0]
    K, D = W1.shape
    D2, N2 = W2.shape
    if A.shape[1] != K or R.shape != (M, D) or D2 != D or g.shape != (D,):
        raise ValueError("shape mismatch")
    idx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    n = idx.shape[0]
    H = np.empty((n, D))
    r = np.empty(n)
    Y = np.empty((n, N2))
    for s in range(0, n, block_rows):
        sel = idx[s:s + block_rows]
        C = _f64(A[sel]) @ W1                    # first GEMM
        Hb = C + _f64(R[sel])                    # residual add
        ms = np.mean(Hb * Hb, axis=1)            # mean square over D
        rb = 1.0 / np.sqrt(ms + eps)             # per-row RMSNorm scale
        Xn = (Hb * rb[:, None]) * g[None, :]     # normalise, then weight
        Y[s:s + len(sel)] = Xn @ W2              # second GEMM
        H[s:s + len(sel)] = Hb
        r[s:s + len(sel)] = rb
    return {"H": H, "r": r, "Y": Y}


def backward(dY, A, W1, R, g, W2, eps: float) -> Dict[str, np.ndarray]:
    """Gradients of <dY, Y> for the unfused chain, reverse-mode step by step.

    Returns float64 dA[M,K], dR[M,D], dW1[K,D], dW2[D,N2], dg[D], and the
    intermediates dH[M,D], r[M], s[M] (s_i = sum_j g_j G_ij H_ij with
    G = dY W2^T) that a fused backward forms on the way.
    """
    A = _f64(A)
    R = _f64(R)
    W1 = _f64(W1)
    W2 = _f64(W2)
    g = _f64(g)
    dY = _f64(dY)
    D = W1.shape[1]
    # forward, keeping what the backward needs
    C = A @ W1
    H = C + R
    ms = np.mean(H * H, axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    Nh = H * r[:, None]                  # normalised rows, before the weight
    Xn = Nh * g[None, :]
    # Y = Xn @ W2
    dXn = dY @ W2.T
    dW2 = Xn.T @ dY
    # Xn = Nh * g
    dg = np.sum(dXn * Nh, axis=0)
    dNh = dXn * g[None, :]
    # Nh_ij = H_ij r_i,  r_i = (mean_k H_ik^2 + eps)^(-1/2),
    # d r_i / d H_ik = -r_i^3 H_ik / D
    s = np.sum(dNh * H, axis=1)
    dH = dNh * r[:, None] - (r ** 3 * s / D)[:, None] * H
    # H = C + R
    dC = dH
    dR = dH.copy()
    # C = A @ W1
    dA = dC @ W1.T
    dW1 = A.T @ dC
    return {"dA": dA, "dR": dR, "dW1": dW1, "dW2": dW2, "dg": dg,
            "dH": dH, "r": r, "s": s}
