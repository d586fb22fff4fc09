"""Plain fp64 CPU oracle of the chain with a SwiGLU epilogue, and its backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the test-suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP path and imports nothing from it.

Sources (the CODA news article by Synced / 机器之心, mirrored by KuCoin News):
  [EPI] section "CODA：「尾声」里藏着宝藏": the same re-parameterisation as
        for RMSNorm applies to SwiGLU, and to the backward pass.
  [EXP] section "实验结果": SwiGLU epilogue compositions and the SwiGLU
        backward are among the measured kernels.
The pages do not write SwiGLU out.  Reading (the LLaMA feed-forward gate):
the second GEMM's weight is W2 = [W_gate | W_up], columns [0, F) and
[F, 2F), and

    Y = X_n W2                       (the plain chain, oracle.chain.forward)
    Z = silu(Y[:, :F]) * Y[:, F:]    silu(x) = x * sigmoid(x) = x / (1 + e^-x)

Backward of Z with respect to Y, given dZ = dL/dZ (s = sigmoid):

    dY_up   = dZ * silu(Y_gate)
    dY_gate = dZ * Y_up * silu'(Y_gate),   silu'(x) = s(x) (1 + x (1 - s(x)))

after which the chain's own backward (oracle.chain.backward) takes dY.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .chain import backward, forward


def sigmoid(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def split(Y: np.ndarray):
    """(gate, up) halves of the second GEMM's output columns."""
    N2 = Y.shape[1]
    if N2 % 2:
        raise ValueError("the gate||up output needs an even width")
    F = N2 // 2
    return Y[:, :F], Y[:, F:]


def forward_swiglu(A, W1, R, g, W2, eps: float, rows: Optional[Sequence[int]] = None,
                   block_rows: int = 1024) -> Dict[str, np.ndarray]:
    """The chain [EPI] followed by the SwiGLU gate: float64 H, r, Y[m,2F], Z[m,F]."""
    out = forward(A, W1, R, g, W2, eps, rows=rows, block_rows=block_rows)
    yg, yu = split(out["Y"])
    out["Z"] = silu(yg) * yu
    return out


def swiglu_dy(dZ, Y) -> np.ndarray:
    """dL/dY[m,2F] from dL/dZ[m,F] through Z = silu(Y_gate) * Y_up."""
    dZ = np.asarray(dZ, dtype=np.float64)
    yg, yu = split(np.asarray(Y, dtype=np.float64))
    s = sigmoid(yg)
    d_gate = dZ * yu * (s * (1.0 + yg * (1.0 - s)))
    d_up = dZ * (yg * s)
    return np.concatenate([d_gate, d_up], axis=1)


def backward_swiglu(dZ, A, W1, R, g, W2, eps: float) -> Dict[str, np.ndarray]:
    """Gradients of <dZ, Z>: dY through the gate, then the chain's backward."""
    Y = forward(A, W1, R, g, W2, eps)["Y"]
    dY = swiglu_dy(dZ, Y)
    out = backward(dY, A, W1, R, g, W2, eps)
    out["dY"] = dY
    out["Y"] = Y
    return out
