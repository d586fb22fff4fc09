"""Plain fp64 CPU oracle of the chain ending in a cross-entropy loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the test-suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP path and imports nothing from it.

Sources (the CODA news article by Synced / 机器之心, mirrored by KuCoin News):
  [EPI]  section "CODA：「尾声」里藏着宝藏": the re-parameterisation applies to
         the cross-entropy loss as well;
  [PRIM] section "五种「积木」和一套「乐高语言」": tile reductions include a
         tile log-sum-exp, and the stateful transform keeps the max and
         sum-exp statistics of online normalisation.
Reading taken: the chain's second GEMM is the LM head (W2 = W_vocab [D, V]),
its output the logits Y; per row i with target class t_i

    lse_i  = log sum_j exp(Y_ij)         (evaluated as m + log sum exp(Y - m))
    loss_i = lse_i - Y_i,t_i

the per-token cross-entropy (no reduction over tokens, no label smoothing).

Backward: for an upstream gradient dloss_i per token (1/M for a mean over
tokens), the gradient of sum_i dloss_i loss_i with respect to the logits is
dloss_i (softmax(Y_i) - onehot(t_i)); the chain's own backward takes it from
there as its dY.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .chain import backward, forward


def logsumexp_rows(Y) -> np.ndarray:
    """log sum_j exp(Y_ij) per row, with the row maximum factored out."""
    Y = np.asarray(Y, dtype=np.float64)
    m = np.max(Y, axis=1)
    return m + np.log(np.sum(np.exp(Y - m[:, None]), axis=1))


def cross_entropy_rows(Y, targets) -> Dict[str, np.ndarray]:
    Y = np.asarray(Y, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    if t.shape != (Y.shape[0],) or np.any(t < 0) or np.any(t >= Y.shape[1]):
        raise ValueError("one target class in [0, V) per row")
    lse = logsumexp_rows(Y)
    tgt = Y[np.arange(Y.shape[0]), t]
    return {"lse": lse, "target_logit": tgt, "loss": lse - tgt}


def forward_ce(A, W1, R, g, Wv, eps: float, targets, rows: Optional[Sequence[int]] = None,
               block_rows: int = 1024) -> Dict[str, np.ndarray]:
    """The chain [EPI] with the LM head as second GEMM, then the per-token
    cross-entropy: float64 H, r, Y (logits), lse, target_logit, loss."""
    out = forward(A, W1, R, g, Wv, eps, rows=rows, block_rows=block_rows)
    t = np.asarray(targets, dtype=np.int64)
    if rows is not None:
        t = t[np.asarray(rows, dtype=np.int64)]
    out.update(cross_entropy_rows(out["Y"], t))
    return out


def cross_entropy_grad(Y, targets, dloss) -> np.ndarray:
    """d(sum_i dloss_i loss_i)/dY = dloss_i (e^(Y_ij - lse_i) - [j == t_i])."""
    Y = np.asarray(Y, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    if t.shape != (Y.shape[0],) or np.any(t < 0) or np.any(t >= Y.shape[1]):
        raise ValueError("one target class in [0, V) per row")
    p = np.exp(Y - logsumexp_rows(Y)[:, None])
    p[np.arange(Y.shape[0]), t] -= 1.0
    return p * np.asarray(dloss, dtype=np.float64)[:, None]


def backward_ce(A, W1, R, g, Wv, eps: float, targets, dloss) -> Dict[str, np.ndarray]:
    """Gradients of sum_i dloss_i loss_i through the chain: dY from the loss,
    then the chain's backward (dA, dR, dW1, dW2 = dWv, dg)."""
    Y = forward(A, W1, R, g, Wv, eps)["Y"]
    dY = cross_entropy_grad(Y, targets, dloss)
    out = backward(dY, A, W1, R, g, Wv, eps)
    out["dY"] = dY
    out["Y"] = Y
    return out
