"""Pure-Python brute force of the GEMM-Residual-RMSNorm-GEMM chain (tiny inputs only).

An independent second implementation used to pin the NumPy oracle: explicit
loops and math.fsum (exactly rounded sums), no NumPy arithmetic.  It follows
the plain definition of the chain (CODA news article, epilogue section):
H = A W1 + R, r_i = 1/sqrt(mean_j H_ij^2 + eps), Y = diag(r) H diag(g) W2.
"""
import math


def chain(A, W1, R, g, W2, eps):
    M, K = len(A), len(A[0])
    D = len(W1[0])
    N2 = len(W2[0])
    H = [[math.fsum([A[i][k] * W1[k][j] for k in range(K)] + [R[i][j]]) for j in range(D)]
         for i in range(M)]
    r = [1.0 / math.sqrt(math.fsum(h * h for h in H[i]) / D + eps) for i in range(M)]
    Y = [[math.fsum(H[i][j] * r[i] * g[j] * W2[j][n] for j in range(D)) for n in range(N2)]
         for i in range(M)]
    return H, r, Y
