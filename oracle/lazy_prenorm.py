"""Plain fp64 reference of the Lazy Pre-Norm GEMM.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

[FreeNorm] (the PyTorch blog "Towards Free Normalization: Fusing Normalization
into GEMM and Attention Kernels"), section 2 (Lazy Pre-Norm):

    C = rmsnorm(A) @ B,   rmsnorm(A) = A * rstd(A)[:, None],
    rstd(A) = rsqrt(sum(A**2, dim=-1) / A.shape[-1] + 1e-5)

(no element-wise affine weight).  The method computes A @ B and the row sums
of squares in the same pass over K and scales each output row by rstd at the
end; that equals the definition exactly in real arithmetic (a row scaling
commutes with the product), so this reference is the definition itself,
written out.

Reading (the page fixes the math, not the memory layout): B is passed as its
transpose W = B^T, [N, K] row-major -- the layout of a linear layer's weight
-- so C[m, n] = rstd[m] * sum_k A[m, k] W[n, k].
"""

import numpy as np

EPS = 1e-5  # [FreeNorm] section 2's rstd


def rstd(a, eps=EPS):
    """rstd of every row: 1 / sqrt(mean of the squares + eps)."""
    a = np.asarray(a, np.float64)
    return 1.0 / np.sqrt(np.mean(a * a, axis=1) + eps)


def rmsnorm(a, eps=EPS):
    """rmsnorm(A) = A * rstd(A)[:, None] (no affine weight)."""
    a = np.asarray(a, np.float64)
    return a * rstd(a, eps)[:, None]


def lazy_prenorm_gemm(a, w, eps=EPS):
    """C = rmsnorm(A) @ W^T for A [M, K], W [N, K].  Returns (C [M, N], rstd [M])."""
    a = np.asarray(a, np.float64)
    w = np.asarray(w, np.float64)
    rs = rstd(a, eps)
    return rmsnorm(a, eps) @ w.T, rs
