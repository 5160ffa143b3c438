"""Brute-force mHC forward in pure-Python loops, for tiny inputs only.

An independent second computation used to pin the fp64 oracle (see
test_oracle_pins.py).  It deliberately computes differently from the oracle:

* X is held per row as a list of n streams, each a list of C values, and phi as
  phi[j][c][k] (the weight for stream j, channel c, output column k), so the
  stream-major reading of X_t and phi is expressed through explicit (j, c)
  indexing rather than a flat reshape;
* every sum is an explicit Python loop (no BLAS, no numpy);
* Sinkhorn-Knopp runs in its textbook diagonal-scaling form (Sinkhorn & Knopp,
  1967): with K = exp(h), v <- 1, then per iteration u = 1 / (K v) and
  v = 1 / (K^T u); the result is diag(u) K diag(v).  In exact arithmetic this
  equals alternating row then column normalisation of K, iteration by
  iteration, as the page "mHC 算法分析 & cutile 高效实现" (section 2.4) states it.
"""

import math


def brute_row(xs, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
              f, n, C, iters=20):
    """One row.  xs[j][c]: stream j, channel c.  phi[j][c][k].  b_res[i][j].
    f[c]: the layer output for this row.  Returns a dict of plain lists."""
    N = n * n + 2 * n
    s = [0.0] * N
    q = 0.0
    for j in range(n):
        for c in range(C):
            xv = xs[j][c]
            q += xv * xv
            for k in range(N):
                s[k] += xv * phi[j][c][k]
    r = math.sqrt(q / (n * C))
    pre = [1.0 / (1.0 + math.exp(-(alpha_pre * s[i] / r + b_pre[i]))) for i in range(n)]
    post = [2.0 / (1.0 + math.exp(-(alpha_post * s[n + i] / r + b_post[i]))) for i in range(n)]
    kmat = [[math.exp(alpha_res * s[2 * n + i * n + j] / r + b_res[i][j]) for j in range(n)]
            for i in range(n)]
    v = [1.0] * n
    u = [1.0] * n
    for _ in range(iters):
        u = [1.0 / sum(kmat[i][j] * v[j] for j in range(n)) for i in range(n)]
        v = [1.0 / sum(kmat[i][j] * u[i] for i in range(n)) for j in range(n)]
    hres = [[u[i] * kmat[i][j] * v[j] for j in range(n)] for i in range(n)]
    fpre = [sum(pre[i] * xs[i][c] for i in range(n)) for c in range(C)]
    xnext = [[sum(hres[i][j] * xs[j][c] for j in range(n)) + post[i] * f[c]
              for c in range(C)] for i in range(n)]
    return {"logits": s, "r": r, "pre": pre, "post": post, "res": hres,
            "F_pre": fpre, "X_next": xnext}


def sinkhorn_scaling(h, iters=20):
    """Diagonal-scaling Sinkhorn-Knopp on one n x n matrix of floats (lists)."""
    n = len(h)
    kmat = [[math.exp(h[i][j]) for j in range(n)] for i in range(n)]
    v = [1.0] * n
    u = [1.0] * n
    for _ in range(iters):
        u = [1.0 / sum(kmat[i][j] * v[j] for j in range(n)) for i in range(n)]
        v = [1.0 / sum(kmat[i][j] * u[i] for i in range(n)) for j in range(n)]
    return [[u[i] * kmat[i][j] * v[j] for j in range(n)] for i in range(n)]
