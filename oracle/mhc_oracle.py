"""Plain, slow, fp64 reference of the mHC residual-stream forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only tests, the smoke check and the
bench's CPU-baseline leg may call this.  It shares no code with the HIP library.

Every function follows one step of the method as [mHC-cutile] section 2 states
it ([mHC-cutile] = the page "mHC 算法分析 & cutile 高效实现"; [FreeNorm] = the
PyTorch blog "Towards Free Normalization: Fusing Normalization into GEMM and
Attention Kernels").  Arithmetic is numpy float64; bf16 inputs are widened
exactly (bf16 -> fp32 is a 16-bit shift, fp32 -> fp64 is exact).  Outputs are
never rounded back to a narrower type, except by round_to_bf16, which a test
calls where one layer's X_next becomes the next layer's bf16 input.

Notation (from [mHC-cutile] section 2):
  B  rows (batch x sequence),  n  expansion rate,  C  hidden size,
  X  [B, n*C], stream-major: stream j is columns [j*C, (j+1)*C),
  phi [n*C, N] with N = n*n + 2n,
  logits columns are [pre (n) | post (n) | res (n*n, row-major (i, j))].

Readings taken where the page leaves a step open (each is listed in the design
notes of the repository):
  * r carries no epsilon (section 2.2 defines it as a plain root-mean-square).
  * sigmoid is the textbook logistic 1 / (1 + e^-z).
  * Sinkhorn-Knopp runs exactly 20 (row, column) normalisation pairs, rows
    first, so the last operation is a column normalisation (the iteration in
    the kernels of sections 4.3 and 5.3); exp is applied with no max shift.
  * H_res acts as out_i = sum_j H_res[i, j] * X_j (the apply kernels of
    sections 4.4 and 5.4 index it this way).

Parity status: every function here is pinned by tests in
tests/test_oracle_pins.py (brute force, closed forms, invariants); none is
"parity unpinned".
"""

import numpy as np

# [mHC-cutile] section 2.4 gives "about 20" iterations; the kernels of
# sections 4.3 and 5.3 fix the count at 20.
SINKHORN_ITERS = 20


def bf16_bits_to_f64(bits):
    """Widen raw bf16 bit patterns (uint16) to float64 exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """float64 -> the nearest bf16 value (ties to even), as float64.

    [mHC-cutile] section 2.5 hands X_next to the next layer as that layer's
    X_t, which is a bf16 tensor in every workload here; rounding to nearest,
    ties to even, is the reading taken for that conversion.  bf16 keeps 8
    significant bits (7 stored) and fp32's exponent range; values here are
    far from its overflow and subnormal ranges, which this does not model.
    Rounding straight from float64 (not through fp32) avoids double
    rounding."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0) / 256.0      # 8 significant bits, ties to even
    return np.ldexp(q, e)


def coefficient_logits(x, phi):
    """O1 -- [mHC-cutile] section 2.1: one product X_t . phi_t gives all
    n*n + 2n unconstrained logits of a row at once.  x [B, nC], phi [nC, N]."""
    return np.asarray(x, np.float64) @ np.asarray(phi, np.float64)


def row_sum_squares(x):
    """O1' -- [mHC-cutile] section 2.2: the per-row sum of X_t squared."""
    x = np.asarray(x, np.float64)
    return np.sum(x * x, axis=1)


def rms_scale(q, n, C):
    """O2 -- [mHC-cutile] section 2.2: r = sqrt(sum(X_t^2) / (n C)), one
    scalar per row, with no epsilon."""
    return np.sqrt(np.asarray(q, np.float64) / float(n * C))


def scale_bias(s, r, alpha, b):
    """O3 (linear part) -- [mHC-cutile] section 2.3: alpha * logit / r + b,
    elementwise; r broadcasts over the columns of its row."""
    s = np.asarray(s, np.float64)
    r = np.asarray(r, np.float64).reshape(-1, *([1] * (s.ndim - 1)))
    return float(alpha) * s / r + np.asarray(b, np.float64)


def sigmoid(z):
    """Textbook logistic function 1 / (1 + e^-z) ([mHC-cutile] section 2.4
    uses it without defining it)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def gate_coefficients(s, r, alpha_pre, alpha_post, alpha_res,
                      b_pre, b_post, b_res, n):
    """O3 -- [mHC-cutile] sections 2.3 and 2.4.

    s: logits [B, n*n + 2n] in the column order of section 2.1 (pre, post,
    res).  Returns (H_pre [B, n], H_post [B, n], h_res [B, n, n]) where H_pre =
    sigmoid(.), H_post = 2 * sigmoid(.), and h_res is the biased, scaled res
    logit block before Sinkhorn-Knopp (no gate)."""
    s = np.asarray(s, np.float64)
    B = s.shape[0]
    pre = scale_bias(s[:, 0:n], r, alpha_pre, b_pre)
    post = scale_bias(s[:, n:2 * n], r, alpha_post, b_post)
    res = scale_bias(s[:, 2 * n:2 * n + n * n], r, alpha_res,
                     np.asarray(b_res, np.float64).reshape(n * n))
    return sigmoid(pre), 2.0 * sigmoid(post), res.reshape(B, n, n)


def sinkhorn_knopp(h_res, iters=SINKHORN_ITERS):
    """O4 -- [mHC-cutile] section 2.4 (and the single-kernel iteration of
    section 3.3): start from exp(h_res), then `iters` times normalise every
    row to sum 1 and then every column to sum 1.  h_res [..., n, n]."""
    m = np.exp(np.asarray(h_res, np.float64))
    for _ in range(iters):
        m = m / np.sum(m, axis=-1, keepdims=True)   # row i divided by sum_l m[i, l]
        m = m / np.sum(m, axis=-2, keepdims=True)   # column j divided by sum_l m[l, j]
    return m


def coefficients(x, phi, alpha_pre, alpha_post, alpha_res,
                 b_pre, b_post, b_res, n, C, iters=SINKHORN_ITERS):
    """Steps (1)-(3) of the forward for a block of rows.

    Returns dict(logits [B, N], r [B], H [B, N]) with H laid out like the
    logits: [H_pre | H_post | H_res row-major]."""
    s = coefficient_logits(x, phi)
    r = rms_scale(row_sum_squares(x), n, C)
    h_pre, h_post, h_res = gate_coefficients(
        s, r, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, n)
    H = np.concatenate(
        [h_pre, h_post, sinkhorn_knopp(h_res, iters).reshape(-1, n * n)], axis=1)
    return {"logits": s, "r": r, "H": H}


def split_h(H, n):
    """View a [B, N] coefficient block as (H_pre [B,n], H_post [B,n],
    H_res [B,n,n]) using the column order of [mHC-cutile] section 2.1."""
    H = np.asarray(H, np.float64)
    return (H[:, 0:n], H[:, n:2 * n],
            H[:, 2 * n:2 * n + n * n].reshape(-1, n, n))


def pre_mix(x, H_pre, n, C):
    """O5 -- [mHC-cutile] section 2.5 (first step): F_pre = sum_i H_pre[i] X_t[i],
    the n streams collapsed to one [B, C] input for the layer."""
    x3 = np.asarray(x, np.float64).reshape(-1, n, C)
    H_pre = np.asarray(H_pre, np.float64)
    out = np.zeros((x3.shape[0], C))
    for i in range(n):
        out += H_pre[:, i:i + 1] * x3[:, i, :]
    return out


def post_res(x, f_out, H_post, H_res, n, C):
    """O6 -- [mHC-cutile] section 2.5 (third step) and section 3.4:
    X_next[i] = sum_j H_res[i, j] X_t[j] + H_post[i] F_out.  Returns [B, n*C]."""
    x3 = np.asarray(x, np.float64).reshape(-1, n, C)
    f = np.asarray(f_out, np.float64)
    H_post = np.asarray(H_post, np.float64)
    H_res = np.asarray(H_res, np.float64)
    out = np.zeros_like(x3)
    for i in range(n):
        acc = H_post[:, i:i + 1] * f
        for j in range(n):
            acc = acc + H_res[:, i, j:j + 1] * x3[:, j, :]
        out[:, i, :] = acc
    return out.reshape(-1, n * C)


def forward(x, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
            f_out, n, C, iters=SINKHORN_ITERS, chunk=256):
    """The whole forward on float64 inputs, in row chunks so a large X is never
    widened at once.  Rows are independent in every step, so chunking changes
    nothing but memory use.  x [B, nC], phi [nC, N], f_out [B, C].

    Returns dict(logits, r, H, F_pre, X_next), all float64."""
    x = np.asarray(x)
    B = x.shape[0]
    N = n * n + 2 * n
    out = {"logits": np.empty((B, N)), "r": np.empty(B), "H": np.empty((B, N)),
           "F_pre": np.empty((B, C)), "X_next": np.empty((B, n * C))}
    phi = np.asarray(phi, np.float64)
    for lo in range(0, B, chunk):
        hi = min(B, lo + chunk)
        xc = np.asarray(x[lo:hi], np.float64)
        co = coefficients(xc, phi, alpha_pre, alpha_post, alpha_res,
                          b_pre, b_post, b_res, n, C, iters)
        h_pre, h_post, h_res = split_h(co["H"], n)
        out["logits"][lo:hi] = co["logits"]
        out["r"][lo:hi] = co["r"]
        out["H"][lo:hi] = co["H"]
        out["F_pre"][lo:hi] = pre_mix(xc, h_pre, n, C)
        out["X_next"][lo:hi] = post_res(xc, np.asarray(f_out[lo:hi], np.float64),
                                        h_post, h_res, n, C)
    return out
