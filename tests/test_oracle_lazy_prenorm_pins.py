"""Pins for the Lazy Pre-Norm GEMM reference (oracle/lazy_prenorm.py), checked
against what the definition and the mathematics fix, independently of the
oracle's code: a pure-Python loop computation, torch's rms_norm followed by a
matrix product (library routines), closed forms, and the row-scaling identity
the method rests on.  A planted mistake must trip at least one pin.

[FreeNorm] = "Towards Free Normalization: Fusing Normalization into GEMM and
Attention Kernels", section 2.
"""

import math

import numpy as np
import pytest
import torch

import oracle.lazy_prenorm as LP

pytestmark = pytest.mark.cpu


def _brute(a, w, eps=1e-5):
    M, K = len(a), len(a[0])
    N = len(w)
    rs = []
    for m in range(M):
        ss = 0.0
        for k in range(K):
            ss += a[m][k] * a[m][k]
        rs.append(1.0 / math.sqrt(ss / K + eps))
    c = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += (a[m][k] * rs[m]) * w[n][k]
            c[m][n] = acc
    return c, rs


def pin_brute_force(m):
    rng = np.random.default_rng(3)
    for M, K, N in ((3, 5, 4), (2, 7, 7), (4, 3, 6)):
        a = rng.standard_normal((M, K)) * rng.uniform(0.01, 3.0, (M, 1))
        w = rng.standard_normal((N, K))
        c, rs = m.lazy_prenorm_gemm(a, w)
        bc, brs = _brute(a.tolist(), w.tolist())
        np.testing.assert_allclose(rs, brs, rtol=1e-13)
        np.testing.assert_allclose(c, bc, rtol=1e-12, atol=1e-13)


def pin_torch_rms_norm(m):
    """torch.nn.functional.rms_norm (x * rsqrt(mean(x^2) + eps)) then @ W^T."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal((17, 64)) * rng.uniform(0.001, 10.0, (17, 1))
    w = rng.standard_normal((9, 64))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(a), (64,), eps=1e-5) @ torch.from_numpy(w).T
    c, _ = m.lazy_prenorm_gemm(a, w)
    np.testing.assert_allclose(c, ref.numpy(), rtol=1e-12, atol=1e-12)


def pin_closed_forms(m):
    K = 8
    a = np.array([[2.0] * K, [-0.5] * K, [0.0] * K])
    rs = m.rstd(a)
    np.testing.assert_allclose(rs, [1 / math.sqrt(4 + 1e-5), 1 / math.sqrt(0.25 + 1e-5),
                                    1 / math.sqrt(1e-5)], rtol=1e-15)
    # W = I: C is rmsnorm(A) itself; a zero row stays zero (eps keeps rstd finite)
    rng = np.random.default_rng(8)
    b = rng.standard_normal((5, K))
    b[2] = 0.0
    c, _ = m.lazy_prenorm_gemm(b, np.eye(K))
    ms = np.mean(b * b, axis=1, keepdims=True)
    np.testing.assert_allclose(c, b / np.sqrt(ms + 1e-5), rtol=1e-14)
    assert np.all(c[2] == 0.0)


def pin_row_scaling_identity(m):
    """(A * rstd[:, None]) @ W^T = (A @ W^T) * rstd[:, None]: the property that
    lets the scaling wait until the end of the k-loop; rstd from the loop
    computation, not from the oracle."""
    rng = np.random.default_rng(9)
    a = rng.standard_normal((6, 40))
    w = rng.standard_normal((11, 40))
    _, brs = _brute(a.tolist(), [[0.0] * 40])
    lazy = (a @ w.T) * np.asarray(brs)[:, None]
    c, _ = m.lazy_prenorm_gemm(a, w)
    np.testing.assert_allclose(c, lazy, rtol=1e-12, atol=1e-13)


PINS = [pin_brute_force, pin_torch_rms_norm, pin_closed_forms, pin_row_scaling_identity]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(LP)


_orig = {k: getattr(LP, k) for k in ("rstd", "rmsnorm", "lazy_prenorm_gemm")}


def _mut_no_eps(a, eps=LP.EPS):
    a = np.asarray(a, np.float64)
    with np.errstate(divide="ignore"):
        return 1.0 / np.sqrt(np.mean(a * a, axis=1))


def _mut_sum_not_mean(a, eps=LP.EPS):
    a = np.asarray(a, np.float64)
    return 1.0 / np.sqrt(np.sum(a * a, axis=1) + eps)


def _mut_sqrt_not_rsqrt(a, eps=LP.EPS):
    a = np.asarray(a, np.float64)
    return np.sqrt(np.mean(a * a, axis=1) + eps)


def _mut_eps_outside(a, eps=LP.EPS):
    a = np.asarray(a, np.float64)
    return 1.0 / (np.sqrt(np.mean(a * a, axis=1)) + eps)


def _mut_w_not_transposed(a, w, eps=LP.EPS):
    a = np.asarray(a, np.float64)
    w = np.asarray(w, np.float64)
    rs = _orig["rstd"](a, eps)
    return _orig["rmsnorm"](a, eps) @ (w if w.shape[0] == a.shape[1] else w.T), rs


def _mut_normalize_w(a, w, eps=LP.EPS):        # the wrong operand normalised
    a = np.asarray(a, np.float64)
    w = np.asarray(w, np.float64)
    return a @ _orig["rmsnorm"](w, eps).T, _orig["rstd"](a, eps)


MUTATIONS = [("rstd", _mut_no_eps), ("rstd", _mut_sum_not_mean), ("rstd", _mut_sqrt_not_rsqrt),
             ("rstd", _mut_eps_outside), ("lazy_prenorm_gemm", _mut_w_not_transposed),
             ("lazy_prenorm_gemm", _mut_normalize_w)]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(LP, name, fn)
    tripped = []
    for pin in PINS:
        try:
            pin(LP)
        except (AssertionError, ValueError):
            tripped.append(pin.__name__)
    assert tripped, f"no pin catches {fn.__name__}"
