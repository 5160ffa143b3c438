"""GPU parity of the Lazy Pre-Norm GEMM (mhc_lazy_prenorm_gemm) against the
fp64 oracle (oracle.lazy_prenorm), on the same bf16 bytes.

[FreeNorm] = "Towards Free Normalization: Fusing Normalization into GEMM and
Attention Kernels", section 2: C = rmsnorm(A) @ B with B given as W = B^T.

Tolerance, derived from the arithmetic (bf16 x bf16 products are exact in
fp32; the kernel sums them in fp32 in some order, sums the squares of each row
in fp32, scales by rstd and rounds once to bf16):
  rstd     relative (K + 8) 2^-24  (an fp32 sum of K positive terms, then a few
           correctly- or nearly-correctly-rounded operations)
  C        |c - exact| <= 2^-8 |exact|                       (one bf16 rounding)
                        + 1.01 * (2 K 2^-24 rstd sum_k |A W|   (fp32 sum, any
                                  order, up to 2u per addition)
                                  + (K + 8) 2^-24 |exact|)   (rstd's error)
  plus a row-normwise check, ||c - exact|| <= 4e-3 ||exact|| per row, which a
  lost chunk of K or a misplaced tile would fail even where the element bound
  is loose.
Full-size workloads are checked on sampled rows (rows are independent), and
rstd on every row.
"""

import sys

import numpy as np
import pytest
import torch

import manifold_constrained_hyper_amd as mhc
import synth
from oracle import lazy_prenorm as LP

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    mhc.load()
    yield


# Both kernels: the eight-wave one (MHC_LPN_ALGO 0) and the four-wave one (1).
@pytest.fixture(autouse=True, params=[0, 1], ids=["w8", "w4"])
def lpn_algo(request, tune):
    tune.setenv("MHC_LPN_ALGO", request.param)
    return request.param


def _bf16_to_f64(t):
    return t.detach().to("cpu", torch.float32).double().numpy()


def _run(A, W, eps=1e-5, want_rstd=True):
    M, K = A.shape
    N = W.shape[0]
    C = torch.empty(M, N, dtype=torch.bfloat16, device=A.device)
    C.fill_(float("nan"))
    r = torch.full((M,), float("nan"), dtype=torch.float32, device=A.device) if want_rstd else None
    mhc.mhc_lazy_prenorm_gemm(M, N, K, A, W, C, r, eps=eps)
    torch.cuda.synchronize()
    return C, r


def _check(a64, w64, c_gpu, r_gpu, eps=1e-5, rows=None):
    """a64: fp64 [R, K] (the rows checked), w64: fp64 [N, K]; c_gpu bf16 [R, N]."""
    K = a64.shape[1]
    exact, rs = LP.lazy_prenorm_gemm(a64, w64, eps)
    c = _bf16_to_f64(c_gpu)
    assert np.all(np.isfinite(c)), "non-finite output"
    if r_gpu is not None:
        r = r_gpu.detach().cpu().double().numpy()
        np.testing.assert_allclose(r, rs, rtol=(K + 8) * U32, atol=0)
    absum = (np.abs(a64) @ np.abs(w64).T) * rs[:, None]
    tol = 2.0 ** -8 * np.abs(exact) + 1.01 * (2 * K * U32 * absum + (K + 8) * U32 * np.abs(exact))
    err = np.abs(c - exact)
    bad = err > tol
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} elements out of tolerance; first at row "
                             f"{rows[i] if rows is not None else i}, col {j}: gpu {c[i, j]} "
                             f"exact {exact[i, j]} tol {tol[i, j]}")
    num = np.linalg.norm(c - exact, axis=1)
    den = np.linalg.norm(exact, axis=1)
    nz = den > 0
    assert np.all(num[nz] <= 4e-3 * den[nz]), float(np.max(num[nz] / den[nz]))
    assert np.all(num[~nz] == 0)


# (M, N, K): several 256 x 256 tiles with ragged M and N, K spanning several
# 64-wide chunks with a ragged tail, single-piece K, single rows and columns.
SMALL = [
    (300, 264, 200),
    (256, 256, 64),
    (1, 8, 8),
    (17, 8, 520),
    (513, 520, 136),
    (1024, 768, 1536),
    (40, 1032, 72),
    (8, 16, 4104),
]


@pytest.mark.parametrize("M,N,K", SMALL, ids=[f"{m}x{n}x{k}" for m, n, k in SMALL])
def test_parity_small(M, N, K):
    _say(f"lazy_prenorm small M={M} N={N} K={K}")
    d = synth.make_lpn_inputs(M, N, K, seed=M * 7 + N * 3 + K)
    A = d["A"].cuda()
    W = d["W"].cuda()
    C, r = _run(A, W)
    _check(_bf16_to_f64(d["A"]), _bf16_to_f64(d["W"]), C, r)


def test_rstd_optional_and_deterministic():
    _say("lazy_prenorm rstd=NULL and determinism")
    d = synth.make_lpn_inputs(300, 264, 200, seed=11)
    A, W = d["A"].cuda(), d["W"].cuda()
    C1, r1 = _run(A, W)
    C2, _ = _run(A, W, want_rstd=False)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    C3, r3 = _run(A, W)
    assert torch.equal(C1.view(torch.int16), C3.view(torch.int16))
    assert torch.equal(r1, r3)


def test_degenerate_rows_and_eps():
    """A zero row gives rstd = eps^-1/2 and a zero output row; eps = 0 gives
    the un-regularised statistic (mHC's r is its reciprocal); rows of very
    different scales stay within the bar (the result does not depend on a
    row's scale)."""
    _say("lazy_prenorm degenerate rows")
    M, N, K = 40, 32, 192
    d = synth.make_lpn_inputs(M, N, K, seed=5)
    A = d["A"].clone()
    A[3] = 0
    A[7] *= 2.0 ** 40
    A[9] *= 2.0 ** -40
    A[11, :] = 0
    A[11, 5] = 1.0                                   # one non-zero element
    A[12] = 1.0                                      # constant row
    Ag, Wg = A.cuda(), d["W"].cuda()
    C, r = _run(Ag, Wg)
    _check(_bf16_to_f64(A), _bf16_to_f64(d["W"]), C, r)
    assert torch.all(C[3].float() == 0)
    assert abs(r[3].item() - 1e-5 ** -0.5) <= 1e-6 * 1e-5 ** -0.5
    A2 = A.clone()
    A2[3] = 0.5                                      # eps = 0 needs non-zero rows
    Ag2 = A2.cuda()
    C0, r0 = _run(Ag2, Wg, eps=0.0)
    _check(_bf16_to_f64(A2), _bf16_to_f64(d["W"]), C0, r0, eps=0.0)


def test_empty_batch():
    _say("lazy_prenorm M=0")
    W = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(0, 8, dtype=torch.bfloat16, device="cuda")
    assert mhc.mhc_lazy_prenorm_gemm(0, 8, 64, A, W, C, None) == mhc.MHC_OK


@pytest.mark.parametrize("name", sorted(synth.LPN_CONFIGS))
def test_parity_full_size_sampled(name):
    """The bench workloads at full size: sampled rows of C against the oracle
    (every column of those rows), rstd on every row."""
    cfg = synth.LPN_CONFIGS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    _say(f"lazy_prenorm full {name} M={M} N={N} K={K}")
    d = synth.make_lpn_inputs(M, N, K, seed=cfg["seed"], device="cuda")
    C, r = _run(d["A"], d["W"])
    w64 = _bf16_to_f64(d["W"])
    rng = np.random.default_rng(cfg["seed"])
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 60)]))
    idx = torch.from_numpy(rows).cuda()
    _check(_bf16_to_f64(d["A"][idx]), w64, C[idx], r[idx], rows=rows)
    # rstd of every row, in chunks
    rg = r.cpu().double().numpy()
    for lo in range(0, M, 2048):
        a = _bf16_to_f64(d["A"][lo:lo + 2048])
        np.testing.assert_allclose(rg[lo:lo + 2048], LP.rstd(a), rtol=(K + 8) * U32, atol=0)
