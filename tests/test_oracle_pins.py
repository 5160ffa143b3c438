"""Pins for the fp64 oracle: checks against what the method and the mathematics
fix, independent of the oracle's own code.

Page references: [mHC-cutile] = "mHC 算法分析 & cutile 高效实现" (the forward is
stated in its section 2; the kernels of sections 4 and 5 fix layouts, the
Sinkhorn order and count); [FreeNorm] = "Towards Free Normalization: Fusing
Normalization into GEMM and Attention Kernels", section 2 (Lazy Pre-Norm).

Every pin is a function of the oracle module, so the mutation test at the
bottom can re-run all of them against oracles with a planted mistake and
require that each mistake trips at least one pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle.mhc_oracle as ORACLE
from tests import brute_mhc

pytestmark = pytest.mark.cpu


# ----------------------------------------------------------------------------
# helpers (input construction only; no method arithmetic)
# ----------------------------------------------------------------------------

def _rand_problem(rng, n, C, B, alphas=(0.7, -0.4, 1.3)):
    K = n * C
    N = n * n + 2 * n
    x = rng.standard_normal((B, K))
    phi = rng.standard_normal((K, N)) / math.sqrt(K)
    b_pre = 0.3 * rng.standard_normal(n)
    b_post = 0.3 * rng.standard_normal(n)
    b_res = (np.eye(n) + 0.5 * rng.standard_normal((n, n))).reshape(-1)
    f = rng.standard_normal((B, C))
    return dict(x=x, phi=phi, alpha_pre=alphas[0], alpha_post=alphas[1],
                alpha_res=alphas[2], b_pre=b_pre, b_post=b_post, b_res=b_res,
                f_out=f, n=n, C=C)


def _oracle_forward(m, p, **kw):
    return m.forward(p["x"], p["phi"], p["alpha_pre"], p["alpha_post"], p["alpha_res"],
                     p["b_pre"], p["b_post"], p["b_res"], p["f_out"], p["n"], p["C"], **kw)


def _close(a, b, rtol=1e-12, atol=1e-12):
    np.testing.assert_allclose(np.asarray(a, np.float64), np.asarray(b, np.float64),
                               rtol=rtol, atol=atol)


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_brute_force(m):
    """Whole forward against the pure-Python loop computation at n = 1, 2, 4."""
    rng = np.random.default_rng(7)
    for n, C, B in ((1, 8, 3), (2, 8, 3), (2, 5, 2), (4, 6, 2)):
        p = _rand_problem(rng, n, C, B)
        o = _oracle_forward(m, p)
        for b in range(B):
            xs = [[p["x"][b, j * C + c] for c in range(C)] for j in range(n)]
            phi = [[[p["phi"][j * C + c, k] for k in range(n * n + 2 * n)]
                    for c in range(C)] for j in range(n)]
            bres = [[p["b_res"][i * n + j] for j in range(n)] for i in range(n)]
            ref = brute_mhc.brute_row(xs, phi, p["alpha_pre"], p["alpha_post"], p["alpha_res"],
                                      list(p["b_pre"]), list(p["b_post"]), bres,
                                      list(p["f_out"][b]), n, C)
            _close(o["logits"][b], ref["logits"])
            _close(o["r"][b], ref["r"])
            h = o["H"][b]
            _close(h[0:n], ref["pre"])
            _close(h[n:2 * n], ref["post"])
            _close(h[2 * n:].reshape(n, n), ref["res"])
            _close(o["F_pre"][b], ref["F_pre"])
            _close(o["X_next"][b].reshape(n, C), ref["X_next"])


def pin_one_hot_phi(m):
    """phi with a single 1 per column selects one entry of X: logit k equals
    X[b, stream j_k, channel c_k] exactly (pins the product's orientation and
    the stream-major layout of X_t and phi, [mHC-cutile] sections 2 and 2.1)."""
    rng = np.random.default_rng(11)
    n, C, B = 4, 16, 5
    K, N = n * C, n * n + 2 * n
    x = rng.standard_normal((B, K))
    phi = np.zeros((K, N))
    picks = [(int(rng.integers(n)), int(rng.integers(C))) for _ in range(N)]
    for k, (j, c) in enumerate(picks):
        phi[j * C + c, k] = 1.0
    s = m.coefficient_logits(x, phi)
    for k, (j, c) in enumerate(picks):
        assert np.array_equal(s[:, k], x[:, j * C + c])


def pin_rms_closed_forms(m):
    """r = sqrt(sum(X^2)/(nC)) with no epsilon ([mHC-cutile] section 2.2)."""
    n, C = 4, 32
    x = np.full((1, n * C), -3.0)
    _close(m.rms_scale(m.row_sum_squares(x), n, C), [3.0], rtol=1e-15)
    x = np.zeros((1, n * C))
    x[0, 77] = 5.0
    _close(m.rms_scale(m.row_sum_squares(x), n, C), [5.0 / math.sqrt(n * C)], rtol=1e-15)
    # no epsilon: an all-zero row has r == 0 exactly
    assert m.rms_scale(m.row_sum_squares(np.zeros((1, n * C))), n, C)[0] == 0.0


def pin_lazy_prenorm(m):
    """[FreeNorm] section 2: scaling rows before the product equals scaling the
    product's rows afterwards.  With alpha = 1 and zero bias the oracle's
    scaled logits must equal the logits of X / r (pins that 1/r divides)."""
    rng = np.random.default_rng(5)
    n, C, B = 2, 24, 6
    p = _rand_problem(rng, n, C, B)
    s = m.coefficient_logits(p["x"], p["phi"])
    r = m.rms_scale(m.row_sum_squares(p["x"]), n, C)
    lhs = m.scale_bias(s, r, 1.0, np.zeros(s.shape[1]))
    rhs = np.asarray(p["x"] / r[:, None]) @ p["phi"]
    _close(lhs, rhs, rtol=1e-12, atol=1e-13)


def pin_gates(m):
    """[mHC-cutile] section 2.4: H_pre = sigmoid, H_post = 2*sigmoid; with
    alpha = 0 the gates reduce to sigmoid(b) independent of X."""
    rng = np.random.default_rng(3)
    n, C, B = 4, 8, 4
    p = _rand_problem(rng, n, C, B)
    p0 = dict(p, alpha_pre=0.0, alpha_post=0.0, alpha_res=0.0)
    o = _oracle_forward(m, p0)
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))  # noqa: E731
    for b in range(B):
        _close(o["H"][b, 0:n], sig(p["b_pre"]), rtol=1e-15)
        _close(o["H"][b, n:2 * n], 2.0 * sig(p["b_post"]), rtol=1e-15)
    # ranges on a random problem
    o = _oracle_forward(m, p)
    assert np.all((o["H"][:, :n] > 0) & (o["H"][:, :n] < 1))
    assert np.all((o["H"][:, n:2 * n] > 0) & (o["H"][:, n:2 * n] < 2))


def pin_column_roles(m):
    """Column order [pre | post | res] ([mHC-cutile] section 2.1 and the
    column masks of the section 4.2 kernel): drive the pre logits strongly
    positive and the post logits strongly negative through a one-hot phi."""
    n, C = 2, 4
    K, N = n * C, n * n + 2 * n
    x = np.zeros((1, K))
    x[0, 0] = 1.0                 # r = 1 / sqrt(nC)
    phi = np.zeros((K, N))
    phi[0, 0:n] = 40.0            # pre logits
    phi[0, n:2 * n] = -40.0       # post logits
    o = m.forward(x, phi, 1.0, 1.0, 1.0, np.zeros(n), np.zeros(n), np.zeros(n * n),
                  np.zeros((1, C)), n, C)
    assert np.all(o["H"][0, 0:n] > 0.999999)
    assert np.all(o["H"][0, n:2 * n] < 1e-6)
    # the res block of a constant logit matrix is uniform 1/n
    _close(o["H"][0, 2 * n:], np.full(n * n, 1.0 / n), rtol=1e-14)


def _slow_matrix():
    # exp of this converges slowly under Sinkhorn-Knopp (nearly decomposable)
    return np.array([[6.0, 0.0, -5.0, 1.0],
                     [-4.0, 5.5, 0.0, -6.0],
                     [0.5, -6.0, 4.0, 2.0],
                     [-3.0, 1.0, -2.0, 7.0]])


def pin_sinkhorn_scaling_form(m):
    """Alternating normalisation equals the textbook diagonal-scaling form at
    exactly 20 iterations, on a matrix where 19 or 21 iterations differ."""
    h = _slow_matrix()
    got = m.sinkhorn_knopp(h[None], 20)[0]
    ref = np.array(brute_mhc.sinkhorn_scaling(h.tolist(), 20))
    _close(got, ref, rtol=1e-12, atol=1e-15)
    # sensitivity of this case to the iteration count (so the pin has teeth)
    r19 = np.array(brute_mhc.sinkhorn_scaling(h.tolist(), 19))
    r21 = np.array(brute_mhc.sinkhorn_scaling(h.tolist(), 21))
    assert np.max(np.abs(r19 - ref)) > 1e-6 and np.max(np.abs(r21 - ref)) > 1e-6
    # the default iteration count is the page's 20
    _close(m.sinkhorn_knopp(h[None])[0], ref, rtol=1e-12, atol=1e-15)


def pin_sinkhorn_column_last(m):
    """The last operation is a column normalisation: columns sum to 1 to
    rounding, rows only approximately on a slowly converging matrix."""
    h = _slow_matrix()
    got = m.sinkhorn_knopp(h[None], 20)[0]
    assert np.max(np.abs(got.sum(axis=0) - 1.0)) < 1e-14
    assert np.max(np.abs(got.sum(axis=1) - 1.0)) > 1e-8


def pin_sinkhorn_closed_forms(m):
    """n = 1 gives [[1]]; h = a*I + c*11^T has equal row and column sums after
    exp, so one step already lands on exp(h)/rowsum and stays there."""
    _close(m.sinkhorn_knopp(np.array([[[3.7]]]))[0], [[1.0]], rtol=0, atol=1e-15)
    for n, a, c in ((4, 2.0, 0.3), (8, 1.5, -0.7), (3, -1.0, 2.0)):
        h = a * np.eye(n) + c
        got = m.sinkhorn_knopp(h[None])[0]
        d = math.exp(a) / (math.exp(a) + n - 1)
        o = 1.0 / (math.exp(a) + n - 1)
        _close(got, np.where(np.eye(n) > 0, d, o), rtol=1e-14)


def pin_sinkhorn_invariants(m):
    """The result is D1 exp(h) D2 for positive diagonals D1, D2, so every
    cross ratio H_ij H_kl / (H_il H_kj) equals exp(h_ij + h_kl - h_il - h_kj);
    the 2 x 2 limit is [[p, 1-p], [1-p, p]] with p = sqrt(ad)/(sqrt(ad)+sqrt(bc));
    relabelling streams permutes the result the same way."""
    rng = np.random.default_rng(9)
    h = rng.standard_normal((5, 5))
    H = m.sinkhorn_knopp(h[None])[0]
    for (i, j, k, l) in ((0, 1, 2, 3), (4, 0, 1, 2), (3, 3, 0, 1)):
        if i == k or j == l:
            continue
        lhs = H[i, j] * H[k, l] / (H[i, l] * H[k, j])
        _close(lhs, math.exp(h[i, j] + h[k, l] - h[i, l] - h[k, j]), rtol=1e-12)
    h2 = np.array([[0.3, -1.2], [0.8, 1.1]])
    e = np.exp(h2)
    p = math.sqrt(e[0, 0] * e[1, 1]) / (math.sqrt(e[0, 0] * e[1, 1]) + math.sqrt(e[0, 1] * e[1, 0]))
    _close(m.sinkhorn_knopp(h2[None], 200)[0], [[p, 1 - p], [1 - p, p]], rtol=1e-12)
    perm = np.array([2, 0, 4, 1, 3])
    Hp = m.sinkhorn_knopp(h[perm][:, perm][None])[0]
    _close(Hp, H[perm][:, perm], rtol=1e-12)


def pin_pre_one_hot(m):
    """One-hot H_pre = e_k makes F_pre the k-th stream exactly
    ([mHC-cutile] section 2.5, first step)."""
    rng = np.random.default_rng(13)
    n, C, B = 4, 8, 3
    x = rng.standard_normal((B, n * C))
    for k in range(n):
        hp = np.zeros((B, n))
        hp[:, k] = 1.0
        assert np.array_equal(m.pre_mix(x, hp, n, C), x[:, k * C:(k + 1) * C])


def pin_post_res_structure(m):
    """[mHC-cutile] section 2.5 third step: identity H_res with zero H_post
    returns X; a permutation H_res[i, pi(i)] = 1 moves stream pi(i) to slot i
    (orientation out_i = sum_j H_res[i, j] X_j); with zero H_res the output is
    H_post[i] * F_out; column sums of H_res = 1 conserve the stream sum."""
    rng = np.random.default_rng(17)
    n, C, B = 4, 8, 3
    x = rng.standard_normal((B, n * C))
    f = rng.standard_normal((B, C))
    eye = np.broadcast_to(np.eye(n), (B, n, n))
    assert np.array_equal(m.post_res(x, f, np.zeros((B, n)), eye, n, C), x)
    pi = [2, 0, 3, 1]
    P = np.zeros((B, n, n))
    for i in range(n):
        P[:, i, pi[i]] = 1.0
    out = m.post_res(x, f, np.zeros((B, n)), P, n, C).reshape(B, n, C)
    for i in range(n):
        assert np.array_equal(out[:, i], x[:, pi[i] * C:(pi[i] + 1) * C])
    hp = rng.uniform(0, 2, (B, n))
    out = m.post_res(x, f, hp, np.zeros((B, n, n)), n, C).reshape(B, n, C)
    _close(out, hp[:, :, None] * f[:, None, :], rtol=1e-15)
    hres = m.sinkhorn_knopp(rng.standard_normal((B, n, n)))
    out = m.post_res(x, f, hp, hres, n, C).reshape(B, n, C)
    lhs = out.sum(axis=1)
    rhs = x.reshape(B, n, C).sum(axis=1) + hp.sum(axis=1)[:, None] * f
    _close(lhs, rhs, rtol=1e-12, atol=1e-12)


def pin_bf16_widening(m):
    """bf16 bit patterns widen exactly: fixed values, and agreement with
    torch's own bf16 -> float64 conversion on every finite pattern."""
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049], np.uint16)
    got = m.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 0.0
    assert math.copysign(1.0, got[3]) == -1.0 and got[4] == math.inf
    assert got[5] == 2.0 ** -133 and got[6] == 3.140625
    allb = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).double().numpy()
    w = m.bf16_bits_to_f64(allb)
    fin = np.isfinite(ref)
    assert np.array_equal(w[fin], ref[fin])
    assert np.array_equal(np.isnan(w), np.isnan(ref))


def pin_chunking(m):
    """Row chunking inside forward changes nothing beyond BLAS blocking order
    (rows are independent)."""
    rng = np.random.default_rng(21)
    p = _rand_problem(rng, 4, 8, 7)
    a = _oracle_forward(m, p, chunk=3)
    b = _oracle_forward(m, p, chunk=256)
    for k in a:
        _close(a[k], b[k], rtol=1e-13, atol=1e-14)


def pin_bf16_rounding(m):
    """round_to_bf16 against torch's fp32 -> bf16 conversion (nearest, ties to
    even) on values exact in fp32, where rounding from fp32 or from fp64 must
    agree; hand-made ties and near-ties; idempotence on bf16 values."""
    import torch
    rng = np.random.default_rng(31)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        rng.standard_t(4, 20000)]).astype(np.float32)
    # every tie: the 16 dropped bits exactly 0x8000, both parities of the kept lsb
    ties = ((rng.integers(0, 2**16, 4000, dtype=np.uint32) << 16) | 0x8000).astype(np.uint32)
    ties = ties[((ties >> 23) & 0xFF) - 127 < 60]      # keep exponents in a sane range
    ties = ties[((ties >> 23) & 0xFF) > 60]
    v = np.concatenate([v, ties.view(np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = m.round_to_bf16(v.astype(np.float64))
    assert np.array_equal(got, want)
    # ties by hand: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (lsb of 1 is even)
    assert m.round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    assert m.round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6        # to the even neighbour above
    assert m.round_to_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert m.round_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7  # just past the tie: up
    assert m.round_to_bf16(255.5) == 256.0 and m.round_to_bf16(254.5) == 254.0
    # just below a tie whose even neighbour is above: fp32 would first round it
    # onto the tie, which then goes up (double rounding); straight from fp64 it goes down
    assert m.round_to_bf16(1.0 + 3 * 2.0 ** -8 - 2.0 ** -40) == 1.0 + 2.0 ** -7
    b = m.round_to_bf16(rng.standard_normal(1000))
    assert np.array_equal(m.round_to_bf16(b), b)


PINS = [pin_brute_force, pin_one_hot_phi, pin_rms_closed_forms, pin_lazy_prenorm,
        pin_gates, pin_column_roles, pin_sinkhorn_scaling_form, pin_sinkhorn_column_last,
        pin_sinkhorn_closed_forms, pin_sinkhorn_invariants, pin_pre_one_hot,
        pin_post_res_structure, pin_bf16_widening, pin_chunking, pin_bf16_rounding]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(ORACLE)


# ----------------------------------------------------------------------------
# planted mistakes: every one must trip at least one pin
# ----------------------------------------------------------------------------

def _mut_sinkhorn_cols_first(h_res, iters=20):
    mm = np.exp(np.asarray(h_res, np.float64))
    for _ in range(iters):
        mm = mm / mm.sum(axis=-2, keepdims=True)
        mm = mm / mm.sum(axis=-1, keepdims=True)
    return mm


def _mut_sinkhorn_19(h_res, iters=20):
    return ORACLE_SINKHORN(h_res, 19)


def _mut_post_res_transposed(x, f_out, H_post, H_res, n, C):
    return ORACLE_POST_RES(x, f_out, H_post, np.swapaxes(np.asarray(H_res), -1, -2), n, C)


def _mut_post_res_no_post(x, f_out, H_post, H_res, n, C):
    return ORACLE_POST_RES(x, f_out, np.zeros_like(np.asarray(H_post)), H_res, n, C)


def _mut_gate_post_single(s, r, ap, aq, ar, bp, bq, br, n):
    hp, hq, hr = ORACLE_GATES(s, r, ap, aq, ar, bp, bq, br, n)
    return hp, hq / 2.0, hr


def _mut_gate_swapped(s, r, ap, aq, ar, bp, bq, br, n):
    s = np.asarray(s).copy()
    s[:, 0:n], s[:, n:2 * n] = s[:, n:2 * n].copy(), s[:, 0:n].copy()
    return ORACLE_GATES(s, r, ap, aq, ar, bp, bq, br, n)


def _mut_gate_res_transposed(s, r, ap, aq, ar, bp, bq, br, n):
    hp, hq, hr = ORACLE_GATES(s, r, ap, aq, ar, bp, bq, br, n)
    return hp, hq, np.swapaxes(hr, -1, -2)


def _mut_rms_eps(q, n, C):
    return np.sqrt(np.asarray(q, np.float64) / float(n * C) + 1e-5)


def _mut_rms_per_stream(q, n, C):
    return np.sqrt(np.asarray(q, np.float64) / float(C))


def _mut_scale_mul(s, r, alpha, b):
    s = np.asarray(s, np.float64)
    return float(alpha) * s * np.asarray(r).reshape(-1, 1) + np.asarray(b)


def _mut_no_bias(s, r, alpha, b):
    return ORACLE_SCALE_BIAS(s, r, alpha, np.zeros_like(np.asarray(b, np.float64)))


def _mut_pre_interleaved(x, H_pre, n, C):
    x = np.asarray(x, np.float64).reshape(-1, C, n).transpose(0, 2, 1).reshape(-1, n * C)
    return ORACLE_PRE(x, H_pre, n, C)


def _mut_logits_interleaved(x, phi):
    x = np.asarray(x, np.float64)
    B, K = x.shape
    n = 2 if K % 2 == 0 else 1
    xp = x.reshape(B, K // n, n).transpose(0, 2, 1).reshape(B, K)
    return xp @ np.asarray(phi, np.float64)


def _mut_exp_shift(h_res, iters=20):
    # a plausible "stabilised" variant that forgets to normalise at all
    m = np.exp(np.asarray(h_res, np.float64))
    for _ in range(iters):
        m = m / np.sum(m, axis=-1, keepdims=True)
    return m


ORACLE_SINKHORN = ORACLE.sinkhorn_knopp
ORACLE_POST_RES = ORACLE.post_res
ORACLE_GATES = ORACLE.gate_coefficients
ORACLE_SCALE_BIAS = ORACLE.scale_bias
ORACLE_PRE = ORACLE.pre_mix

def _mut_round_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    mm, e = np.frexp(x)
    return np.ldexp(np.trunc(mm * 256.0) / 256.0, e)


def _mut_round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    mm, e = np.frexp(x)
    return np.ldexp(np.floor(mm * 256.0 + 0.5) / 256.0, e)


def _mut_round_via_fp32(x):
    return ORACLE_ROUND(np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64))


ORACLE_ROUND = ORACLE.round_to_bf16

MUTATIONS = [
    ("round_to_bf16", _mut_round_truncate),
    ("round_to_bf16", _mut_round_half_up),
    ("round_to_bf16", _mut_round_via_fp32),
    ("sinkhorn_knopp", _mut_sinkhorn_cols_first),
    ("sinkhorn_knopp", _mut_sinkhorn_19),
    ("sinkhorn_knopp", _mut_exp_shift),
    ("post_res", _mut_post_res_transposed),
    ("post_res", _mut_post_res_no_post),
    ("gate_coefficients", _mut_gate_post_single),
    ("gate_coefficients", _mut_gate_swapped),
    ("gate_coefficients", _mut_gate_res_transposed),
    ("rms_scale", _mut_rms_eps),
    ("rms_scale", _mut_rms_per_stream),
    ("scale_bias", _mut_scale_mul),
    ("scale_bias", _mut_no_bias),
    ("pre_mix", _mut_pre_interleaved),
    ("coefficient_logits", _mut_logits_interleaved),
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(ORACLE, name, fn)
    failed = []
    for pin in PINS:
        try:
            pin(ORACLE)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake in {name} ({fn.__name__}) tripped no pin"
