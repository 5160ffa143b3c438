"""GPU parity of the FP8 (E4M3) residual-stream variant against the fp64 oracle.

The oracle decodes the same E4M3 bytes exactly (oracle.fp8.e4m3_decode) and
computes in fp64.  Tolerances:
  logits, r, H           as for the bf16 calls (the E4M3 inputs widen exactly):
                         logits row-normwise 2e-3, r relative 2e-3, H absolute 1e-3
  F_pre, X_next (E4M3)   tight: with the GPU's own H fed to the oracle's apply,
                         every code equals the E4M3 rounding (nearest even,
                         saturating) of the exact fp64 value, except where the
                         exact value lies within the fp32 accumulation error of
                         a rounding midpoint -- the kernel takes the decision on
                         its fp32 value (the apply's arithmetic is fp32) -- where
                         either neighbour is accepted (oracle.fp8.e4m3_neighbors_ok
                         with the standard bound (k+1) 2^-24 sum|terms| of a
                         k-term fp32 FMA chain; for X_next at n = 4, whose mix
                         runs on the matrix core with the coefficients carried
                         to 2^-18 relative, 2^-17 sum|terms| more);
                         loose: against the oracle's own coefficients,
                         |decoded - exact| <= 0.07 |exact| + 2^-9 (half a code
                         plus the H tolerance).
Full-size workloads are checked on every row, in chunks of rows (rows are
independent).
"""

import sys

import numpy as np
import pytest
import torch

import manifold_constrained_hyper_amd as mhc
import oracle
import synth
from oracle import fp8 as F8

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    mhc.load()
    yield


# mhc_coeffs_fp8 has three implementations: the one-launch small-B kernel
# (default up to 256 rows), the split-K product with X staged through LDS
# (default above), and the persistent product kernel (MHC_GEMM_ALGO=2).  The
# fused call is the fused kernel by default at n <= 4 (MHC_FUSED_FP8=0 gives
# the apply + product instead, MHC_FUSED_FP8=1 the fused kernel also at n = 8
# with MHC_FUSED_N8), all exercised here; the split-K product runs eight waves
# per workgroup by default and is also run with four waves of one or two
# 16-row blocks (split_w4mb1, split_w4mb2: MHC_GEMM_WAVES=4, MHC_GEMM_MB).
# Every one must meet the bar at every size it supports.
@pytest.fixture(params=["default", "small", "split", "persistent", "split_w4mb1", "split_w4mb2"])
def path(request, tune):
    for k in ("MHC_SMALL_MAX_B", "MHC_GEMM_ALGO", "MHC_FUSED_N8"):
        tune.delenv(k, raising=False)
    if request.param == "small":
        tune.setenv("MHC_SMALL_MAX_B", str(1 << 30))
    elif request.param.startswith("split"):
        tune.setenv("MHC_SMALL_MAX_B", "0")
        if request.param.startswith("split_w4mb"):
            tune.setenv("MHC_GEMM_WAVES", 4)
            tune.setenv("MHC_GEMM_MB", int(request.param[-1]))
    elif request.param == "persistent":
        tune.setenv("MHC_SMALL_MAX_B", "0")
        tune.setenv("MHC_GEMM_ALGO", "2")
        tune.setenv("MHC_FUSED_N8", "1")
        tune.setenv("MHC_FUSED_FP8", "1")
    return request.param


def _alloc(B, n, C):
    N = n * n + 2 * n
    ws = max(mhc.mhc_coeffs_fp8_workspace_size(B, n, C),
             mhc.mhc_post_res_coeffs_fp8_workspace_size(B, n, C), 16)
    return {"logits": torch.empty(B, N, device="cuda"), "r": torch.empty(B, device="cuda"),
            "H": torch.empty(B, N, device="cuda"),
            "F_pre": torch.empty(B, C, dtype=torch.uint8, device="cuda"),
            "X_next": torch.empty(B, n * C, dtype=torch.uint8, device="cuda"),
            "workspace": torch.empty(ws, dtype=torch.uint8, device="cuda")}


def run_three_calls(inp):
    B, n, C = inp["B"], inp["n"], inp["C"]
    o = _alloc(B, n, C)
    mhc.mhc_coeffs_fp8(B, n, C, inp["X"], inp["phi"], inp["alpha_pre"], inp["alpha_post"],
                       inp["alpha_res"], inp["b_pre"], inp["b_post"], inp["b_res"],
                       o["logits"], o["r"], o["H"], o["workspace"])
    mhc.mhc_pre_fp8(B, n, C, inp["X"], o["H"], o["F_pre"])
    mhc.mhc_post_res_fp8(B, n, C, inp["X"], inp["F_out"], o["H"], o["X_next"])
    torch.cuda.synchronize()
    return o


def fp32_slack_pre(x, h_pre, n, C):
    """Bound on the fp32 error of the pre-mix FMA chain (n terms): (n+1) 2^-24
    times the sum of the terms' magnitudes."""
    return (n + 1) * 2.0 ** -24 * oracle.pre_mix(np.abs(x), np.abs(h_pre), n, C) + 1e-30


def fp32_slack_post(x, f, h_post, h_res, n, C):
    """Bound on the error of the post/res mix (n+1 terms) before its rounding
    to E4M3: (n+2) 2^-24 times the sum of the terms' magnitudes for the fp32
    FMA chain; at n = 4 the mix runs on the matrix core with each coefficient
    carried as two bf16 parts (off by at most 2^-18 relative) and about 16
    fp32 roundings over the three MFMAs, so 2^-17 of that sum is added."""
    extra = 2.0 ** -17 if n == 4 else 0.0
    return ((n + 2) * 2.0 ** -24 + extra) * oracle.post_res(np.abs(x), np.abs(f), np.abs(h_post),
                                                            np.abs(h_res), n, C) + 1e-30


def _rows_f64(t, rows):
    idx = torch.as_tensor(rows, device=t.device, dtype=torch.long)
    return F8.e4m3_decode(synth.e4m3_codes(t.index_select(0, idx)))


def check(inp, o, rows, label):
    n, C = inp["n"], inp["C"]
    x = _rows_f64(inp["X"], rows)
    f = _rows_f64(inp["F_out"], rows)
    phi = oracle.bf16_bits_to_f64(synth.bf16_bits(inp["phi"]))
    bp, bq, br = (inp[k].double().cpu().numpy() for k in ("b_pre", "b_post", "b_res"))
    co = oracle.coefficients(x, phi, inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
                             bp, bq, br, n, C)
    idx = torch.as_tensor(rows, device="cuda", dtype=torch.long)
    g = {k: o[k].index_select(0, idx).double().cpu().numpy() for k in ("logits", "r", "H")}
    row_err = np.abs(g["logits"] - co["logits"]).max(1)
    assert np.all(row_err <= 2e-3 * np.abs(co["logits"]).max(1)), f"{label}: logits"
    assert np.all(np.abs(g["r"] - co["r"]) <= 2e-3 * co["r"]), f"{label}: r"
    assert np.abs(g["H"] - co["H"]).max() <= 1e-3, f"{label}: H"
    # apply steps with the GPU's own coefficients: exact E4M3 rounding rule
    pre_g, post_g, res_g = oracle.split_h(g["H"], n)
    fpre_exact = oracle.pre_mix(x, pre_g, n, C)
    xnext_exact = oracle.post_res(x, f, post_g, res_g, n, C)
    fpre_codes = synth.e4m3_codes(o["F_pre"].index_select(0, idx))
    xnext_codes = synth.e4m3_codes(o["X_next"].index_select(0, idx))
    bad = ~F8.e4m3_neighbors_ok(fpre_codes, fpre_exact, absolute=fp32_slack_pre(x, pre_g, n, C))
    assert not bad.any(), f"{label}: F_pre codes off at {np.argwhere(bad)[:5].tolist()}"
    bad = ~F8.e4m3_neighbors_ok(xnext_codes, xnext_exact, absolute=fp32_slack_post(x, f, post_g, res_g, n, C))
    assert not bad.any(), f"{label}: X_next codes off at {np.argwhere(bad)[:5].tolist()}"
    # against the oracle's own coefficients
    pre_o, post_o, res_o = oracle.split_h(co["H"], n)
    for name, codes, exact in (("F_pre", fpre_codes, oracle.pre_mix(x, pre_o, n, C)),
                               ("X_next", xnext_codes, oracle.post_res(x, f, post_o, res_o, n, C))):
        err = np.abs(F8.e4m3_decode(codes) - exact)
        assert np.all(err <= 0.07 * np.abs(exact) + 2.0 ** -9), f"{label}: {name} vs oracle"


def _sample(B):
    if B <= 64:
        return list(range(B))
    return sorted(set([0, 1, B // 2, B - 1] + np.random.default_rng(B).choice(B, 40, replace=False).tolist()))


def _chunks(B, size=1024):
    """Every row, in chunks (rows are independent; chunks bound host memory)."""
    return [list(range(lo, min(B, lo + size))) for lo in range(0, B, size)]


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large", "wide"])
def test_fp8_named(name):
    _say(f"fp8 three calls {name}")
    inp = synth.make_config_fp8(name, device="cuda")
    o = run_three_calls(inp)
    for rows in _chunks(inp["B"]):
        check(inp, o, rows, f"{name} rows {rows[0]}..{rows[-1]}")


FP8_RAGGED = [(77, 4, 272), (1, 4, 16), (130, 8, 96), (33, 1, 48), (65, 2, 2064), (300, 4, 1040),
              (3, 8, 16), (257, 4, 528)]


@pytest.mark.parametrize("B,n,C", FP8_RAGGED, ids=[f"B{b}n{n}C{c}" for b, n, c in FP8_RAGGED])
def test_fp8_ragged(B, n, C, path):
    _say(f"fp8 ragged B={B} n={n} C={C} path={path}")
    inp = synth.make_inputs_fp8(n, C, B, "student_t4" if B % 2 else "normal", seed=B * 17 + C,
                                device="cuda")
    o = run_three_calls(inp)
    check(inp, o, list(range(B)), f"B{B}n{n}C{C}")


def test_fp8_saturates():
    """Outputs past the E4M3 range saturate to +-448 (the variant's reading)."""
    _say("fp8 saturation")
    B, n, C = 32, 4, 64
    inp = synth.make_inputs_fp8(n, C, B, "normal", seed=9, device="cuda")
    big = synth.to_e4m3(torch.full((B, n * C), 400.0, device="cuda"))
    fbig = synth.to_e4m3(torch.full((B, C), 448.0, device="cuda"))
    N = n * n + 2 * n
    H = torch.zeros(B, N, device="cuda")
    H[:, n:2 * n] = 2.0                                          # H_post = 2
    H[:, 2 * n:] = torch.eye(n, device="cuda").reshape(-1)      # H_res = I
    H[:, :n] = 1.0                                               # H_pre = 1: F_pre = n * 400
    o = _alloc(B, n, C)
    mhc.mhc_post_res_fp8(B, n, C, big, fbig, H, o["X_next"])     # 400 + 2 * 448 = 1296 -> 448
    mhc.mhc_pre_fp8(B, n, C, big, H, o["F_pre"])
    torch.cuda.synchronize()
    assert (synth.e4m3_codes(o["X_next"]) == 0x7E).all()
    assert (synth.e4m3_codes(o["F_pre"]) == 0x7E).all()
    neg = synth.to_e4m3(torch.full((B, n * C), -400.0, device="cuda"))
    mhc.mhc_post_res_fp8(B, n, C, neg, synth.to_e4m3(-torch.full((B, C), 448.0, device="cuda")), H,
                         o["X_next"])
    torch.cuda.synchronize()
    assert (synth.e4m3_codes(o["X_next"]) == 0xFE).all()


# ----------------------------------------------------------------------------
# fused: mhc_post_res_coeffs_fp8
# ----------------------------------------------------------------------------

def _fused(inp, nxt):
    B, n, C = inp["B"], inp["n"], inp["C"]
    o = run_three_calls(inp)
    ref = _alloc(B, n, C)
    mhc.mhc_coeffs_fp8(B, n, C, o["X_next"], nxt["phi"], nxt["alpha_pre"], nxt["alpha_post"],
                       nxt["alpha_res"], nxt["b_pre"], nxt["b_post"], nxt["b_res"],
                       ref["logits"], ref["r"], ref["H"], ref["workspace"])
    f = _alloc(B, n, C)
    mhc.mhc_post_res_coeffs_fp8(B, n, C, inp["X"], inp["F_out"], o["H"], f["X_next"], nxt["phi"],
                                nxt["alpha_pre"], nxt["alpha_post"], nxt["alpha_res"],
                                nxt["b_pre"], nxt["b_post"], nxt["b_res"], f["logits"], f["r"],
                                f["H"], f["workspace"])
    torch.cuda.synchronize()
    return o, ref, f


def _check_fused(inp, nxt, o, ref, f, rows, label):
    n, C = inp["n"], inp["C"]
    assert torch.equal(f["X_next"], o["X_next"]), f"{label}: fused X_next differs from mhc_post_res_fp8"
    xn = _rows_f64(f["X_next"], rows)
    co = oracle.coefficients(xn, oracle.bf16_bits_to_f64(synth.bf16_bits(nxt["phi"])),
                             nxt["alpha_pre"], nxt["alpha_post"], nxt["alpha_res"],
                             nxt["b_pre"].double().cpu().numpy(), nxt["b_post"].double().cpu().numpy(),
                             nxt["b_res"].double().cpu().numpy(), n, C)
    idx = torch.as_tensor(rows, device="cuda", dtype=torch.long)
    g = {k: f[k].index_select(0, idx).double().cpu().numpy() for k in ("logits", "r", "H")}
    row_err = np.abs(g["logits"] - co["logits"]).max(1)
    assert np.all(row_err <= 2e-3 * np.abs(co["logits"]).max(1)), f"{label}: logits"
    assert np.all(np.abs(g["r"] - co["r"]) <= 2e-3 * co["r"]), f"{label}: r"
    assert np.abs(g["H"] - co["H"]).max() <= 1e-3, f"{label}: H"
    rel = ((f["logits"] - ref["logits"]).abs().max() / ref["logits"].abs().max()).item()
    assert rel < 1e-4, f"{label}: logits vs mhc_coeffs_fp8 {rel}"
    assert (f["H"] - ref["H"]).abs().max().item() < 1e-4, f"{label}: H vs mhc_coeffs_fp8"


def _layers(n, C, B, dist, seed):
    cur = synth.make_inputs_fp8(n, C, B, dist, seed=seed, device="cuda")
    nxt = synth.make_inputs(n, C, 1, "normal", seed=seed + 7919, device="cuda")
    return cur, nxt


@pytest.mark.parametrize("kernel", ["default", "fused", "twopass", "fused_spu"])
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large", "wide"])
def test_fp8_fused_named(name, kernel, tune):
    if kernel in ("fused", "fused_spu"):
        tune.setenv("MHC_FUSED_FP8", "1")
        tune.setenv("MHC_FUSED_N8", "1")
        if kernel == "fused_spu":
            if synth.CONFIGS[name]["n"] == 8:
                pytest.skip("n = 8 always runs this layout (kernel 'fused')")
            tune.setenv("MHC_FUSED_FIXED", "0")
    elif kernel == "twopass":
        tune.setenv("MHC_FUSED_FP8", "0")
    _say(f"fp8 fused {name} kernel={kernel}")
    cfg = synth.CONFIGS[name]
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    o, ref, f = _fused(cur, nxt)
    # every row on the default route; sampled rows on the others
    chunks = _chunks(cfg["B"]) if kernel == "default" else [_sample(cfg["B"])]
    for rows in chunks:
        _check_fused(cur, nxt, o, ref, f, rows, f"{name} rows {rows[0]}..{rows[-1]}")


FP8_FUSED_RAGGED = [(77, 4, 544), (1, 4, 32), (130, 8, 96), (33, 1, 64), (300, 4, 1536),
                    (17, 8, 32), (65, 2, 2080)]


@pytest.mark.parametrize("B,n,C", FP8_FUSED_RAGGED, ids=[f"B{b}n{n}C{c}" for b, n, c in FP8_FUSED_RAGGED])
def test_fp8_fused_ragged(B, n, C, path):
    _say(f"fp8 fused ragged B={B} n={n} C={C} path={path}")
    cur, nxt = _layers(n, C, B, "student_t4" if B % 2 else "normal", B * 29 + C)
    o, ref, f = _fused(cur, nxt)
    _check_fused(cur, nxt, o, ref, f, list(range(B)), f"B{B}n{n}C{C}")


@pytest.mark.parametrize("kernel", ["default", "fused", "twopass"])
def test_fp8_fused_deterministic(kernel, tune):
    if kernel == "fused":
        tune.setenv("MHC_FUSED_FP8", "1")
    elif kernel == "twopass":
        tune.setenv("MHC_FUSED_FP8", "0")
    _say(f"fp8 fused determinism kernel={kernel}")
    cfg = synth.CONFIGS["prefill"]
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    _, _, a = _fused(cur, nxt)
    _, _, b = _fused(cur, nxt)
    for k in ("X_next", "logits", "r", "H"):
        assert torch.equal(a[k].view(torch.int8), b[k].view(torch.int8)), k


def test_fp8_nan_codes():
    """NaN inputs (E4M3 codes 0x7F and 0xFF) give a NaN code (S.1111.111:
    0x7F, the oracle's, or 0xFF -- OCP E4M3 has the two and the pages fix no
    sign for a NaN) in every output they reach and nowhere else (the plain
    saturating clamp would turn them into -448), in the stand-alone apply and
    pre-mix; every other code is the oracle's."""
    _say("fp8 NaN codes")
    B, n, C = 64, 4, 256
    N = n * n + 2 * n
    inp = synth.make_inputs_fp8(n, C, B, "normal", seed=21, device="cuda")
    X, F = inp["X"].clone(), inp["F_out"].clone()
    X[3, 5] = 0x7F
    X[10, C + 17] = 0xFF
    X[20, 3 * C + 100] = 0x7F
    F[30, 7] = 0xFF
    g = torch.Generator(device="cpu").manual_seed(5)
    H = torch.rand(B, N, generator=g).to("cuda")
    H[:, n:2 * n] *= 2.0
    o = _alloc(B, n, C)
    mhc.mhc_post_res_fp8(B, n, C, X, F, H, o["X_next"])
    mhc.mhc_pre_fp8(B, n, C, X, H, o["F_pre"])
    torch.cuda.synchronize()
    x = F8.e4m3_decode(synth.e4m3_codes(X))
    f = F8.e4m3_decode(synth.e4m3_codes(F))
    pre, post, res = oracle.split_h(H.double().cpu().numpy(), n)
    want_x = F8.e4m3_encode(oracle.post_res(x, f, post, res, n, C))
    want_f = F8.e4m3_encode(oracle.pre_mix(x, pre, n, C))
    got_x, got_f = synth.e4m3_codes(o["X_next"]), synth.e4m3_codes(o["F_pre"])
    assert (want_x == 0x7F).sum() == 4 * 4 and (want_f == 0x7F).sum() == 3
    nan_x, nan_f = want_x == 0x7F, want_f == 0x7F
    is_nan = lambda c: (c & 0x7F) == 0x7F  # noqa: E731
    assert is_nan(got_x[nan_x]).all() and not is_nan(got_x[~nan_x]).any()
    assert is_nan(got_f[nan_f]).all() and not is_nan(got_f[~nan_f]).any()
    _say(f"NaN codes produced: {sorted(set(got_x[nan_x].tolist()) | set(got_f[nan_f].tolist()))}")
    exact_x = oracle.post_res(x, f, post, res, n, C)
    exact_f = oracle.pre_mix(x, pre, n, C)
    sx = fp32_slack_post(np.nan_to_num(x), np.nan_to_num(f), post, res, n, C)
    sf = fp32_slack_pre(np.nan_to_num(x), pre, n, C)
    assert F8.e4m3_neighbors_ok(got_x[~nan_x], exact_x[~nan_x], absolute=sx[~nan_x]).all()
    assert F8.e4m3_neighbors_ok(got_f[~nan_f], exact_f[~nan_f], absolute=sf[~nan_f]).all()
