"""GPU parity of mhc_post_res_coeffs_pre_fp8: the one-pass layer call on the
E4M3 residual stream (a layer's post/res apply, then the next layer's
coefficients and pre-mix).

Checks, for every shape:
  X_next      bitwise what mhc_post_res_fp8 writes;
  F_pre_next  bitwise what mhc_pre_fp8(X_next, H_next) writes with the call's
              own H_next, no NaN code (a wait that gave up), and every code
              one of the two E4M3 neighbours of the exact fp64 mix with
              those coefficients (the rounding rule), and within the E4M3
              tolerance of the mix with the oracle's coefficients;
  logits, r, H_next against the fp64 oracle on the call's X_next (decoded
              exactly), on every row of the small shapes and on sampled rows
              of the full-size workloads, and against mhc_coeffs_fp8 on
              X_next up to fp32 summation order.
The next layer has its own phi and biases (a second seeded draw).

Routes: "default" (one pass above 256 rows for n <= 4 and at most sixteen
512-channel steps per row; the two calls otherwise), "onepass" (small-B
limit 0, so the one-pass kernel also runs the small shapes it can take) and
"twocalls" (MHC_FUSED_FP8=0: mhc_post_res_coeffs_fp8 as apply + product,
then mhc_pre_fp8).
"""

import sys

import numpy as np
import pytest
import torch

import manifold_constrained_hyper_amd as mhc
import oracle
from oracle import fp8 as F8
import synth

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


@pytest.fixture(params=["default", "onepass", "twocalls"])
def route(request, tune):
    for k in ("MHC_FUSED_PRE", "MHC_SMALL_MAX_B", "MHC_FUSED_FP8", "MHC_FUSED_FIXED"):
        tune.delenv(k, raising=False)
    if request.param == "onepass":
        tune.setenv("MHC_SMALL_MAX_B", "0")
    elif request.param == "twocalls":
        tune.setenv("MHC_FUSED_FP8", "0")
    return request.param


def _layers(n, C, B, x_dist, seed):
    cur = synth.make_inputs_fp8(n, C, B, x_dist, seed=seed, device="cuda")
    nxt = synth.make_inputs(n, C, 1, "normal", seed=seed + 7919, device="cuda")  # phi, biases of layer t+1
    return cur, nxt


def _ws(nbytes):
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")


def _coeffs(inp, X, o):
    B, n, C = X.shape[0], inp["n"], inp["C"]
    N = n * n + 2 * n
    for k, shape in (("logits", (B, N)), ("r", (B,)), ("H", (B, N))):
        o.setdefault(k, torch.empty(shape, device="cuda"))
    mhc.mhc_coeffs_fp8(B, n, C, X, inp["phi"], inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
                       inp["b_pre"], inp["b_post"], inp["b_res"], o["logits"], o["r"], o["H"],
                       _ws(mhc.mhc_coeffs_fp8_workspace_size(B, n, C)))


def _call(cur, nxt, H, ws=None, fill=None):
    """mhc_post_res_coeffs_pre_fp8 on (cur, H) with layer t+1 = nxt; fresh outputs."""
    B, n, C = cur["B"], cur["n"], cur["C"]
    N = n * n + 2 * n
    if ws is None:
        ws = _ws(mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(B, n, C))
    if fill is not None:
        fill(ws)
    f = {"X_next": torch.empty_like(cur["X"]), "logits": torch.empty(B, N, device="cuda"),
         "r": torch.empty(B, device="cuda"), "H": torch.empty(B, N, device="cuda"),
         "F_pre": torch.empty(B, C, dtype=torch.uint8, device="cuda")}
    mhc.mhc_post_res_coeffs_pre_fp8(B, n, C, cur["X"], cur["F_out"], H, f["X_next"], nxt["phi"],
                                    nxt["alpha_pre"], nxt["alpha_post"], nxt["alpha_res"],
                                    nxt["b_pre"], nxt["b_post"], nxt["b_res"], f["logits"], f["r"],
                                    f["H"], f["F_pre"], ws)
    torch.cuda.synchronize()
    return f


def _run(cur, nxt, fill=None):
    B, n, C = cur["B"], cur["n"], cur["C"]
    o = {}
    _coeffs(cur, cur["X"], o)
    o["X_next"] = torch.empty_like(cur["X"])
    mhc.mhc_post_res_fp8(B, n, C, cur["X"], cur["F_out"], o["H"], o["X_next"])
    f = _call(cur, nxt, o["H"], fill=fill)
    ref = {}
    _coeffs(nxt | {"n": n, "C": C}, f["X_next"], ref)     # mhc_coeffs_fp8 on the call's X_next
    pre_own = torch.empty_like(f["F_pre"])
    mhc.mhc_pre_fp8(B, n, C, f["X_next"], f["H"], pre_own)
    torch.cuda.synchronize()
    return o, ref, f, pre_own


def _decode_rows(t, idx):
    return F8.e4m3_decode(synth.e4m3_codes(t.index_select(0, idx)))


def _check(cur, nxt, o, ref, f, pre_own, rows, label):
    n, C = cur["n"], cur["C"]
    assert torch.equal(f["X_next"], o["X_next"]), f"{label}: X_next differs from mhc_post_res_fp8"
    codes = f["F_pre"]
    assert not ((codes & 0x7F) == 0x7F).any(), f"{label}: NaN code in F_pre (a wait gave up?)"
    assert torch.equal(codes, pre_own), f"{label}: F_pre differs from mhc_pre_fp8(X_next, H_next)"
    idx = torch.as_tensor(rows, device="cuda", dtype=torch.long)
    xn = _decode_rows(f["X_next"], idx)
    co = oracle.coefficients(xn, oracle.bf16_bits_to_f64(synth.bf16_bits(nxt["phi"])),
                             nxt["alpha_pre"], nxt["alpha_post"], nxt["alpha_res"],
                             nxt["b_pre"].double().cpu().numpy(), nxt["b_post"].double().cpu().numpy(),
                             nxt["b_res"].double().cpu().numpy(), n, C)
    g = {k: f[k].index_select(0, idx).double().cpu().numpy() for k in ("logits", "r", "H")}
    row_err = np.abs(g["logits"] - co["logits"]).max(1)
    assert np.all(row_err <= 2e-3 * np.abs(co["logits"]).max(1)), f"{label}: logits"
    assert np.all(np.abs(g["r"] - co["r"]) <= 2e-3 * co["r"]), f"{label}: r"
    assert np.abs(g["H"] - co["H"]).max() <= 1e-3, f"{label}: H"
    # with the call's own H_pre: each code is a neighbour of the exact mix
    fcodes = synth.e4m3_codes(codes.index_select(0, idx))
    slack = (n + 1) * 2.0 ** -24 * oracle.pre_mix(np.abs(xn), np.abs(g["H"][:, :n]), n, C) + 1e-30
    bad = ~F8.e4m3_neighbors_ok(fcodes, oracle.pre_mix(xn, g["H"][:, :n], n, C), absolute=slack)
    assert not bad.any(), f"{label}: F_pre codes off at {np.argwhere(bad)[:5].tolist()}"
    # with the oracle's coefficients: E4M3 tolerance
    exact = oracle.pre_mix(xn, co["H"][:, :n], n, C)
    err = np.abs(F8.e4m3_decode(fcodes) - exact)
    assert np.all(err <= 0.07 * np.abs(exact) + 2.0 ** -9), f"{label}: F_pre vs oracle"
    # against mhc_coeffs_fp8 on the same X_next: only summation order differs
    rel = ((f["logits"] - ref["logits"]).abs().max() / ref["logits"].abs().max()).item()
    assert rel < 1e-4, f"{label}: logits vs mhc_coeffs_fp8 {rel}"
    assert (f["H"] - ref["H"]).abs().max().item() < 1e-4, f"{label}: H vs mhc_coeffs_fp8"
    assert ((f["r"] - ref["r"]).abs() / ref["r"]).max().item() < 1e-5, f"{label}: r vs mhc_coeffs_fp8"


def _rows(B):
    if B <= 256:
        return list(range(B))
    rng = np.random.default_rng(B)
    return sorted(set([0, 1, 15, 16, B // 2, B - 17, B - 1] + rng.choice(B, 40, replace=False).tolist()))


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large", "wide"])
def test_named(name, route):
    cfg = synth.CONFIGS[name]
    one = mhc.mhc_post_res_coeffs_pre_fp8_one_pass(cfg["B"], cfg["n"], cfg["C"])
    _say(f"post_res_coeffs_pre_fp8 {name} route={route} one_pass={one}")
    if route == "onepass" and cfg["B"] > 256:
        pytest.skip("above 256 rows the default route already takes the one-pass kernel where it fits")
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    o, ref, f, pre_own = _run(cur, nxt)
    # every row on the default route, in chunks (rows are independent);
    # sampled rows on the others
    chunks = ([list(range(lo, min(cfg["B"], lo + 1024))) for lo in range(0, cfg["B"], 1024)]
              if route == "default" else [_rows(cfg["B"])])
    for rows in chunks:
        _check(cur, nxt, o, ref, f, pre_own, rows, f"{name} rows {rows[0]}..{rows[-1]}")


def test_route_query(tune):
    for k in ("MHC_SMALL_MAX_B", "MHC_FUSED_PRE", "MHC_FUSED_FP8", "MHC_FUSED_FIXED"):
        tune.delenv(k, raising=False)
    q = mhc.mhc_post_res_coeffs_pre_fp8_one_pass
    assert q(16384, 4, 7168)
    assert q(4096, 4, 4096)
    assert not q(64, 4, 7168)       # small B
    assert not q(8192, 8, 4096)     # n = 8
    assert not q(4096, 4, 8704)     # 17 steps per row
    assert not q(4096, 4, 7160)     # C % 32 != 0
    tune.setenv("MHC_FUSED_FP8", "0")
    assert not q(16384, 4, 7168)
    tune.setenv("MHC_FUSED_FP8", "1")
    tune.setenv("MHC_FUSED_PRE", "0")
    assert not q(16384, 4, 7168)


# (B, n, C): ragged row tiles, a ragged last 512-channel step, one to sixteen
# steps per row, n = 1, 2, 4; n = 8 and 17 steps take the two-call route.
RAGGED = [(77, 4, 544), (1, 4, 32), (33, 1, 64), (65, 2, 2080), (300, 4, 1536), (16, 2, 512),
          (257, 4, 8192), (19, 4, 3104), (130, 8, 96), (21, 4, 8704), (513, 2, 4096)]


@pytest.mark.parametrize("B,n,C", RAGGED, ids=[f"B{b}n{n}C{c}" for b, n, c in RAGGED])
def test_ragged(B, n, C, route):
    _say(f"post_res_coeffs_pre_fp8 ragged B={B} n={n} C={C} route={route} "
         f"one_pass={mhc.mhc_post_res_coeffs_pre_fp8_one_pass(B, n, C)}")
    cur, nxt = _layers(n, C, B, "student_t4" if B % 2 else "normal", B * 37 + C)
    o, ref, f, pre_own = _run(cur, nxt)
    _check(cur, nxt, o, ref, f, pre_own, list(range(B)), f"B{B}n{n}C{C}")


def _rand_fill(ws):
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device="cuda", dtype=torch.uint8))


@pytest.mark.parametrize("B,n,C", [(300, 4, 1536), (600, 4, 7168)])
def test_workspace_contents(B, n, C):
    _say(f"post_res_coeffs_pre_fp8 random workspace B={B} n={n} C={C}")
    cur, nxt = _layers(n, C, B, "normal", B + n + C)
    o, ref, f, pre_own = _run(cur, nxt, fill=_rand_fill)
    _check(cur, nxt, o, ref, f, pre_own, _rows(B), f"B{B}n{n}C{C}/random")


@pytest.mark.parametrize("B", [16384, 65536], ids=["large", "B65536"])
def test_two_routes_agree(tune, B):
    """The one-pass kernel and the two calls it replaces at n=4, C=7168 (the
    large workload, and B = 65536 for a long run of the record hand-off):
    X_next bitwise, coefficients up to summation order, F_pre codes at most
    one E4M3 step apart (H_pre may differ in its last bits)."""
    _say(f"post_res_coeffs_pre_fp8 one pass vs two calls (n=4 C=7168 B={B})")
    cfg = dict(synth.CONFIGS["large"], B=B)
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    o = {}
    _coeffs(cur, cur["X"], o)
    for k in ("MHC_FUSED_PRE", "MHC_FUSED_FP8"):
        tune.delenv(k, raising=False)
    a = _call(cur, nxt, o["H"])
    tune.setenv("MHC_FUSED_PRE", "0")
    b = _call(cur, nxt, o["H"])
    assert torch.equal(a["X_next"], b["X_next"])
    assert (a["H"] - b["H"]).abs().max().item() < 1e-4
    va = F8.e4m3_decode(synth.e4m3_codes(a["F_pre"]))
    vb = F8.e4m3_decode(synth.e4m3_codes(b["F_pre"]))
    assert np.all(np.abs(va - vb) <= 2.0 ** -3 * np.abs(vb) + 2.0 ** -9)


def test_deterministic():
    _say("post_res_coeffs_pre_fp8 determinism (prefill)")
    cfg = synth.CONFIGS["prefill"]
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    o = {}
    _coeffs(cur, cur["X"], o)
    a = _call(cur, nxt, o["H"])
    b = _call(cur, nxt, o["H"])
    for k in ("X_next", "logits", "r", "H", "F_pre"):
        assert torch.equal(a[k].view(torch.int8), b[k].view(torch.int8)), k


def test_guard_bands(route):
    _say(f"post_res_coeffs_pre_fp8 guard bands route={route}")
    B, n, C = 77, 4, 544
    N = n * n + 2 * n
    cur, nxt = _layers(n, C, B, "normal", 13)
    o = {}
    _coeffs(cur, cur["X"], o)
    G = 4096
    ws_bytes = mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(B, n, C)

    def guarded(nbytes):
        buf = torch.full((nbytes + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
        return buf, buf[G:G + nbytes]

    bufs = {k: guarded(sz) for k, sz in (("X_next", B * n * C), ("logits", B * N * 4), ("r", B * 4),
                                          ("H", B * N * 4), ("F_pre", B * C), ("ws", ws_bytes))}
    mhc.mhc_post_res_coeffs_pre_fp8(B, n, C, cur["X"], cur["F_out"], o["H"], bufs["X_next"][1],
                                    nxt["phi"], 0.01, 0.01, 0.01, nxt["b_pre"], nxt["b_post"],
                                    nxt["b_res"], bufs["logits"][1], bufs["r"][1], bufs["H"][1],
                                    bufs["F_pre"][1], bufs["ws"][1], ws_bytes)
    torch.cuda.synchronize()
    for k, (buf, _) in bufs.items():
        assert (buf[:G] == 0x5A).all() and (buf[-G:] == 0x5A).all(), f"write outside {k}"
