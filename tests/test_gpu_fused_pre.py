"""GPU parity of mhc_post_res_coeffs_pre: a layer's post/res apply, then the
next layer's coefficients and pre-mix, in one pass where the shape allows.

Checks, for every shape:
  X_next      bitwise what mhc_post_res writes;
  F_pre_next  bitwise what mhc_pre(X_next, H_next) writes with the call's own
              H_next (the one-pass kernel forms H_pre from the same sums, in
              the same order, with the same gate);
  logits, r, H_next and F_pre_next against the fp64 oracle on the call's
              X_next (tolerances of test_gpu_parity.py), on every row;
  at the large workload also an oracle-only chain: the oracle's X_next from
              X_t and H, rounded to bf16 as the next layer's input, then the
              oracle's coefficients and F_pre from that X_next;
  the coefficients against mhc_coeffs on X_next up to fp32 summation order.
The next layer has its own phi and biases (a second seeded draw).

Routes: "default" (up to 256 rows at n <= 4 with n*C <= 1024 the
single-slice kernel of mhc_layer_small.hip; one pass above 256 rows for
n <= 4 and at most sixteen 512-channel steps per row, and at n = 8 for at
most thirty-two 128-channel slices per row (mhc_onepass8.hip); the two calls
otherwise) and "onepass", which lowers the small-B limit to 0 so that the
one-pass kernels also run every small shape they can take.
"""

import sys

import numpy as np
import pytest
import torch

import manifold_constrained_hyper_amd as mhc
import oracle
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


# "pass8pre": the n = 8 pass in one pass (MHC_PASS8_PRE=1; n = 8 shapes only,
# which by default run as the two calls).
@pytest.fixture(params=["default", "onepass", "pass8pre"])
def route(request, tune):
    tune.delenv("MHC_FUSED_PRE", raising=False)
    tune.delenv("MHC_PASS8_PRE", raising=False)
    if request.param == "onepass":
        tune.setenv("MHC_SMALL_MAX_B", "0")
    else:
        tune.delenv("MHC_SMALL_MAX_B", raising=False)
    if request.param == "pass8pre":
        tune.setenv("MHC_PASS8_PRE", "1")
    return request.param


def _only_pass8(route, n):
    if route == "pass8pre" and n != 8:
        pytest.skip("MHC_PASS8_PRE changes n = 8 only")


def _f64(t):
    return oracle.bf16_bits_to_f64(synth.bf16_bits(t))


def _layers(n, C, B, x_dist, seed):
    cur = synth.make_inputs(n, C, B, x_dist, seed=seed, device="cuda")
    nxt = synth.make_inputs(n, C, 1, "normal", seed=seed + 7919, device="cuda")  # phi, biases of layer t+1
    return cur, nxt


def _coeffs(inp, X, o):
    B, n, C = X.shape[0], inp["n"], inp["C"]
    mhc.mhc_coeffs(B, n, C, X, inp["phi"], inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
                   inp["b_pre"], inp["b_post"], inp["b_res"], o["logits"], o["r"], o["H"],
                   o["workspace"])


def _call(cur, nxt, H, ws=None, fill=None):
    """mhc_post_res_coeffs_pre on (cur, H) with layer t+1 = nxt; fresh outputs."""
    B, n, C = cur["B"], cur["n"], cur["C"]
    N = n * n + 2 * n
    if ws is None:
        ws = torch.empty(max(mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C), 16),
                         dtype=torch.uint8, device="cuda")
    if fill is not None:
        fill(ws)
    f = {"X_next": torch.empty_like(cur["X"]), "logits": torch.empty(B, N, device="cuda"),
         "r": torch.empty(B, device="cuda"), "H": torch.empty(B, N, device="cuda"),
         "F_pre": torch.empty(B, C, dtype=torch.bfloat16, device="cuda")}
    mhc.mhc_post_res_coeffs_pre(B, n, C, cur["X"], cur["F_out"], H, f["X_next"], nxt["phi"],
                                nxt["alpha_pre"], nxt["alpha_post"], nxt["alpha_res"], nxt["b_pre"],
                                nxt["b_post"], nxt["b_res"], f["logits"], f["r"], f["H"], f["F_pre"], ws)
    torch.cuda.synchronize()
    return f


def _run(cur, nxt, fill=None):
    B, n, C = cur["B"], cur["n"], cur["C"]
    o = mhc.alloc_outputs(B, n, C)
    _coeffs(cur, cur["X"], o)
    mhc.mhc_post_res(B, n, C, cur["X"], cur["F_out"], o["H"], o["X_next"])
    f = _call(cur, nxt, o["H"], fill=fill)
    ref = mhc.alloc_outputs(B, n, C)   # mhc_coeffs and mhc_pre on the call's X_next
    _coeffs(nxt, f["X_next"], ref)
    pre_own = torch.empty_like(f["F_pre"])
    mhc.mhc_pre(B, n, C, f["X_next"], f["H"], pre_own)
    torch.cuda.synchronize()
    return o, ref, f, pre_own


def _check(cur, nxt, o, ref, f, pre_own, rows, label):
    n, C = cur["n"], cur["C"]
    bits = lambda t: t.view(torch.int16)  # noqa: E731
    assert torch.equal(bits(f["X_next"]), bits(o["X_next"])), f"{label}: X_next differs from mhc_post_res"
    assert torch.isfinite(f["F_pre"].float()).all(), f"{label}: non-finite F_pre (a wait gave up?)"
    assert torch.equal(bits(f["F_pre"]), bits(pre_own)), f"{label}: F_pre differs from mhc_pre(X_next, H_next)"
    idx = torch.as_tensor(rows, device="cuda", dtype=torch.long)
    xn = _f64(f["X_next"].index_select(0, idx))
    co = oracle.coefficients(xn, _f64(nxt["phi"]), nxt["alpha_pre"], nxt["alpha_post"],
                             nxt["alpha_res"], nxt["b_pre"].double().cpu().numpy(),
                             nxt["b_post"].double().cpu().numpy(),
                             nxt["b_res"].double().cpu().numpy(), n, C)
    g = {k: f[k].index_select(0, idx).double().cpu().numpy() for k in ("logits", "r", "H")}
    row_err = np.abs(g["logits"] - co["logits"]).max(1)
    assert np.all(row_err <= 2e-3 * np.abs(co["logits"]).max(1)), f"{label}: logits"
    assert np.all(np.abs(g["r"] - co["r"]) <= 2e-3 * co["r"]), f"{label}: r"
    assert np.abs(g["H"] - co["H"]).max() <= 1e-3, f"{label}: H"
    fo = oracle.pre_mix(xn, co["H"][:, :n], n, C)
    gp = _f64(f["F_pre"].index_select(0, idx))
    assert np.all(np.abs(gp - fo) <= 2e-2 + 1e-2 * np.abs(fo)), f"{label}: F_pre vs oracle"
    # with the call's own H_pre, F_pre is one bf16 rounding (2^-8 relative) of
    # the exact mix, plus fp32 accumulation slack
    fo_own = oracle.pre_mix(xn, g["H"][:, :n], n, C)
    slack = 2.0 ** -8 * np.abs(fo_own) + 1e-6 * (np.abs(fo_own).max() + 1.0)
    assert np.all(np.abs(gp - fo_own) <= slack), f"{label}: F_pre rounding"
    # against mhc_coeffs on the same X_next: only summation order differs
    rel = ((f["logits"] - ref["logits"]).abs().max() / ref["logits"].abs().max()).item()
    assert rel < 1e-4, f"{label}: logits vs mhc_coeffs {rel}"
    assert (f["H"] - ref["H"]).abs().max().item() < 1e-4, f"{label}: H vs mhc_coeffs"
    assert ((f["r"] - ref["r"]).abs() / ref["r"]).max().item() < 1e-5, f"{label}: r vs mhc_coeffs"


def _rows(B):
    if B <= 256:
        return list(range(B))
    rng = np.random.default_rng(B)
    return sorted(set([0, 1, 15, 16, B // 2, B - 17, B - 1] + rng.choice(B, 40, replace=False).tolist()))


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large", "wide"])
def test_named(name, route):
    cfg = synth.CONFIGS[name]
    _only_pass8(route, cfg["n"])
    one = mhc.mhc_post_res_coeffs_pre_one_pass(cfg["B"], cfg["n"], cfg["C"])
    _say(f"post_res_coeffs_pre {name} route={route} one_pass={one}")
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


@pytest.mark.parametrize("n", [4, 8])
def test_giveup_word_is_reported(n, tune):
    """mhc_post_res_coeffs_pre_check reports a set give-up word as
    MHC_ERR_INCOMPLETE, and the next call clears the word before its kernel
    runs.  The word (the last 16 bytes of the one-pass workspace) is set from
    the host after a complete call: no wait is made to give up."""
    B, C = 1024, 1024
    if n == 8:
        tune.setenv("MHC_PASS8_PRE", "1")
    assert mhc.mhc_post_res_coeffs_pre_one_pass(B, n, C)
    _say(f"post_res_coeffs_pre give-up word n={n}")
    cur, nxt = _layers(n, C, B, "normal", 4242)
    o = mhc.alloc_outputs(B, n, C)
    _coeffs(cur, cur["X"], o)
    need = mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _call(cur, nxt, o["H"], ws=ws)
    assert mhc.mhc_post_res_coeffs_pre_check(B, n, C, ws) == mhc.MHC_OK
    ws[need - 16:need - 12] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    assert mhc.mhc_post_res_coeffs_pre_check(B, n, C, ws) == mhc.MHC_ERR_INCOMPLETE
    f = _call(cur, nxt, o["H"], ws=ws)
    assert mhc.mhc_post_res_coeffs_pre_check(B, n, C, ws) == mhc.MHC_OK
    assert not torch.isnan(f["F_pre"].float()).any()


def test_route_query(tune):
    tune.delenv("MHC_SMALL_MAX_B", raising=False)
    tune.delenv("MHC_FUSED_PRE", raising=False)
    assert mhc.mhc_post_res_coeffs_pre_one_pass(16384, 4, 7168)
    assert mhc.mhc_post_res_coeffs_pre_one_pass(4096, 4, 4096)
    assert not mhc.mhc_post_res_coeffs_pre_one_pass(64, 4, 7168)      # small B
    assert mhc.mhc_post_res_coeffs_pre_one_pass(64, 4, 256)           # small B, one slice
    assert not mhc.mhc_post_res_coeffs_pre_one_pass(8192, 8, 4096)    # n = 8: two calls by default
    tune.setenv("MHC_PASS8_PRE", "1")
    assert mhc.mhc_post_res_coeffs_pre_one_pass(8192, 8, 4096)        # ... the n = 8 pass on request
    assert not mhc.mhc_post_res_coeffs_pre_one_pass(8192, 8, 4224)    # n = 8, 33 slices per row
    tune.delenv("MHC_PASS8_PRE")
    assert not mhc.mhc_post_res_coeffs_pre_one_pass(4096, 4, 8704)    # 17 steps per row
    tune.setenv("MHC_FUSED_PRE", "0")
    assert not mhc.mhc_post_res_coeffs_pre_one_pass(16384, 4, 7168)


# (B, n, C): ragged row tiles, a ragged last 512-channel step (C % 512 != 0),
# one to sixteen steps per row, n = 1, 2, 4; at n = 8 (the n = 8 pass) a
# ragged last 128-channel slice and 1 to 32 slices per row; n = 8 above 32
# slices and 17 steps take the two-call route.
RAGGED = [(77, 4, 544), (1, 4, 32), (33, 1, 64), (65, 2, 2080), (200, 4, 1056), (300, 4, 1536),
          (16, 2, 512), (5, 1, 1024), (257, 4, 8192), (40, 4, 8192), (19, 4, 3104), (130, 8, 96),
          (21, 4, 8704), (513, 2, 4096), (256, 4, 256), (250, 1, 992), (300, 8, 160), (257, 8, 4096),
          (1000, 8, 1056), (40, 8, 4224), (513, 8, 32), (17, 8, 4096)]


@pytest.mark.parametrize("B,n,C", RAGGED, ids=[f"B{b}n{n}C{c}" for b, n, c in RAGGED])
def test_ragged(B, n, C, route):
    _only_pass8(route, n)
    _say(f"post_res_coeffs_pre ragged B={B} n={n} C={C} route={route} "
         f"one_pass={mhc.mhc_post_res_coeffs_pre_one_pass(B, n, C)}")
    cur, nxt = _layers(n, C, B, "student_t4" if B % 2 else "normal", B * 31 + C)
    o, ref, f, pre_own = _run(cur, nxt)
    _check(cur, nxt, o, ref, f, pre_own, list(range(B)), f"B{B}n{n}C{C}")


def _tag_fill(ws):
    """Workspace words that look like complete hand-off records (the tag in
    the high half) and random bytes: the call must not read any of them."""
    w = ws[: ws.numel() // 8 * 8].view(torch.int64)
    w.fill_(0x6D48437012345678)
    ws[w.numel() * 8:].fill_(0x5A)


def _rand_fill(ws):
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device="cuda", dtype=torch.uint8))


@pytest.mark.parametrize("fill", [_tag_fill, _rand_fill], ids=["tags", "random"])
@pytest.mark.parametrize("B,n,C", [(300, 4, 1536), (600, 4, 7168), (1000, 2, 4096), (600, 8, 4096)])
def test_workspace_contents(B, n, C, fill, route):
    _only_pass8(route, n)
    _say(f"post_res_coeffs_pre workspace {fill.__name__} B={B} n={n} C={C} route={route}")
    cur, nxt = _layers(n, C, B, "normal", B + n + C)
    o, ref, f, pre_own = _run(cur, nxt, fill=fill)
    _check(cur, nxt, o, ref, f, pre_own, _rows(B), f"B{B}n{n}C{C}/{fill.__name__}")


@pytest.mark.parametrize("B", [16384, 65536], ids=["large", "B65536"])
def test_two_routes_agree(tune, B):
    """The one-pass kernel and the two calls it replaces: X_next bitwise,
    coefficients up to summation order, F_pre within one bf16 step.  At
    B = 65536 every workgroup runs 228 steps of the record hand-off (57 at the
    large workload)."""
    _say(f"post_res_coeffs_pre one pass vs two calls (n=4 C=7168 B={B})")
    cfg = dict(synth.CONFIGS["large"], B=B)
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    o = mhc.alloc_outputs(cfg["B"], cfg["n"], cfg["C"])
    _coeffs(cur, cur["X"], o)
    tune.delenv("MHC_FUSED_PRE", raising=False)
    a = _call(cur, nxt, o["H"])
    tune.setenv("MHC_FUSED_PRE", "0")
    b = _call(cur, nxt, o["H"])
    assert torch.equal(a["X_next"].view(torch.int16), b["X_next"].view(torch.int16))
    assert (a["H"] - b["H"]).abs().max().item() < 1e-4
    d = (a["F_pre"].float() - b["F_pre"].float()).abs()
    assert (d <= 2.0 ** -7 * b["F_pre"].float().abs() + 1e-6).all()


def test_deterministic():
    _say("post_res_coeffs_pre determinism (prefill)")
    cfg = synth.CONFIGS["prefill"]
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    o = mhc.alloc_outputs(cfg["B"], cfg["n"], cfg["C"])
    _coeffs(cur, cur["X"], o)
    a = _call(cur, nxt, o["H"])
    b = _call(cur, nxt, o["H"])
    for k in ("X_next", "logits", "r", "H", "F_pre"):
        assert torch.equal(a[k].view(torch.int8), b[k].view(torch.int8)), k


def test_chained_layers():
    """Three layers run as a model runs them (this call per layer) against the
    separate calls per layer (mhc_post_res, then mhc_coeffs and mhc_pre on
    X_next): X_next and F_pre stay within the bf16 tolerance of each other
    (the two routes add the split-K partials in different orders)."""
    _say("post_res_coeffs_pre chained layers (prefill)")
    cfg = synth.CONFIGS["prefill"]
    B, n, C = cfg["B"], cfg["n"], cfg["C"]
    cur, _ = _layers(n, C, B, cfg["x_dist"], cfg["seed"])
    o = mhc.alloc_outputs(B, n, C)
    _coeffs(cur, cur["X"], o)
    X, H, Xr, Hr = cur["X"], o["H"], cur["X"], o["H"]
    close = lambda a, b: ((a.float() - b.float()).abs() <= 2e-2 + 1e-2 * b.float().abs()).all()  # noqa: E731
    for layer in range(3):
        f = _call(cur | {"X": X}, cur, H)
        r = mhc.alloc_outputs(B, n, C)
        mhc.mhc_post_res(B, n, C, Xr, cur["F_out"], Hr, r["X_next"])
        _coeffs(cur, r["X_next"], r)
        mhc.mhc_pre(B, n, C, r["X_next"], r["H"], r["F_pre"])
        torch.cuda.synchronize()
        if layer == 0:
            assert torch.equal(f["X_next"].view(torch.int16), r["X_next"].view(torch.int16))
        assert close(f["X_next"], r["X_next"]), f"layer {layer}: X_next"
        assert close(f["F_pre"], r["F_pre"]), f"layer {layer}: F_pre"
        X, H, Xr, Hr = f["X_next"], f["H"], r["X_next"], r["H"]


def test_guard_bands(route):
    _say(f"post_res_coeffs_pre guard bands route={route}")
    B, n, C = 77, 4, 544
    N = n * n + 2 * n
    cur, nxt = _layers(n, C, B, "normal", 11)
    o = mhc.alloc_outputs(B, n, C)
    _coeffs(cur, cur["X"], o)
    G = 4096
    ws_bytes = mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C)

    def guarded(nbytes):
        buf = torch.full((nbytes + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
        return buf, buf[G:G + nbytes]

    bufs = {k: guarded(sz) for k, sz in (("X_next", B * n * C * 2), ("logits", B * N * 4),
                                          ("r", B * 4), ("H", B * N * 4), ("F_pre", B * C * 2),
                                          ("ws", ws_bytes))}
    mhc.mhc_post_res_coeffs_pre(B, n, C, cur["X"], cur["F_out"], o["H"], bufs["X_next"][1], nxt["phi"],
                                0.01, 0.01, 0.01, nxt["b_pre"], nxt["b_post"], nxt["b_res"],
                                bufs["logits"][1], bufs["r"][1], bufs["H"][1], bufs["F_pre"][1],
                                bufs["ws"][1], ws_bytes)
    torch.cuda.synchronize()
    for k, (buf, _) in bufs.items():
        assert (buf[:G] == 0x5A).all() and (buf[-G:] == 0x5A).all(), f"write outside {k}"


def test_oracle_chain_large():
    """The one-pass call at the large workload (n=4, C=7168, B=16384) against a
    chain the oracle computes on its own: X_next = H_res X_t + H_post F_out
    from the call's inputs ([mHC-cutile] section 2.5), rounded to bf16 as the
    next layer's input; then the next layer's logits, r, H
    (sections 2.1-2.4) and F_pre = sum_i H_pre[i] X_next[i] from that X_next.
    Every row, at the parity tolerances."""
    cfg = synth.CONFIGS["large"]
    B, n, C = cfg["B"], cfg["n"], cfg["C"]
    assert mhc.mhc_post_res_coeffs_pre_one_pass(B, n, C)
    _say("post_res_coeffs_pre oracle chain, large")
    cur, nxt = _layers(n, C, B, cfg["x_dist"], cfg["seed"])
    o = mhc.alloc_outputs(B, n, C)
    _coeffs(cur, cur["X"], o)           # this layer's H (an input of the call)
    f = _call(cur, nxt, o["H"])
    H = o["H"].double().cpu().numpy()
    phi = _f64(nxt["phi"])
    bp, bq, br = (nxt[k].double().cpu().numpy() for k in ("b_pre", "b_post", "b_res"))
    for lo in range(0, B, 1024):
        hi = min(B, lo + 1024)
        lab = f"rows {lo}..{hi - 1}"
        x = _f64(cur["X"][lo:hi])
        _, hq, hr = oracle.split_h(H[lo:hi], n)
        xn = oracle.post_res(x, _f64(cur["F_out"][lo:hi]), hq, hr, n, C)
        gx = _f64(f["X_next"][lo:hi])
        assert np.all(np.abs(gx - xn) <= 2e-2 + 1e-2 * np.abs(xn)), f"{lab}: X_next"
        xb = oracle.round_to_bf16(xn)
        co = oracle.coefficients(xb, phi, nxt["alpha_pre"], nxt["alpha_post"], nxt["alpha_res"],
                                 bp, bq, br, n, C)
        g = {k: f[k][lo:hi].double().cpu().numpy() for k in ("logits", "r", "H")}
        row_err = np.abs(g["logits"] - co["logits"]).max(1)
        assert np.all(row_err <= 2e-3 * np.abs(co["logits"]).max(1)), f"{lab}: logits"
        assert np.all(np.abs(g["r"] - co["r"]) <= 2e-3 * co["r"]), f"{lab}: r"
        assert np.abs(g["H"] - co["H"]).max() <= 1e-3, f"{lab}: H"
        fo = oracle.pre_mix(xb, co["H"][:, :n], n, C)
        gp = _f64(f["F_pre"][lo:hi])
        assert np.all(np.abs(gp - fo) <= 2e-2 + 1e-2 * np.abs(fo)), f"{lab}: F_pre"
