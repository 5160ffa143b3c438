"""GPU parity of mhc_coeffs_pre and mhc_coeffs_pre_fp8: one layer's
coefficients and pre-mix from X_t in one pass where the shape allows (the
first layer's counterpart of mhc_post_res_coeffs_pre).

Checks, for every shape, in bf16 and in E4M3:
  F_pre       bitwise what mhc_pre(X_t, H) (mhc_pre_fp8) writes with the
              call's own H, and no NaN (a wait that gave up);
  logits, r, H and F_pre against the fp64 oracle on X_t (tolerances of
              test_gpu_parity.py; for E4M3 each F_pre code is one of the two
              neighbours of the exact mix with the call's own H_pre), on
              every row on the default route;
  the coefficients against mhc_coeffs (mhc_coeffs_fp8) on X_t up to fp32
              summation order.

Routes: "default" (bf16 up to 256 rows at n <= 4 with n*C <= 1024: the
single-slice kernel of mhc_layer_small.hip; one pass above 256 rows for
n <= 4, C % 32 == 0 and at most sixteen 512-channel steps per row; mhc_coeffs
then mhc_pre otherwise),
"onepass" (small-B limit 0, so the one-pass kernel also runs the small shapes
it can take) and "twocalls" (MHC_FUSED_PRE=0).
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


# "pass8pre": the n = 8 pass in one pass (MHC_PASS8_PRE=1, bf16 n = 8 shapes
# only; by default n = 8 runs as the two calls).
@pytest.fixture(params=["default", "onepass", "twocalls", "pass8pre"])
def route(request, tune):
    for k in ("MHC_FUSED_PRE", "MHC_SMALL_MAX_B", "MHC_FUSED_FP8", "MHC_PASS8_PRE"):
        tune.delenv(k, raising=False)
    if request.param == "onepass":
        tune.setenv("MHC_SMALL_MAX_B", "0")
    elif request.param == "twocalls":
        tune.setenv("MHC_FUSED_PRE", "0")
    elif request.param == "pass8pre":
        tune.setenv("MHC_PASS8_PRE", "1")
    return request.param


def _only_pass8(route, n, dt="bf16"):
    if route == "pass8pre" and (n != 8 or dt != "bf16"):
        pytest.skip("MHC_PASS8_PRE changes bf16 n = 8 only")


class _Api:
    """The entry points and decoders of one element type."""

    def __init__(self, fp8):
        self.fp8 = fp8
        self.call = mhc.mhc_coeffs_pre_fp8 if fp8 else mhc.mhc_coeffs_pre
        self.ws_size = mhc.mhc_coeffs_pre_fp8_workspace_size if fp8 else mhc.mhc_coeffs_pre_workspace_size
        self.one_pass = mhc.mhc_coeffs_pre_fp8_one_pass if fp8 else mhc.mhc_coeffs_pre_one_pass
        self.coeffs = mhc.mhc_coeffs_fp8 if fp8 else mhc.mhc_coeffs
        self.coeffs_ws = mhc.mhc_coeffs_fp8_workspace_size if fp8 else mhc.mhc_coeffs_workspace_size
        self.pre = mhc.mhc_pre_fp8 if fp8 else mhc.mhc_pre

    def inputs(self, n, C, B, x_dist, seed):
        make = synth.make_inputs_fp8 if self.fp8 else synth.make_inputs
        return make(n, C, B, x_dist, seed=seed, device="cuda")

    def f_pre(self, B, C):
        return torch.empty(B, C, dtype=torch.uint8 if self.fp8 else torch.bfloat16, device="cuda")

    def decode(self, t):
        """Exact fp64 values of bf16 or E4M3 rows."""
        if self.fp8:
            return F8.e4m3_decode(synth.e4m3_codes(t))
        return oracle.bf16_bits_to_f64(synth.bf16_bits(t))

    def same_bits(self, a, b):
        return torch.equal(a.view(torch.uint8), b.view(torch.uint8))

    def has_nan(self, t):
        if self.fp8:
            return bool(((t.view(torch.uint8) & 0x7F) == 0x7F).any())
        return bool(torch.isnan(t.float()).any())


APIS = {"bf16": _Api(False), "fp8": _Api(True)}


def _ws(nbytes):
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")


def _call(api, inp, ws=None, fill=None):
    """mhc_coeffs_pre(_fp8) on inp; fresh outputs."""
    B, n, C = inp["B"], inp["n"], inp["C"]
    N = n * n + 2 * n
    if ws is None:
        ws = _ws(api.ws_size(B, n, C))
    if fill is not None:
        fill(ws)
    f = {"logits": torch.empty(B, N, device="cuda"), "r": torch.empty(B, device="cuda"),
         "H": torch.empty(B, N, device="cuda"), "F_pre": api.f_pre(B, C)}
    api.call(B, n, C, inp["X"], inp["phi"], inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
             inp["b_pre"], inp["b_post"], inp["b_res"], f["logits"], f["r"], f["H"], f["F_pre"], ws)
    torch.cuda.synchronize()
    return f


def _run(api, inp, fill=None):
    """The call, mhc_coeffs on the same X_t, and mhc_pre with the call's own H."""
    B, n, C = inp["B"], inp["n"], inp["C"]
    N = n * n + 2 * n
    f = _call(api, inp, fill=fill)
    ref = {"logits": torch.empty(B, N, device="cuda"), "r": torch.empty(B, device="cuda"),
           "H": torch.empty(B, N, device="cuda")}
    api.coeffs(B, n, C, inp["X"], inp["phi"], inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
               inp["b_pre"], inp["b_post"], inp["b_res"], ref["logits"], ref["r"], ref["H"],
               _ws(api.coeffs_ws(B, n, C)))
    pre_own = api.f_pre(B, C)
    api.pre(B, n, C, inp["X"], f["H"], pre_own)
    torch.cuda.synchronize()
    return f, ref, pre_own


def _check(api, inp, f, ref, pre_own, rows, label):
    n, C = inp["n"], inp["C"]
    assert not api.has_nan(f["F_pre"]), f"{label}: NaN in F_pre (a wait gave up?)"
    assert api.same_bits(f["F_pre"], pre_own), f"{label}: F_pre differs from mhc_pre(X_t, H)"
    idx = torch.as_tensor(rows, device="cuda", dtype=torch.long)
    x = api.decode(inp["X"].index_select(0, idx))
    co = oracle.coefficients(x, oracle.bf16_bits_to_f64(synth.bf16_bits(inp["phi"])),
                             inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
                             inp["b_pre"].double().cpu().numpy(), inp["b_post"].double().cpu().numpy(),
                             inp["b_res"].double().cpu().numpy(), n, C)
    g = {k: f[k].index_select(0, idx).double().cpu().numpy() for k in ("logits", "r", "H")}
    row_err = np.abs(g["logits"] - co["logits"]).max(1)
    assert np.all(row_err <= 2e-3 * np.abs(co["logits"]).max(1)), f"{label}: logits"
    assert np.all(np.abs(g["r"] - co["r"]) <= 2e-3 * co["r"]), f"{label}: r"
    assert np.abs(g["H"] - co["H"]).max() <= 1e-3, f"{label}: H"
    gp_raw = f["F_pre"].index_select(0, idx)
    exact_own = oracle.pre_mix(x, g["H"][:, :n], n, C)
    exact = oracle.pre_mix(x, co["H"][:, :n], n, C)
    if api.fp8:
        # with the call's own H_pre: each code is a neighbour of the exact mix
        codes = synth.e4m3_codes(gp_raw)
        slack = (n + 1) * 2.0 ** -24 * oracle.pre_mix(np.abs(x), np.abs(g["H"][:, :n]), n, C) + 1e-30
        bad = ~F8.e4m3_neighbors_ok(codes, exact_own, absolute=slack)
        assert not bad.any(), f"{label}: F_pre codes off at {np.argwhere(bad)[:5].tolist()}"
        err = np.abs(F8.e4m3_decode(codes) - exact)
        assert np.all(err <= 0.07 * np.abs(exact) + 2.0 ** -9), f"{label}: F_pre vs oracle"
    else:
        gp = api.decode(gp_raw)
        assert np.all(np.abs(gp - exact) <= 2e-2 + 1e-2 * np.abs(exact)), f"{label}: F_pre vs oracle"
        # one bf16 rounding (2^-8 relative) of the exact mix with the call's
        # own H_pre, plus fp32 accumulation slack
        slack = 2.0 ** -8 * np.abs(exact_own) + 1e-6 * (np.abs(exact_own).max() + 1.0)
        assert np.all(np.abs(gp - exact_own) <= slack), f"{label}: F_pre rounding"
    # against mhc_coeffs on the same X_t: only summation order differs
    rel = ((f["logits"] - ref["logits"]).abs().max() / ref["logits"].abs().max()).item()
    assert rel < 1e-4, f"{label}: logits vs mhc_coeffs {rel}"
    assert (f["H"] - ref["H"]).abs().max().item() < 1e-4, f"{label}: H vs mhc_coeffs"
    assert ((f["r"] - ref["r"]).abs() / ref["r"]).max().item() < 1e-5, f"{label}: r vs mhc_coeffs"


def _rows(B):
    if B <= 256:
        return list(range(B))
    rng = np.random.default_rng(B)
    return sorted(set([0, 1, 15, 16, B // 2, B - 17, B - 1] + rng.choice(B, 40, replace=False).tolist()))


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large", "wide"])
def test_named(name, dt, route):
    api = APIS[dt]
    cfg = synth.CONFIGS[name]
    _only_pass8(route, cfg["n"], dt)
    one = api.one_pass(cfg["B"], cfg["n"], cfg["C"])
    _say(f"coeffs_pre {dt} {name} route={route} one_pass={one}")
    if route == "onepass" and cfg["B"] > 256:
        pytest.skip("above 256 rows the default route already takes the one-pass kernel where it fits")
    inp = api.inputs(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    f, ref, pre_own = _run(api, inp)
    chunks = ([list(range(lo, min(cfg["B"], lo + 1024))) for lo in range(0, cfg["B"], 1024)]
              if route == "default" else [_rows(cfg["B"])])
    for rows in chunks:
        _check(api, inp, f, ref, pre_own, rows, f"{dt} {name} rows {rows[0]}..{rows[-1]}")


def test_route_query(tune):
    for k in ("MHC_SMALL_MAX_B", "MHC_FUSED_PRE", "MHC_FUSED_FP8"):
        tune.delenv(k, raising=False)
    for q in (mhc.mhc_coeffs_pre_one_pass, mhc.mhc_coeffs_pre_fp8_one_pass):
        assert q(16384, 4, 7168)
        assert q(4096, 2, 4096)
        assert not q(64, 4, 7168)       # small B
        assert not q(8192, 8, 4224)     # n = 8 above 32 slices of 128 channels
        assert not q(4096, 4, 8704)     # 17 steps per row
        assert not q(4096, 4, 7184)     # C % 32 != 0
    assert mhc.mhc_coeffs_pre_one_pass(64, 4, 256)           # small B, one slice: bf16 only
    assert not mhc.mhc_coeffs_pre_fp8_one_pass(64, 4, 256)
    assert not mhc.mhc_coeffs_pre_one_pass(8192, 8, 4096)    # n = 8: two calls by default
    tune.setenv("MHC_PASS8_PRE", "1")
    assert mhc.mhc_coeffs_pre_one_pass(8192, 8, 4096)        # ... the n = 8 pass on request, bf16 only
    assert not mhc.mhc_coeffs_pre_fp8_one_pass(8192, 8, 4096)
    tune.delenv("MHC_PASS8_PRE")
    tune.setenv("MHC_FUSED_PRE", "0")
    assert not mhc.mhc_coeffs_pre_one_pass(16384, 4, 7168)
    assert not mhc.mhc_coeffs_pre_fp8_one_pass(16384, 4, 7168)


# (B, n, C): ragged row tiles, a ragged last 512-channel step, one to sixteen
# steps per row, n = 1, 2, 4; n = 8 (bf16) in the n = 8 pass: a ragged last
# 128-channel slice, 1 to 32 slices; n = 8 above 32 slices, C % 32 != 0 and
# 17 steps take the two calls.
RAGGED = [(77, 4, 544), (1, 4, 32), (33, 1, 64), (65, 2, 2080), (300, 4, 1536), (16, 2, 512),
          (257, 4, 8192), (19, 4, 3104), (130, 8, 96), (21, 4, 8704), (513, 2, 4096), (300, 4, 1040),
          (7, 4, 48), (250, 1, 1008), (256, 2, 512), (300, 8, 160), (257, 8, 4096), (1000, 8, 1056),
          (40, 8, 4224)]


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
@pytest.mark.parametrize("B,n,C", RAGGED, ids=[f"B{b}n{n}C{c}" for b, n, c in RAGGED])
def test_ragged(B, n, C, dt, route):
    _only_pass8(route, n, dt)
    api = APIS[dt]
    _say(f"coeffs_pre {dt} ragged B={B} n={n} C={C} route={route} one_pass={api.one_pass(B, n, C)}")
    inp = api.inputs(n, C, B, "student_t4" if B % 2 else "normal", B * 37 + C)
    f, ref, pre_own = _run(api, inp)
    _check(api, inp, f, ref, pre_own, list(range(B)), f"{dt} B{B}n{n}C{C}")


def _tag_fill(ws):
    """Workspace words that look like written hand-off records, then random
    bytes: the call must read none of what it did not write itself."""
    w = ws[: ws.numel() // 8 * 8].view(torch.int64)
    w.fill_(0x3F8000003F800000)
    ws[w.numel() * 8:].fill_(0x5A)


def _rand_fill(ws):
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device="cuda", dtype=torch.uint8))


@pytest.mark.parametrize("fill", [_tag_fill, _rand_fill], ids=["records", "random"])
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_workspace_contents(dt, fill):
    api = APIS[dt]
    B, n, C = 600, 4, 7168
    _say(f"coeffs_pre {dt} workspace {fill.__name__} B={B} n={n} C={C}")
    inp = api.inputs(n, C, B, "normal", 601)
    f, ref, pre_own = _run(api, inp, fill=fill)
    _check(api, inp, f, ref, pre_own, list(range(B)), f"{dt} {fill.__name__}")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_deterministic(dt):
    api = APIS[dt]
    _say(f"coeffs_pre {dt} determinism (prefill)")
    cfg = synth.CONFIGS["prefill"]
    inp = api.inputs(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    a, b = _call(api, inp), _call(api, inp)
    for k in ("logits", "r", "H", "F_pre"):
        assert api.same_bits(a[k], b[k]), k


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_two_routes_agree(tune, dt):
    """The one pass and the two calls it replaces at the large workload:
    coefficients up to summation order, F_pre within one rounding step."""
    api = APIS[dt]
    _say(f"coeffs_pre {dt} one pass vs two calls (large)")
    cfg = synth.CONFIGS["large"]
    inp = api.inputs(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    tune.delenv("MHC_FUSED_PRE", raising=False)
    assert api.one_pass(cfg["B"], cfg["n"], cfg["C"])
    a = _call(api, inp)
    tune.setenv("MHC_FUSED_PRE", "0")
    b = _call(api, inp)
    assert (a["H"] - b["H"]).abs().max().item() < 1e-4
    assert ((a["r"] - b["r"]).abs() / b["r"]).max().item() < 1e-5
    widen = (lambda t: t.view(torch.float8_e4m3fn).float()) if api.fp8 else (lambda t: t.float())  # noqa: E731
    fa, fb = widen(a["F_pre"]), widen(b["F_pre"])
    step = 2.0 ** -3 if api.fp8 else 2.0 ** -7   # one rounding step either way, relative
    assert ((fa - fb).abs() <= step * fb.abs() + 2.0 ** -9).all()


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_giveup_word_is_reported(dt):
    """mhc_coeffs_pre_check reports a set give-up word as MHC_ERR_INCOMPLETE,
    and the next call clears it before its kernel runs.  The word is set
    from the host after a complete call: no wait is made to give up."""
    api = APIS[dt]
    B, n, C = 1024, 4, 1024
    assert api.one_pass(B, n, C)
    _say(f"coeffs_pre {dt} give-up word")
    inp = api.inputs(n, C, B, "normal", 4243)
    need = api.ws_size(B, n, C)
    ws = _ws(need)
    _call(api, inp, ws=ws)
    assert mhc.mhc_coeffs_pre_check(B, n, C, ws, fp8=api.fp8) == mhc.MHC_OK
    # the give-up word: the last 16 bytes of the pre-mix layout (that of
    # mhc_post_res_coeffs_pre); the workspace may be larger, when the two
    # calls' workspace (mhc_coeffs's) is
    word = mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C) - 16
    assert 0 < word and word + 16 <= need
    ws[word:word + 4] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    assert mhc.mhc_coeffs_pre_check(B, n, C, ws, fp8=api.fp8) == mhc.MHC_ERR_INCOMPLETE
    f = _call(api, inp, ws=ws)
    assert mhc.mhc_coeffs_pre_check(B, n, C, ws, fp8=api.fp8) == mhc.MHC_OK
    assert not api.has_nan(f["F_pre"])


def test_model_recipe():
    """The first layer by mhc_coeffs_pre, then two layers of
    mhc_post_res_coeffs_pre, against the same three layers run as separate
    calls (mhc_coeffs, mhc_pre, mhc_post_res per layer): the streams stay
    within the bf16 tolerance of each other."""
    _say("coeffs_pre model recipe (prefill)")
    cfg = synth.CONFIGS["prefill"]
    B, n, C = cfg["B"], cfg["n"], cfg["C"]
    inp = synth.make_inputs(n, C, B, cfg["x_dist"], seed=cfg["seed"], device="cuda")
    close = lambda a, b: ((a.float() - b.float()).abs() <= 2e-2 + 1e-2 * b.float().abs()).all()  # noqa: E731
    f = _call(APIS["bf16"], inp)
    r = mhc.alloc_outputs(B, n, C)
    mhc.mhc_coeffs(B, n, C, inp["X"], inp["phi"], inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
                   inp["b_pre"], inp["b_post"], inp["b_res"], r["logits"], r["r"], r["H"], r["workspace"])
    mhc.mhc_pre(B, n, C, inp["X"], r["H"], r["F_pre"])
    torch.cuda.synchronize()
    assert close(f["F_pre"], r["F_pre"])
    X, H, Xr, Hr = inp["X"], f["H"], inp["X"], r["H"]
    N = n * n + 2 * n
    for layer in range(2):
        nx = {"X_next": torch.empty_like(X), "logits": torch.empty(B, N, device="cuda"),
              "r": torch.empty(B, device="cuda"), "H": torch.empty(B, N, device="cuda"),
              "F_pre": torch.empty(B, C, dtype=torch.bfloat16, device="cuda")}
        ws = _ws(mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C))
        mhc.mhc_post_res_coeffs_pre(B, n, C, X, inp["F_out"], H, nx["X_next"], inp["phi"], inp["alpha_pre"],
                                    inp["alpha_post"], inp["alpha_res"], inp["b_pre"], inp["b_post"],
                                    inp["b_res"], nx["logits"], nx["r"], nx["H"], nx["F_pre"], ws)
        rn = mhc.alloc_outputs(B, n, C)
        mhc.mhc_post_res(B, n, C, Xr, inp["F_out"], Hr, rn["X_next"])
        mhc.mhc_coeffs(B, n, C, rn["X_next"], inp["phi"], inp["alpha_pre"], inp["alpha_post"],
                       inp["alpha_res"], inp["b_pre"], inp["b_post"], inp["b_res"], rn["logits"],
                       rn["r"], rn["H"], rn["workspace"])
        mhc.mhc_pre(B, n, C, rn["X_next"], rn["H"], rn["F_pre"])
        torch.cuda.synchronize()
        assert close(nx["X_next"], rn["X_next"]), f"layer {layer + 1}: X_next"
        assert close(nx["F_pre"], rn["F_pre"]), f"layer {layer + 1}: F_pre"
        X, H, Xr, Hr = nx["X_next"], nx["H"], rn["X_next"], rn["H"]
