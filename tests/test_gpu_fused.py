"""GPU parity of mhc_post_res_coeffs: a layer's post/res apply fused with the
next layer's coefficients.

X_next must be bitwise what mhc_post_res writes; the next layer's logits, r
and H must match the fp64 oracle's coefficients of that X_next (tolerances as
in test_gpu_parity.py) and agree with mhc_coeffs run on X_next up to fp32
summation order.  The next layer uses its own phi and biases (a second seeded
draw), so a mix-up between the two layers' parameters cannot pass.
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


# Up to 256 rows mhc_post_res_coeffs runs the stand-alone apply and the
# one-launch small-B coefficient kernel; above, at n = 8, the n = 8 pass
# (mhc_onepass8.hip) up to C = 4096 and the apply with the split-K product
# beyond; "fused" forces the fused kernel of mhc_post_res_fused.hip at every
# size and n (in its default layout: several 512-channel steps per unit,
# slices changing from round to round), "fused_fixed" the same kernel in its
# fixed-slice layout (n <= 4: one step per unit, each workgroup keeping one
# slice), and "two_pass" the apply and the split-K product at n = 8
# (MHC_FUSED_N8=0).
@pytest.fixture(params=["default", "fused", "fused_fixed", "two_pass"])
def route(request, tune):
    tune.delenv("MHC_FUSED_FIXED", raising=False)
    if request.param == "two_pass":
        tune.delenv("MHC_SMALL_MAX_B", raising=False)
        tune.setenv("MHC_FUSED_N8", "0")
    elif request.param in ("fused", "fused_fixed"):
        tune.setenv("MHC_SMALL_MAX_B", "0")
        tune.setenv("MHC_FUSED_N8", "1")
        if request.param == "fused_fixed":
            tune.setenv("MHC_FUSED_FIXED", "1")
    else:
        tune.delenv("MHC_SMALL_MAX_B", raising=False)
        tune.delenv("MHC_FUSED_N8", raising=False)
    return request.param


def _f64(t):
    return oracle.bf16_bits_to_f64(synth.bf16_bits(t))


def _layers(n, C, B, x_dist, seed):
    cur = synth.make_inputs(n, C, B, x_dist, seed=seed, device="cuda")
    nxt = synth.make_inputs(n, C, 1, "normal", seed=seed + 7919, device="cuda")  # phi, biases of layer t+1
    return cur, nxt


def _run(cur, nxt):
    B, n, C = cur["B"], cur["n"], cur["C"]
    N = n * n + 2 * n
    o = mhc.alloc_outputs(B, n, C)
    mhc.mhc_coeffs(B, n, C, cur["X"], cur["phi"], cur["alpha_pre"], cur["alpha_post"],
                   cur["alpha_res"], cur["b_pre"], cur["b_post"], cur["b_res"],
                   o["logits"], o["r"], o["H"], o["workspace"])
    # reference path: stand-alone apply, then stand-alone coefficients of X_next
    mhc.mhc_post_res(B, n, C, cur["X"], cur["F_out"], o["H"], o["X_next"])
    ref = mhc.alloc_outputs(B, n, C)
    mhc.mhc_coeffs(B, n, C, o["X_next"], nxt["phi"], nxt["alpha_pre"], nxt["alpha_post"],
                   nxt["alpha_res"], nxt["b_pre"], nxt["b_post"], nxt["b_res"],
                   ref["logits"], ref["r"], ref["H"], ref["workspace"])
    # fused path
    ws = torch.empty(max(mhc.mhc_post_res_coeffs_workspace_size(B, n, C), 16), dtype=torch.uint8,
                     device="cuda")
    f = {"X_next": torch.empty_like(cur["X"]),
         "logits": torch.empty(B, N, device="cuda"), "r": torch.empty(B, device="cuda"),
         "H": torch.empty(B, N, device="cuda")}
    mhc.mhc_post_res_coeffs(B, n, C, cur["X"], cur["F_out"], o["H"], f["X_next"], nxt["phi"],
                            nxt["alpha_pre"], nxt["alpha_post"], nxt["alpha_res"], nxt["b_pre"],
                            nxt["b_post"], nxt["b_res"], f["logits"], f["r"], f["H"], ws)
    torch.cuda.synchronize()
    return o, ref, f


def _check(cur, nxt, o, ref, f, rows, label):
    n, C = cur["n"], cur["C"]
    assert torch.equal(f["X_next"].view(torch.int16), o["X_next"].view(torch.int16)), \
        f"{label}: fused X_next differs from mhc_post_res"
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
    # against the stand-alone coefficients: only summation order differs
    rel = ((f["logits"] - ref["logits"]).abs().max() / ref["logits"].abs().max()).item()
    assert rel < 1e-4, f"{label}: logits vs mhc_coeffs {rel}"
    assert (f["H"] - ref["H"]).abs().max().item() < 1e-4, f"{label}: H vs mhc_coeffs"
    assert ((f["r"] - ref["r"]).abs() / ref["r"]).max().item() < 1e-5, f"{label}: r vs mhc_coeffs"


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large", "wide"])
def test_fused_named(name, route):
    if route == "fused" and synth.CONFIGS[name]["B"] > 256 and synth.CONFIGS[name]["n"] != 8:
        pytest.skip("above 256 rows (n < 8) the default route is the fused kernel")
    if route == "fused_fixed" and synth.CONFIGS[name]["n"] == 8:
        pytest.skip("the fixed-slice layout is for n <= 4")
    if route == "two_pass" and synth.CONFIGS[name]["n"] != 8:
        pytest.skip("MHC_FUSED_N8 changes n = 8 only")
    _say(f"fused {name} route={route}")
    cfg = synth.CONFIGS[name]
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    o, ref, f = _run(cur, nxt)
    B = cfg["B"]
    # every row on the default route, in chunks (rows are independent);
    # sampled rows on the forced routes
    if route == "default" or B <= 64:
        chunks = [list(range(lo, min(B, lo + 1024))) for lo in range(0, B, 1024)]
    else:
        chunks = [sorted(set([0, 1, B // 2, B - 1] + np.random.default_rng(B).choice(B, 40, replace=False).tolist()))]
    for rows in chunks:
        _check(cur, nxt, o, ref, f, rows, f"{name} rows {rows[0]}..{rows[-1]}")


FUSED_RAGGED = [(77, 4, 544), (1, 4, 32), (130, 8, 96), (33, 1, 64), (65, 2, 2080), (200, 4, 1056),
                (17, 8, 32), (300, 4, 1536), (16, 2, 512), (5, 1, 1024), (300, 8, 160), (257, 8, 4096),
                (1000, 8, 1056), (40, 8, 4224), (513, 8, 32)]


@pytest.mark.parametrize("B,n,C", FUSED_RAGGED, ids=[f"B{b}n{n}C{c}" for b, n, c in FUSED_RAGGED])
def test_fused_ragged(B, n, C, route):
    if route == "two_pass" and n != 8:
        pytest.skip("MHC_FUSED_N8 changes n = 8 only")
    _say(f"fused ragged B={B} n={n} C={C} route={route}")
    cur, nxt = _layers(n, C, B, "student_t4" if B % 2 else "normal", B * 13 + C)
    o, ref, f = _run(cur, nxt)
    _check(cur, nxt, o, ref, f, list(range(B)), f"B{B}n{n}C{C}")


SMALL_SHAPES = [(64, 4, 256), (64, 4, 7168), (77, 4, 544), (1, 4, 32), (33, 1, 64), (65, 2, 2080),
                (200, 4, 1056), (16, 2, 512), (5, 1, 1024), (256, 4, 7168), (19, 1, 2976)]


@pytest.mark.parametrize("apply_small", [1, 0], ids=["one_kernel", "apply_then_coeffs"])
@pytest.mark.parametrize("B,n,C", SMALL_SHAPES, ids=[f"B{b}n{n}C{c}" for b, n, c in SMALL_SHAPES])
def test_fused_small_routes(B, n, C, apply_small, tune):
    """Both small-B routes of bf16 mhc_post_res_coeffs (n <= 4, up to 256 rows):
    the kernel that applies and forms the coefficients in one launch (split
    over channel ranges of all n streams, the last workgroup of a tile
    finishing it), and the apply kernel followed by the small-B coefficient
    kernel; every row against the oracle."""
    tune.delenv("MHC_SMALL_MAX_B", raising=False)
    tune.setenv("MHC_APPLY_SMALL", apply_small)
    if C % 32:
        pytest.skip("mhc_post_res_coeffs takes C % 32 == 0")
    _say(f"fused small route B={B} n={n} C={C} apply_small={apply_small}")
    cur, nxt = _layers(n, C, B, "student_t4" if B % 2 else "normal", B * 7 + C)
    o, ref, f = _run(cur, nxt)
    _check(cur, nxt, o, ref, f, list(range(B)), f"B{B}n{n}C{C} apply_small={apply_small}")


def test_fused_deterministic():
    _say("fused determinism")
    cfg = synth.CONFIGS["prefill"]
    cur, nxt = _layers(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"])
    _, _, a = _run(cur, nxt)
    _, _, b = _run(cur, nxt)
    for k in ("X_next", "logits", "r", "H"):
        assert torch.equal(a[k].view(torch.int8), b[k].view(torch.int8)), k


@pytest.mark.parametrize("B,n,C", [(77, 4, 544), (300, 8, 160)], ids=["n4", "n8"])
def test_fused_guard_bands(route, B, n, C):
    if route == "two_pass" and n != 8:
        pytest.skip("MHC_FUSED_N8 changes n = 8 only")
    _say(f"fused guard bands B={B} n={n} C={C} route={route}")
    N = n * n + 2 * n
    cur, nxt = _layers(n, C, B, "normal", 11)
    o = mhc.alloc_outputs(B, n, C)
    mhc.mhc_coeffs(B, n, C, cur["X"], cur["phi"], 0.01, 0.01, 0.01, cur["b_pre"], cur["b_post"],
                   cur["b_res"], o["logits"], o["r"], o["H"], o["workspace"])
    G = 4096
    ws_bytes = mhc.mhc_post_res_coeffs_workspace_size(B, n, C)

    def guarded(nbytes):
        buf = torch.full((nbytes + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
        return buf, buf[G:G + nbytes]

    bufs = {k: guarded(sz) for k, sz in (("X_next", B * n * C * 2), ("logits", B * N * 4),
                                          ("r", B * 4), ("H", B * N * 4), ("ws", ws_bytes))}
    mhc.mhc_post_res_coeffs(B, n, C, cur["X"], cur["F_out"], o["H"], bufs["X_next"][1], nxt["phi"],
                            0.01, 0.01, 0.01, nxt["b_pre"], nxt["b_post"], nxt["b_res"],
                            bufs["logits"][1], bufs["r"][1], bufs["H"][1], bufs["ws"][1], ws_bytes)
    torch.cuda.synchronize()
    for k, (buf, _) in bufs.items():
        assert (buf[:G] == 0x5A).all() and (buf[-G:] == 0x5A).all(), f"write outside {k}"
