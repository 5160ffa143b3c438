"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (fixed for the method's outputs):
  logits  row-normwise: max_k |g - o| <= 2e-3 * max_k |o|   (per row)
  r       elementwise relative 2e-3
  H       absolute 1e-3 (H_pre, H_post, H_res)
  F_pre, X_next (bf16)  |g - o| <= 2e-2 + 1e-2 * |o|   elementwise
Stricter checks on top: with the GPU's own H fed to the oracle's apply steps,
the bf16 outputs must sit within one bf16 rounding of the fp64 value.

Every output element is compared with the oracle, at the full-size workloads
too (in chunks of rows: rows are independent in every step) on the default
product, and on sampled rows for the alternative products, plus properties
checked on all rows.
"""

import os
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
    mhc.load()  # fails loudly if libmhc.so is missing
    yield


# mhc_coeffs has several implementations, and every one must meet the bar:
#   default  whatever the call picks (above 256 rows: the persistent product
#          for bf16 at n <= 4, the split-K product through LDS at n = 8);
#   pass8  the product-only mode of the n = 8 pass (MHC_GEMM_ALGO=3; n = 8
#          shapes only);
#   lds    split-K product with X staged through LDS by direct-to-LDS loads,
#          then the combine kernel (MHC_GEMM_ALGO=1);
#   reg    the same with MFMA operands loaded straight from global memory
#          (MHC_GEMM_ALGO=0);
#   small  the one-launch small-B kernel (the default up to 256 rows; forced
#          here for every size it supports with MHC_SMALL_MAX_B);
#   persist  the product in the persistent kernel of mhc_post_res_coeffs
#          (product only, MHC_GEMM_ALGO=2, also at n = 8), then the combine
#          kernel.
#   lds128x5, lds128x6  the LDS-staged product in 128-k chunks with a 5- or
#          6-deep ring (MHC_GEMM_KC, MHC_GEMM_STAGES; bf16, n <= 4).
#   lds8, lds8k256  the LDS-staged product with eight waves per workgroup
#          (128-row tiles; MHC_GEMM_WAVES=8), in 128-k chunks (four stages;
#          three at n = 8) or 256-k chunks (two stages, n <= 4).
#   ldsmb2  four waves with two 16-row blocks each (MHC_GEMM_MB=2; changes
#          the shape at n = 8 only).
#   ldsk256 four waves, 256-k chunks in two stages (MHC_GEMM_KC=256; changes
#          the shape at n = 8 only).
#   xreg   eight waves with X and phi through registers into single LDS slots
#          (MHC_GEMM_XREG=2; n = 4 and 8, bf16).
GEMM_ALGOS = ["default", "lds", "reg", "small", "persist", "lds128x5", "lds128x6", "lds8", "lds8k256",
              "ldsmb2", "ldsk256", "xreg", "pass8"]


def _only_n8(gemm_algo, n, C=0):
    if gemm_algo == "pass8" and (n != 8 or C % 32):
        pytest.skip("the n = 8 pass takes n = 8, C % 32 == 0")


@pytest.fixture(params=GEMM_ALGOS)
def gemm_algo(request, tune):
    tune.delenv("MHC_GEMM_ALGO", raising=False)
    if request.param == "small":
        tune.setenv("MHC_SMALL_MAX_B", str(1 << 30))
    else:
        tune.setenv("MHC_SMALL_MAX_B", "0")
        if request.param == "reg":
            tune.setenv("MHC_GEMM_ALGO", "0")
        elif request.param.startswith("lds"):
            tune.setenv("MHC_GEMM_ALGO", "1")
        elif request.param == "persist":
            tune.setenv("MHC_GEMM_ALGO", "2")
        elif request.param == "pass8":
            tune.setenv("MHC_GEMM_ALGO", "3")
        if request.param.startswith("lds128x"):
            tune.setenv("MHC_GEMM_KC", 128)
            tune.setenv("MHC_GEMM_STAGES", int(request.param[-1]))
        if request.param.startswith("lds8"):
            tune.setenv("MHC_GEMM_WAVES", 8)
            if request.param == "lds8k256":
                tune.setenv("MHC_GEMM_KC", 256)
        if request.param == "ldsmb2":
            tune.setenv("MHC_GEMM_MB", 2)
        if request.param == "ldsk256":
            tune.setenv("MHC_GEMM_KC", 256)
        if request.param == "xreg":
            tune.setenv("MHC_GEMM_ALGO", "1")
            tune.setenv("MHC_GEMM_XREG", 2)
    return request.param


def run_forward(inp, out=None):
    B, n, C = inp["B"], inp["n"], inp["C"]
    o = out if out is not None else mhc.alloc_outputs(B, n, C)
    mhc.mhc_coeffs(B, n, C, inp["X"], inp["phi"], inp["alpha_pre"], inp["alpha_post"],
                   inp["alpha_res"], inp["b_pre"], inp["b_post"], inp["b_res"],
                   o["logits"], o["r"], o["H"], o["workspace"])
    mhc.mhc_pre(B, n, C, inp["X"], o["H"], o["F_pre"])
    mhc.mhc_post_res(B, n, C, inp["X"], inp["F_out"], o["H"], o["X_next"])
    torch.cuda.synchronize()
    return o


def _f64_bf16(t):
    return oracle.bf16_bits_to_f64(synth.bf16_bits(t))


def oracle_rows(inp, rows):
    """fp64 oracle on the given rows of a device input set."""
    idx = torch.as_tensor(rows, device=inp["X"].device, dtype=torch.long)
    return oracle.forward(
        _f64_bf16(inp["X"].index_select(0, idx)), _f64_bf16(inp["phi"]),
        inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"],
        inp["b_pre"].double().cpu().numpy(), inp["b_post"].double().cpu().numpy(),
        inp["b_res"].double().cpu().numpy(), _f64_bf16(inp["F_out"].index_select(0, idx)),
        inp["n"], inp["C"])


def gpu_rows(o, rows):
    idx = torch.as_tensor(rows, device=o["H"].device, dtype=torch.long)
    return {
        "logits": o["logits"].index_select(0, idx).double().cpu().numpy(),
        "r": o["r"].index_select(0, idx).double().cpu().numpy(),
        "H": o["H"].index_select(0, idx).double().cpu().numpy(),
        "F_pre": _f64_bf16(o["F_pre"].index_select(0, idx)),
        "X_next": _f64_bf16(o["X_next"].index_select(0, idx)),
    }


def assert_parity(g, ref, label):
    lg, lo = g["logits"], ref["logits"]
    row_err = np.abs(lg - lo).max(axis=1)
    row_scale = np.abs(lo).max(axis=1)
    assert np.all(row_err <= 2e-3 * row_scale), f"{label}: logits {row_err.max()} vs {row_scale.min()}"
    assert np.all(np.abs(g["r"] - ref["r"]) <= 2e-3 * np.abs(ref["r"])), f"{label}: r"
    herr = np.abs(g["H"] - ref["H"]).max()
    assert herr <= 1e-3, f"{label}: H abs err {herr}"
    for k in ("F_pre", "X_next"):
        d = np.abs(g[k] - ref[k])
        bound = 2e-2 + 1e-2 * np.abs(ref[k])
        bad = np.count_nonzero(d > bound)
        assert bad == 0, f"{label}: {k} {bad} elements out of tolerance, max err {d.max()}"
    assert np.all(np.isfinite(g["X_next"])) and np.all(np.isfinite(g["F_pre"]))


def assert_apply_tight(inp, o, rows, g):
    """Apply steps with the GPU's own H: within one bf16 rounding (2^-8
    relative) plus fp32 accumulation slack of the fp64 value."""
    n, C = inp["n"], inp["C"]
    idx = torch.as_tensor(rows, device=inp["X"].device, dtype=torch.long)
    x = _f64_bf16(inp["X"].index_select(0, idx))
    f = _f64_bf16(inp["F_out"].index_select(0, idx))
    hp, hq, hr = oracle.split_h(g["H"], n)
    fpre = oracle.pre_mix(x, hp, n, C)
    xn = oracle.post_res(x, f, hq, hr, n, C)
    for got, ref in ((g["F_pre"], fpre), (g["X_next"], xn)):
        slack = 2.0 ** -8 * np.abs(ref) + 1e-6 * (np.abs(ref).max() + 1.0)
        d = np.abs(got - ref)
        assert np.all(d <= slack), f"apply: max excess {(d - slack).max()}"


def sample_rows(B, k=64, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, B // 2, B - 2, B - 1]
    rest = rng.choice(B, size=min(B, k), replace=False).tolist()
    return sorted(set(r for r in fixed + rest if 0 <= r < B))


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_parity_full(name, gemm_algo):
    _only_n8(gemm_algo, synth.CONFIGS[name]["n"])
    _say(f"parity full {name} gemm={gemm_algo}")
    inp = synth.make_config(name, device="cuda")
    o = run_forward(inp)
    rows = list(range(inp["B"]))
    g = gpu_rows(o, rows)
    assert_parity(g, oracle_rows(inp, rows), name)
    assert_apply_tight(inp, o, rows, g)


@pytest.mark.parametrize("name", ["prefill", "large", "wide"])
def test_parity_every_row_and_properties(name, gemm_algo):
    _only_n8(gemm_algo, synth.CONFIGS[name]["n"])
    _say(f"parity every row {name} gemm={gemm_algo}")
    inp = synth.make_config(name, device="cuda")
    o = run_forward(inp)
    B, n, C = inp["B"], inp["n"], inp["C"]
    # every row against the oracle on the default product (in chunks of rows:
    # rows are independent); the other products on sampled rows here, and on
    # every row at the smaller shapes
    chunks = ([list(range(lo, min(B, lo + 1024))) for lo in range(0, B, 1024)] if gemm_algo == "default"
              else [sample_rows(B, 48, seed=B)])
    for rows in chunks:
        g = gpu_rows(o, rows)
        assert_parity(g, oracle_rows(inp, rows), f"{name} rows {rows[0]}..{rows[-1]}")
        assert_apply_tight(inp, o, rows, g)
    # properties on every row
    H = o["H"].double()
    assert torch.isfinite(H).all() and torch.isfinite(o["logits"]).all()
    assert ((H[:, :n] > 0) & (H[:, :n] < 1)).all()
    assert ((H[:, n:2 * n] > 0) & (H[:, n:2 * n] < 2)).all()
    hres = H[:, 2 * n:].reshape(B, n, n)
    assert (hres.sum(1) - 1).abs().max().item() < 1e-5        # columns: last step
    assert (hres.sum(2) - 1).abs().max().item() < 1e-3        # rows: near 1
    assert (o["r"] > 0).all()
    # stream-sum conservation per row chunk: sum_i X_next_i = sum_j colsum_j X_j + (sum H_post) F
    for lo in range(0, B, 1024):
        hi = min(B, lo + 1024)
        x3 = inp["X"][lo:hi].double().reshape(hi - lo, n, C)
        y = o["X_next"][lo:hi].double().reshape(hi - lo, n, C).sum(1)
        want = torch.einsum("bj,bjc->bc", hres[lo:hi].sum(1), x3) + \
            H[lo:hi, n:2 * n].sum(1, keepdim=True) * inp["F_out"][lo:hi].double()
        # each of the n bf16 outputs carries at most half an ulp (2^-9 relative)
        mag = x3.abs().amax(1) + 2.0 * inp["F_out"][lo:hi].double().abs()
        tol = n * 2.0 ** -8 * mag + 1e-3 + 1e-5 * want.abs()
        assert ((y - want).abs() <= tol).all(), f"{name}: conservation rows {lo}..{hi}"
        assert torch.isfinite(o["X_next"][lo:hi]).all() and torch.isfinite(o["F_pre"][lo:hi]).all()


# ----------------------------------------------------------------------------
# ragged and degenerate shapes (every element against the oracle)
# ----------------------------------------------------------------------------

RAGGED = [(77, 4, 264), (1, 4, 8), (130, 8, 72), (33, 1, 24), (65, 2, 40), (200, 4, 2056),
          (3, 8, 8), (129, 2, 8), (1000, 1, 8), (64, 4, 64), (257, 4, 520), (300, 8, 160),
          (257, 8, 4096), (1000, 8, 1056), (40, 8, 4224)]


@pytest.mark.parametrize("B,n,C", RAGGED, ids=[f"B{b}n{n}C{c}" for b, n, c in RAGGED])
def test_parity_ragged(B, n, C, gemm_algo):
    _only_n8(gemm_algo, n, C)
    _say(f"parity ragged B={B} n={n} C={C} gemm={gemm_algo}")
    inp = synth.make_inputs(n, C, B, "student_t4" if B % 2 else "normal", seed=B * 31 + C,
                            device="cuda")
    o = run_forward(inp)
    rows = list(range(B))
    g = gpu_rows(o, rows)
    assert_parity(g, oracle_rows(inp, rows), f"B{B}n{n}C{C}")
    assert_apply_tight(inp, o, rows, g)


def test_empty_batch_is_noop():
    _say("empty batch")
    for fn_args in ((mhc.mhc_pre, (0, 4, 64, None, None, None)),
                    (mhc.mhc_post_res, (0, 4, 64, None, None, None, None))):
        assert fn_args[0](*fn_args[1]) == mhc.MHC_OK
    e = torch.empty(0, device="cuda")
    assert mhc.mhc_coeffs(0, 4, 64, e, e, 0.01, 0.01, 0.01, e, e, e, e, e, e, e) == mhc.MHC_OK


# ----------------------------------------------------------------------------
# injected coefficients: exact structure of the apply steps
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_injected_coefficients_exact(n):
    _say(f"injected coefficients n={n}")
    B, C = 37, 136
    inp = synth.make_inputs(n, C, B, seed=5 + n, device="cuda")
    N = n * n + 2 * n
    X, F = inp["X"], inp["F_out"]
    x3 = X.reshape(B, n, C)
    H = torch.zeros(B, N, device="cuda")
    H[:, 2 * n:] = torch.eye(n, device="cuda").reshape(-1)        # H_res = I, H_post = 0
    Y = torch.empty_like(X)
    mhc.mhc_post_res(B, n, C, X, F, H, Y)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), X.view(torch.int16))
    perm = torch.roll(torch.arange(n, device="cuda"), 1)
    P = torch.zeros(n, n, device="cuda")
    P[torch.arange(n, device="cuda"), perm] = 1.0                    # out_i = X_{perm[i]}
    H[:, 2 * n:] = P.reshape(-1)
    mhc.mhc_post_res(B, n, C, X, F, H, Y)
    torch.cuda.synchronize()
    assert torch.equal(Y.reshape(B, n, C).view(torch.int16), x3[:, perm].view(torch.int16))
    H[:, 2 * n:] = 0
    H[:, n:2 * n] = 1.0                                              # X_next_i = F_out
    mhc.mhc_post_res(B, n, C, X, F, H, Y)
    torch.cuda.synchronize()
    assert torch.equal(Y.reshape(B, n, C).view(torch.int16),
                       F[:, None, :].expand(B, n, C).view(torch.int16))
    Fp = torch.empty(B, C, dtype=torch.bfloat16, device="cuda")
    for k in range(n):
        H.zero_()
        H[:, k] = 1.0
        mhc.mhc_pre(B, n, C, X, H, Fp)
        torch.cuda.synchronize()
        assert torch.equal(Fp.view(torch.int16), x3[:, k].contiguous().view(torch.int16))


# ----------------------------------------------------------------------------
# determinism, split invariance, buffer bounds
# ----------------------------------------------------------------------------

def test_bitwise_deterministic():
    _say("determinism prefill")
    inp = synth.make_config("prefill", device="cuda")
    a = run_forward(inp)
    b = run_forward(inp)
    for k in ("logits", "r", "H", "F_pre", "X_next"):
        assert torch.equal(a[k].view(torch.int8), b[k].view(torch.int8)), k


def test_small_path_deterministic_and_matches_split(tune):
    _say("small path vs split path, decode")
    inp = synth.make_config("decode", device="cuda")
    tune.setenv("MHC_SMALL_MAX_B", str(1 << 30))
    a = run_forward(inp)
    b = run_forward(inp)
    for k in ("logits", "r", "H"):
        assert torch.equal(a[k].view(torch.int8), b[k].view(torch.int8)), k
    tune.setenv("MHC_SMALL_MAX_B", "0")
    c = run_forward(inp)
    rel = (a["logits"] - c["logits"]).abs().max() / c["logits"].abs().max()
    assert rel.item() < 1e-5
    assert ((a["r"] - c["r"]).abs() / c["r"]).max().item() < 1e-5
    assert (a["H"] - c["H"]).abs().max().item() < 1e-5


@pytest.mark.parametrize("fill", ["zeros", "ones", "random", "near_done"])
def test_small_path_any_workspace_contents(tune, fill):
    """The small-B kernel keeps per-tile counters in the workspace; whatever
    the workspace held before the call, the result is the same bits."""
    _say(f"small path, workspace filled with {fill}")
    tune.setenv("MHC_SMALL_MAX_B", str(1 << 30))
    inp = synth.make_inputs(4, 1024, 77, "normal", seed=4242, device="cuda")
    ref = run_forward(inp)
    B, n, C = inp["B"], inp["n"], inp["C"]
    o = mhc.alloc_outputs(B, n, C)
    ws = o["workspace"]
    if fill == "zeros":
        ws.zero_()
    elif fill == "ones":
        ws.fill_(-1)
    elif fill == "random":
        g = torch.Generator(device="cpu").manual_seed(5)
        ws.copy_(torch.randint(-128, 128, ws.shape, generator=g, dtype=torch.int8).to(ws.device))
    else:
        # every 64-bit word holds an arbitrary epoch with a count one short of a
        # full tile, the worst case for a counter that is not reset
        w64 = ws[: ws.numel() // 8 * 8].view(torch.int64)
        S = mhc.mhc_coeffs_split_k(B, n, C)
        w64.fill_((0x123456789A << 16) | (S - 1))
    for _ in range(2):
        mhc.mhc_coeffs(B, n, C, inp["X"], inp["phi"], inp["alpha_pre"], inp["alpha_post"],
                       inp["alpha_res"], inp["b_pre"], inp["b_post"], inp["b_res"],
                       o["logits"], o["r"], o["H"], ws)
        torch.cuda.synchronize()
        for k in ("logits", "r", "H"):
            assert torch.equal(o[k].view(torch.int8), ref[k].view(torch.int8)), (fill, k)


def test_split_k_invariance(tune, gemm_algo):
    _only_n8(gemm_algo, synth.CONFIGS["decode"]["n"])
    _say(f"split-K invariance decode gemm={gemm_algo}")
    inp = synth.make_config("decode", device="cuda")
    ref = None
    for s in ("1", "3", "17", "112"):
        tune.setenv("MHC_SPLIT_K", s)
        o = run_forward(inp)
        if ref is None:
            ref = {k: v.clone() for k, v in o.items()}
            continue
        rel = (o["logits"] - ref["logits"]).abs().max() / ref["logits"].abs().max()
        assert rel.item() < 1e-5, s
        assert (o["H"] - ref["H"]).abs().max().item() < 1e-5, s


def test_output_guard_bands():
    _say("guard bands")
    B, n, C = 77, 4, 264
    N = n * n + 2 * n
    inp = synth.make_inputs(n, C, B, seed=3, device="cuda")
    G = 4096  # guard bytes on each side

    def guarded(nbytes):
        buf = torch.full((nbytes + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
        return buf, buf[G:G + nbytes]

    ws_bytes = mhc.mhc_coeffs_workspace_size(B, n, C)
    bufs = {k: guarded(sz) for k, sz in (("logits", B * N * 4), ("r", B * 4), ("H", B * N * 4),
                                          ("F_pre", B * C * 2), ("X_next", B * n * C * 2),
                                          ("ws", ws_bytes))}
    mhc.mhc_coeffs(B, n, C, inp["X"], inp["phi"], 0.01, 0.01, 0.01, inp["b_pre"], inp["b_post"],
                   inp["b_res"], bufs["logits"][1], bufs["r"][1], bufs["H"][1], bufs["ws"][1],
                   ws_bytes)
    Hf = bufs["H"][1].view(torch.float32)
    mhc.mhc_pre(B, n, C, inp["X"], Hf, bufs["F_pre"][1])
    mhc.mhc_post_res(B, n, C, inp["X"], inp["F_out"], Hf, bufs["X_next"][1])
    torch.cuda.synchronize()
    for k, (buf, _) in bufs.items():
        assert (buf[:G] == 0x5A).all() and (buf[-G:] == 0x5A).all(), f"write outside {k}"
