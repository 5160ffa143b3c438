"""Replay of the per-layer call from a captured HIP graph.

A serving loop removes launch overhead by capturing a chain of layers once
and replaying it.  Every call of the library only enqueues kernels on the
caller's stream (no allocation, no host synchronisation, no memset node:
buffers that must start at zero are cleared by a kernel), so the calls can be
captured.  This test captures three chained layers of mhc_post_res_coeffs_pre
(or its E4M3 twin) in one graph and replays it three times.  Between replays
eager work refills the layer-0 inputs and overwrites every output and the
workspace with garbage; each replay must reproduce the eager run bitwise.

Shapes: the decode workload (bf16: the apply and the split-K coefficients in
one kernel with its arrival flags, then the pre-mix; E4M3: apply, one-launch
small-B coefficient kernel, pre-mix), the tiny workload (bf16: the
single-slice kernel, one launch per layer) and prefill-sized shapes on the
one-pass kernel (hand-off records cleared in-graph by a fill kernel).  The Lazy Pre-Norm GEMM (one persistent launch) is replayed the same
way.
"""

import sys

import pytest
import torch

import manifold_constrained_hyper_amd as mhc
import synth

pytestmark = pytest.mark.gpu

LAYERS = 3


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    mhc.load()
    yield


def _setup(n, C, B, fp8):
    make = synth.make_inputs_fp8 if fp8 else synth.make_inputs
    inp = make(n, C, B, "normal", seed=B + C, device="cuda")
    N = n * n + 2 * n
    sfx = "_fp8" if fp8 else ""
    H0 = torch.empty(B, N, device="cuda")
    lg = torch.empty(B, N, device="cuda")
    r = torch.empty(B, device="cuda")
    wsc = torch.empty(max(getattr(mhc, "mhc_coeffs" + sfx + "_workspace_size")(B, n, C), 16),
                      dtype=torch.uint8, device="cuda")
    getattr(mhc, "mhc_coeffs" + sfx)(B, n, C, inp["X"], inp["phi"], inp["alpha_pre"], inp["alpha_post"],
                                     inp["alpha_res"], inp["b_pre"], inp["b_post"], inp["b_res"],
                                     lg, r, H0, wsc)
    torch.cuda.synchronize()
    sd = torch.uint8 if fp8 else torch.bfloat16
    bufs = {
        "X": [torch.empty_like(inp["X"]) for _ in range(LAYERS + 1)],
        "H": [torch.empty(B, N, device="cuda") for _ in range(LAYERS + 1)],
        "logits": [torch.empty(B, N, device="cuda") for _ in range(LAYERS)],
        "r": [torch.empty(B, device="cuda") for _ in range(LAYERS)],
        "F_pre": [torch.empty(B, C, dtype=sd, device="cuda") for _ in range(LAYERS)],
        "ws": torch.empty(max(getattr(mhc, "mhc_post_res_coeffs_pre" + sfx + "_workspace_size")(B, n, C), 16),
                          dtype=torch.uint8, device="cuda"),
    }
    return inp, H0, bufs, getattr(mhc, "mhc_post_res_coeffs_pre" + sfx)


def _layers(inp, bufs, call, B, n, C):
    ab = (inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"], inp["b_pre"], inp["b_post"], inp["b_res"])
    for l in range(LAYERS):
        call(B, n, C, bufs["X"][l], inp["F_out"], bufs["H"][l], bufs["X"][l + 1], inp["phi"], *ab,
             bufs["logits"][l], bufs["r"][l], bufs["H"][l + 1], bufs["F_pre"][l], bufs["ws"])


def _outputs(bufs):
    out = []
    for k in ("X", "H"):
        out += [t.clone() for t in bufs[k][1:]]
    for k in ("logits", "r", "F_pre"):
        out += [t.clone() for t in bufs[k]]
    return out


def _reset(inp, H0, bufs):
    """Eager work between replays: layer-0 inputs refilled, every output and
    the workspace overwritten with garbage."""
    bufs["X"][0].copy_(inp["X"])
    bufs["H"][0].copy_(H0)
    for k in ("X", "H"):
        for t in bufs[k][1:]:
            t.view(torch.uint8).fill_(0x7F)
    for k in ("logits", "r", "F_pre"):
        for t in bufs[k]:
            t.view(torch.uint8).fill_(0x7F)
    bufs["ws"].fill_(0xA5)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("B,n,C", [(64, 4, 7168), (1024, 4, 4096), (600, 2, 2048), (64, 4, 256), (600, 8, 1024)],
                         ids=["decode", "one-pass", "one-pass-n2", "single-slice", "n8"])
def test_graph_replay_matches_eager(B, n, C, fp8):
    _replay_check(B, n, C, fp8)


def test_graph_replay_n8_one_pass(tune):
    """The n = 8 pass with the record hand-off (MHC_PASS8_PRE=1): a zero-fill
    kernel and the pass, replayed."""
    tune.setenv("MHC_PASS8_PRE", "1")
    assert mhc.mhc_post_res_coeffs_pre_one_pass(600, 8, 1024)
    _replay_check(600, 8, 1024, False)


def _replay_check(B, n, C, fp8):
    route = (mhc.mhc_post_res_coeffs_pre_fp8_one_pass if fp8 else mhc.mhc_post_res_coeffs_pre_one_pass)(B, n, C)
    _say(f"graph replay B={B} n={n} C={C} fp8={fp8} one_pass={route}")
    inp, H0, bufs, call = _setup(n, C, B, fp8)
    # eager reference
    _reset(inp, H0, bufs)
    _layers(inp, bufs, call, B, n, C)
    torch.cuda.synchronize()
    ref = _outputs(bufs)
    # capture on a side stream (as torch requires), then replay
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _layers(inp, bufs, call, B, n, C)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _layers(inp, bufs, call, B, n, C)
    torch.cuda.synchronize()
    for rep in range(3):
        _reset(inp, H0, bufs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(bufs)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i} differs"


def test_graph_replay_lazy_prenorm():
    """mhc_lazy_prenorm_gemm is one persistent launch with no memset: captured
    twice in a graph (two shapes, one the ragged case), replayed three times
    with the outputs overwritten in between, bitwise equal to the eager run."""
    _say("graph replay lazy_prenorm")
    cases = []
    for M, N, K, seed in ((1000, 776, 520, 31), (4096, 1536, 1024, 32)):
        d = synth.make_lpn_inputs(M, N, K, seed=seed, device="cuda")
        C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        r = torch.empty(M, device="cuda")
        cases.append((M, N, K, d["A"], d["W"], C, r))

    def run():
        for M, N, K, A, W, C, r in cases:
            assert mhc.mhc_lazy_prenorm_gemm(M, N, K, A, W, C, r) == mhc.MHC_OK

    run()
    torch.cuda.synchronize()
    ref = [(c[5].clone(), c[6].clone()) for c in cases]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for c in cases:
            c[5].view(torch.uint8).fill_(0x7F)
            c[6].view(torch.uint8).fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (c, (rc, rr)) in enumerate(zip(cases, ref)):
            assert torch.equal(c[5].view(torch.int16), rc.view(torch.int16)), f"replay {rep}: C of case {i} differs"
            assert torch.equal(c[6], rr), f"replay {rep}: rstd of case {i} differs"
