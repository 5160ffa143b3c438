"""mhc_post_res_coeffs_pre_noalloc (the allocation-free variant of
mhc_post_res_coeffs_pre, workspace in the library's own device array)
against mhc_post_res_coeffs_pre with a caller workspace: bitwise equal
outputs on two calls in a row, the second on a smaller problem (the array
keeps the first call's contents), plus the size limit."""

import sys

import pytest
import torch

import manifold_constrained_hyper_amd as mhc
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
    mhc.mhc_tuning_reset()
    yield


def _outputs(B, n, C):
    N = n * n + 2 * n
    return {"X_next": torch.empty(B, n * C, dtype=torch.bfloat16, device="cuda"),
            "logits": torch.full((B, N), float("nan"), device="cuda"),
            "r": torch.full((B,), float("nan"), device="cuda"),
            "H": torch.full((B, N), float("nan"), device="cuda"),
            "F_pre": torch.empty(B, C, dtype=torch.bfloat16, device="cuda")}


def _layer(B, n, C, seed):
    cur = synth.make_inputs(n, C, B, "student_t4", seed=seed, device="cuda")
    nxt = synth.make_inputs(n, C, 1, "normal", seed=seed + 1, device="cuda")
    N = n * n + 2 * n
    # this layer's coefficients: an mhc_coeffs call with a caller workspace
    H = torch.empty(B, N, device="cuda")
    ws = torch.empty(max(mhc.mhc_coeffs_workspace_size(B, n, C), 16), dtype=torch.uint8, device="cuda")
    mhc.mhc_coeffs(B, n, C, cur["X"], cur["phi"], cur["alpha_pre"], cur["alpha_post"], cur["alpha_res"],
                   cur["b_pre"], cur["b_post"], cur["b_res"], torch.empty(B, N, device="cuda"),
                   torch.empty(B, device="cuda"), H, ws)
    return cur, nxt, H


def _args(cur, nxt, H, o):
    return (cur["X"], cur["F_out"], H, o["X_next"], nxt["phi"], nxt["alpha_pre"], nxt["alpha_post"],
            nxt["alpha_res"], nxt["b_pre"], nxt["b_post"], nxt["b_res"], o["logits"], o["r"], o["H"],
            o["F_pre"])


# (B, n, C): one-pass route at a prefill-like size, then a smaller one-pass
# shape with a ragged row tile, then a shape that takes the two calls, then
# n = 8 (the n = 8 pass and mhc_pre) with a ragged last slice.
SHAPES = [(4096, 4, 4096), (333, 4, 1024), (200, 4, 512), (300, 8, 160)]


def test_noalloc_matches_caller_workspace():
    for k, (B, n, C) in enumerate(SHAPES):
        _say(f"no-alloc call {k}: B={B} n={n} C={C} one_pass={mhc.mhc_post_res_coeffs_pre_one_pass(B, n, C)}")
        cur, nxt, H = _layer(B, n, C, seed=500 + k)
        ref, got = _outputs(B, n, C), _outputs(B, n, C)
        ws = torch.empty(mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C), dtype=torch.uint8, device="cuda")
        mhc.mhc_post_res_coeffs_pre(B, n, C, *_args(cur, nxt, H, ref), ws)
        mhc.mhc_post_res_coeffs_pre_noalloc(B, n, C, *_args(cur, nxt, H, got))
        torch.cuda.synchronize()
        for name in ("X_next", "logits", "r", "H", "F_pre"):
            assert torch.equal(got[name].view(torch.int16 if got[name].dtype == torch.bfloat16 else torch.int32),
                               ref[name].view(torch.int16 if ref[name].dtype == torch.bfloat16 else torch.int32)), \
                f"call {k}: {name} differs from mhc_post_res_coeffs_pre"
        assert mhc.mhc_post_res_coeffs_pre_check(B, n, C, None) == mhc.MHC_OK
        assert mhc.mhc_post_res_coeffs_pre_check(B, n, C, ws) == mhc.MHC_OK


def test_noalloc_n8_beyond_the_array(tune):
    """At n = 8 the n = 8 pass's partials outgrow the array above B = 3236
    (C = 4096): the call then runs the apply and split-K product route, the
    workspace call's route with MHC_FUSED_N8=0 (bitwise the same results)."""
    B, n, C = 4096, 8, 4096
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C) > mhc.MHC_NOALLOC_SCRATCH_BYTES
    _say(f"no-alloc call beyond the array: B={B} n={n} C={C}")
    cur, nxt, H = _layer(B, n, C, seed=777)
    ref, got = _outputs(B, n, C), _outputs(B, n, C)
    mhc.mhc_post_res_coeffs_pre_noalloc(B, n, C, *_args(cur, nxt, H, got))
    assert mhc.mhc_post_res_coeffs_pre_check(B, n, C, None) == mhc.MHC_OK
    tune.setenv("MHC_FUSED_N8", "0")
    ws = torch.empty(mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C), dtype=torch.uint8, device="cuda")
    mhc.mhc_post_res_coeffs_pre(B, n, C, *_args(cur, nxt, H, ref), ws)
    torch.cuda.synchronize()
    for name in ("X_next", "logits", "r", "H", "F_pre"):
        assert torch.equal(got[name].view(torch.int16 if got[name].dtype == torch.bfloat16 else torch.int32),
                           ref[name].view(torch.int16 if ref[name].dtype == torch.bfloat16 else torch.int32)), \
            f"{name} differs from the split-K route's workspace call"


def test_noalloc_rejects_oversized_shape():
    B, n, C = 65536, 4, 7168
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C) > mhc.MHC_NOALLOC_SCRATCH_BYTES
    A = 1 << 44
    a = [A + k * (1 << 38) for k in range(12)]
    st = mhc.mhc_post_res_coeffs_pre_noalloc(B, n, C, *a[:5], 0.01, 0.01, 0.01, *a[5:], stream=0,
                                             check=False)
    assert st == mhc.MHC_ERR_WORKSPACE
