"""Host-only checks of the C ABI: the library loads, exports every function
include/mhc.h declares, and rejects bad arguments before launching anything.

Almost every call here fails validation or has B == 0, so nothing is
launched and the tests run without a GPU.  Pointers are fake addresses; the
library never dereferences them on the host.  The one test that lets calls
reach a launch (to see MHC_ERR_HIP without a device) runs only on a host with
no HIP device.
"""

import ctypes
import os
import re

import pytest
import torch

import manifold_constrained_hyper_amd as mhc

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

A = 0x10000000  # fake, 16-byte aligned device addresses, far apart
STEP = 0x10000000


def _addrs(k):
    return [A + i * STEP for i in range(k)]


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(mhc.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mhc.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), f"libmhc.so does not export {name}"


def test_status_strings():
    for code in range(6):
        assert mhc.mhc_status_string(code).startswith("MHC_")
    assert mhc.mhc_status_string(99) == "MHC_ERR_UNKNOWN"


def test_workspace_and_split_host_functions():
    for (B, n, C) in ((64, 4, 256), (4096, 4, 4096), (64, 4, 7168), (16384, 4, 7168),
                      (8192, 8, 4096), (77, 1, 24), (5, 2, 8)):
        S = mhc.mhc_coeffs_split_k(B, n, C)
        N = n * n + 2 * n
        assert 1 <= S <= max(1, (n * C + 127) // 128)
        # fp32 partials [S, B, N+1] plus, for the LDS-staged product, a packed
        # copy of phi and a small zero block
        ws = mhc.mhc_coeffs_workspace_size(B, n, C)
        assert ws >= S * B * (N + 1) * 4
        assert ws <= S * B * (N + 1) * 4 + 1024 + ((n * C + 255) // 32 + 8) * ((N + 15) // 16) * 1024 + 256
    assert mhc.mhc_coeffs_workspace_size(0, 4, 256) == 0
    assert mhc.mhc_coeffs_workspace_size(10, 3, 256) == 0
    assert mhc.mhc_coeffs_split_k(10, 4, 12) == 0


def _coeffs(B=16, n=4, C=64, ptrs=None, ws_bytes=None, **over):
    p = dict(zip(["X", "phi", "bp", "bq", "br", "logits", "r", "H", "ws"], ptrs or _addrs(9)))
    p.update(over)
    if ws_bytes is None:
        ws_bytes = max(mhc.mhc_coeffs_workspace_size(B, n, C), 16)
    return mhc.mhc_coeffs(B, n, C, p["X"], p["phi"], 0.01, 0.01, 0.01, p["bp"], p["bq"], p["br"],
                          p["logits"], p["r"], p["H"], p["ws"], ws_bytes, stream=0, check=False)


def test_coeffs_validation():
    assert _coeffs(B=0) == mhc.MHC_OK                                   # empty: nothing launched
    assert _coeffs(B=0, X=None, H=None, ws=None) == mhc.MHC_OK          # pointers not inspected at B == 0
    assert _coeffs(B=-1) == mhc.MHC_ERR_INVALID_ARG
    assert _coeffs(n=0) == mhc.MHC_ERR_INVALID_ARG
    assert _coeffs(C=0) == mhc.MHC_ERR_INVALID_ARG
    assert _coeffs(n=3) == mhc.MHC_ERR_UNSUPPORTED
    assert _coeffs(C=12) == mhc.MHC_ERR_UNSUPPORTED
    for k in ("X", "phi", "bp", "bq", "br", "logits", "r", "H", "ws"):
        assert _coeffs(**{k: None}) == mhc.MHC_ERR_INVALID_ARG, k
    assert _coeffs(X=A + 8) == mhc.MHC_ERR_UNSUPPORTED                  # bf16 needs 16-byte alignment
    assert _coeffs(ws=A + 8 * STEP + 4) == mhc.MHC_ERR_UNSUPPORTED
    assert _coeffs(H=A + 7 * STEP + 2) == mhc.MHC_ERR_UNSUPPORTED       # fp32 needs 4-byte alignment
    assert _coeffs(H=A) == mhc.MHC_ERR_INVALID_ARG                      # output overlaps X
    assert _coeffs(r=A + 5 * STEP + 64) == mhc.MHC_ERR_INVALID_ARG      # r inside logits
    assert _coeffs(ws=A + 7 * STEP) == mhc.MHC_ERR_INVALID_ARG          # workspace overlaps H
    need = mhc.mhc_coeffs_workspace_size(16, 4, 64)
    assert _coeffs(ws_bytes=need - 1) == mhc.MHC_ERR_WORKSPACE


def test_pre_and_post_res_validation():
    X, H, F, Y = _addrs(4)
    ok_shape = (16, 4, 64)
    assert mhc.mhc_pre(0, 4, 64, None, None, None, stream=0, check=False) == mhc.MHC_OK
    assert mhc.mhc_pre(*ok_shape, None, H, F, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    assert mhc.mhc_pre(16, 5, 64, X, H, F, stream=0, check=False) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_pre(*ok_shape, X, H, F + 2, stream=0, check=False) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_pre(*ok_shape, X, H, X + 256, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    assert mhc.mhc_post_res(0, 4, 64, None, None, None, None, stream=0, check=False) == mhc.MHC_OK
    assert mhc.mhc_post_res(*ok_shape, X, F, H, None, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    assert mhc.mhc_post_res(*ok_shape, X, F, H, X, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    assert mhc.mhc_post_res(*ok_shape, X, F, H, F + 16, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    assert mhc.mhc_post_res(16, 4, 60, X, F, H, Y, stream=0, check=False) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_post_res(-3, 4, 64, X, F, H, Y, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG


def _fused(B=16, n=4, C=64, ws_bytes=None, **over):
    names = ["X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "ws"]
    p = dict(zip(names, _addrs(len(names))))
    p.update(over)
    if ws_bytes is None:
        ws_bytes = max(mhc.mhc_post_res_coeffs_workspace_size(B, n, C), 16)
    return mhc.mhc_post_res_coeffs(B, n, C, p["X"], p["F"], p["H"], p["Y"], p["phi"], 0.01, 0.01,
                                   0.01, p["bp"], p["bq"], p["br"], p["logits"], p["r"], p["Hn"],
                                   p["ws"], ws_bytes, stream=0, check=False)


def test_fused_validation():
    assert _fused(B=0) == mhc.MHC_OK
    assert _fused(C=40) == mhc.MHC_ERR_UNSUPPORTED                     # needs C % 32 == 0
    assert mhc.mhc_post_res_coeffs_workspace_size(16, 4, 40) == 0
    assert _fused(n=3) == mhc.MHC_ERR_UNSUPPORTED
    assert _fused(B=-2) == mhc.MHC_ERR_INVALID_ARG
    for k in ("X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "ws"):
        assert _fused(**{k: None}) == mhc.MHC_ERR_INVALID_ARG, k
    assert _fused(Y=A) == mhc.MHC_ERR_INVALID_ARG                      # X_next overlaps X_t
    assert _fused(Hn=A + 2 * STEP) == mhc.MHC_ERR_INVALID_ARG          # H_next overlaps H
    assert _fused(ws=A + 3 * STEP) == mhc.MHC_ERR_INVALID_ARG          # workspace overlaps X_next
    assert _fused(phi=A + 4 * STEP + 8) == mhc.MHC_ERR_UNSUPPORTED
    need = mhc.mhc_post_res_coeffs_workspace_size(16, 4, 64)
    assert need > 0 and _fused(ws_bytes=need - 1) == mhc.MHC_ERR_WORKSPACE


def _fused_pre(B=16, n=4, C=64, ws_bytes=None, **over):
    names = ["X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "Fp", "ws"]
    p = dict(zip(names, _addrs(len(names))))
    p.update(over)
    if ws_bytes is None:
        ws_bytes = max(mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C), 16)
    return mhc.mhc_post_res_coeffs_pre(B, n, C, p["X"], p["F"], p["H"], p["Y"], p["phi"], 0.01, 0.01,
                                       0.01, p["bp"], p["bq"], p["br"], p["logits"], p["r"], p["Hn"],
                                       p["Fp"], p["ws"], ws_bytes, stream=0, check=False)


def test_fused_pre_validation():
    assert _fused_pre(B=0) == mhc.MHC_OK
    assert _fused_pre(B=0, X=None, Fp=None, ws=None) == mhc.MHC_OK
    assert _fused_pre(C=40) == mhc.MHC_ERR_UNSUPPORTED                 # needs C % 32 == 0
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(16, 4, 40) == 0
    assert _fused_pre(n=3) == mhc.MHC_ERR_UNSUPPORTED
    assert _fused_pre(B=-2) == mhc.MHC_ERR_INVALID_ARG
    for k in ("X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "Fp", "ws"):
        assert _fused_pre(**{k: None}) == mhc.MHC_ERR_INVALID_ARG, k
    assert _fused_pre(Fp=A) == mhc.MHC_ERR_INVALID_ARG                 # F_pre overlaps X_t
    assert _fused_pre(Fp=A + 3 * STEP + 256) == mhc.MHC_ERR_INVALID_ARG   # F_pre inside X_next
    assert _fused_pre(Fp=A + 10 * STEP) == mhc.MHC_ERR_INVALID_ARG     # F_pre overlaps H_next
    assert _fused_pre(ws=A + 11 * STEP) == mhc.MHC_ERR_INVALID_ARG     # workspace overlaps F_pre
    assert _fused_pre(Fp=A + 11 * STEP + 8) == mhc.MHC_ERR_UNSUPPORTED  # F_pre needs 16-byte alignment
    need = mhc.mhc_post_res_coeffs_pre_workspace_size(16, 4, 64)
    assert need > 0 and _fused_pre(ws_bytes=need - 1) == mhc.MHC_ERR_WORKSPACE


def test_fused_pre_route_and_workspace(tune):
    tune.delenv("MHC_FUSED_PRE", raising=False)
    tune.delenv("MHC_SMALL_MAX_B", raising=False)
    one = mhc.mhc_post_res_coeffs_pre_one_pass
    assert one(16384, 4, 7168) and one(4096, 4, 4096) and one(1000, 2, 4096) and one(300, 1, 1024)
    assert not one(64, 4, 7168)          # small B: the two calls
    # small B with all n*C <= 1024 channels of a row in one slice: the single-slice kernel
    assert one(64, 4, 256) and one(1, 2, 32) and one(256, 1, 1024) and one(16, 2, 512)
    assert not one(64, 4, 288) and not one(64, 8, 96)
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(64, 4, 256) == \
        mhc.mhc_post_res_coeffs_workspace_size(64, 4, 256)
    assert not one(8192, 8, 4096)        # n = 8: two calls (the n = 8 apply pass, then mhc_pre)
    assert not one(4096, 4, 8704)        # 17 steps of 512 channels per row
    assert not one(0, 4, 7168) and not one(16, 4, 40)
    # one pass: partials [S, B, N+1] fp32 + packed phi + records [B, S, PW] of 4 bytes
    B, n, C = 16384, 4, 7168
    S, N, PW = C // 512, n * n + 2 * n, (n + 2) & ~1
    ws = mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C)
    assert ws >= S * B * (N + 1) * 4 + S * B * PW * 4
    assert ws <= S * B * (N + 1) * 4 + S * B * PW * 4 + (n * C // 32) * 2 * 1024 + 8192
    # the n = 8 apply pass: partials [S, B, 81], S = C / 128
    B8, C8 = 8192, 4096
    S8 = C8 // 128
    assert S8 * B8 * 81 * 4 <= mhc.mhc_post_res_coeffs_workspace_size(B8, 8, C8) <= S8 * B8 * 81 * 4 + 1024
    # ... and its one pass (MHC_PASS8_PRE=1): + records [B, 9, S] + the give-up word
    tune.setenv("MHC_PASS8_PRE", 1)
    assert one(8192, 8, 4096) and one(300, 8, 160)
    assert not one(8192, 8, 4224)        # n = 8 with 33 slices per row
    ws8 = mhc.mhc_post_res_coeffs_pre_workspace_size(B8, 8, C8)
    assert S8 * B8 * 81 * 4 + B8 * 9 * S8 * 4 <= ws8 <= S8 * B8 * 81 * 4 + B8 * 9 * S8 * 4 + 2048
    tune.delenv("MHC_PASS8_PRE")
    # the two-call routes need what mhc_post_res_coeffs needs
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(8192, 8, 4096) == \
        mhc.mhc_post_res_coeffs_workspace_size(8192, 8, 4096)
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(8192, 8, 4224) == \
        mhc.mhc_post_res_coeffs_workspace_size(8192, 8, 4224)
    tune.setenv("MHC_FUSED_N8", "0")     # n = 8 as the apply and the split-K product
    tune.setenv("MHC_PASS8_PRE", 1)      # (no n = 8 pass to run in one pass)
    assert not one(8192, 8, 4096)
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(8192, 8, 4096) == \
        mhc.mhc_post_res_coeffs_workspace_size(8192, 8, 4096)
    tune.delenv("MHC_FUSED_N8")
    tune.delenv("MHC_PASS8_PRE")
    tune.setenv("MHC_FUSED_PRE", "0")
    assert not one(16384, 4, 7168) and not one(64, 4, 256)
    assert mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C) == mhc.mhc_post_res_coeffs_workspace_size(B, n, C)
    tune.delenv("MHC_FUSED_PRE")
    tune.setenv("MHC_SMALL_MAX_B", "0")  # no small-B routes: the persistent pass takes the small shape
    assert one(64, 4, 256)


def _fused_pre_fp8(B=16, n=4, C=64, ws_bytes=None, **over):
    names = ["X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "Fp", "ws"]
    p = dict(zip(names, _addrs(len(names))))
    p.update(over)
    if ws_bytes is None:
        ws_bytes = max(mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(B, n, C), 16)
    return mhc.mhc_post_res_coeffs_pre_fp8(B, n, C, p["X"], p["F"], p["H"], p["Y"], p["phi"], 0.01,
                                           0.01, 0.01, p["bp"], p["bq"], p["br"], p["logits"], p["r"],
                                           p["Hn"], p["Fp"], p["ws"], ws_bytes, stream=0, check=False)


def test_fused_pre_fp8_validation():
    """The E4M3 one-pass call: the bf16 call's rules with one-byte stream
    elements (overlaps in bytes)."""
    assert _fused_pre_fp8(B=0) == mhc.MHC_OK
    assert _fused_pre_fp8(B=0, X=None, Fp=None, ws=None) == mhc.MHC_OK
    assert _fused_pre_fp8(C=48) == mhc.MHC_ERR_UNSUPPORTED             # C % 16 == 0 but not % 32
    assert mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(16, 4, 48) == 0
    assert _fused_pre_fp8(n=3) == mhc.MHC_ERR_UNSUPPORTED
    assert _fused_pre_fp8(B=-2) == mhc.MHC_ERR_INVALID_ARG
    for k in ("X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "Fp", "ws"):
        assert _fused_pre_fp8(**{k: None}) == mhc.MHC_ERR_INVALID_ARG, k
    # F_pre (16 * 64 bytes) starting 16 bytes before the end of X_t's
    # 16 * 4 * 64 bytes overlaps it
    assert _fused_pre_fp8(Fp=A + 16 * 4 * 64 - 16) == mhc.MHC_ERR_INVALID_ARG
    assert _fused_pre_fp8(Fp=A + 3 * STEP + 16 * 4 * 64 - 16) == mhc.MHC_ERR_INVALID_ARG  # inside X_next
    assert _fused_pre_fp8(ws=A + 11 * STEP + 16 * 64 - 16) == mhc.MHC_ERR_INVALID_ARG     # overlaps F_pre
    assert _fused_pre_fp8(Fp=A + 11 * STEP + 8) == mhc.MHC_ERR_UNSUPPORTED                 # alignment
    need = mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(16, 4, 64)
    assert need > 0 and _fused_pre_fp8(ws_bytes=need - 1) == mhc.MHC_ERR_WORKSPACE


def test_fused_pre_fp8_route_and_workspace(tune):
    for k in ("MHC_FUSED_PRE", "MHC_SMALL_MAX_B", "MHC_FUSED_FP8", "MHC_FUSED_FIXED"):
        tune.delenv(k, raising=False)
    one = mhc.mhc_post_res_coeffs_pre_fp8_one_pass
    assert one(16384, 4, 7168) and one(4096, 4, 4096) and one(1000, 2, 4096) and one(300, 1, 1024)
    assert not one(64, 4, 7168)          # small B: the two calls
    assert not one(8192, 8, 4096)        # n = 8
    assert not one(4096, 4, 8704)        # 17 steps of 512 channels per row
    assert not one(0, 4, 7168) and not one(16, 4, 48)
    # one pass: the bf16 call's workspace (partials, packed phi, records)
    assert mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(16384, 4, 7168) == \
        mhc.mhc_post_res_coeffs_pre_workspace_size(16384, 4, 7168)
    # two calls: what mhc_post_res_coeffs_fp8 needs
    assert mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(8192, 8, 4096) == \
        mhc.mhc_post_res_coeffs_fp8_workspace_size(8192, 8, 4096)
    tune.setenv("MHC_FUSED_FP8", "0")       # E4M3 fused call as apply + product
    assert not one(16384, 4, 7168)
    assert mhc.mhc_post_res_coeffs_pre_fp8_workspace_size(16384, 4, 7168) == \
        mhc.mhc_post_res_coeffs_fp8_workspace_size(16384, 4, 7168)


def _coeffs_pre(B=16, n=4, C=64, ws_bytes=None, fp8=False, **over):
    names = ["X", "phi", "bp", "bq", "br", "logits", "r", "H", "Fp", "ws"]
    p = dict(zip(names, _addrs(len(names))))
    p.update(over)
    size = mhc.mhc_coeffs_pre_fp8_workspace_size if fp8 else mhc.mhc_coeffs_pre_workspace_size
    if ws_bytes is None:
        ws_bytes = max(size(B, n, C), 16)
    fn = mhc.mhc_coeffs_pre_fp8 if fp8 else mhc.mhc_coeffs_pre
    return fn(B, n, C, p["X"], p["phi"], 0.01, 0.01, 0.01, p["bp"], p["bq"], p["br"], p["logits"],
              p["r"], p["H"], p["Fp"], p["ws"], ws_bytes, stream=0, check=False)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_coeffs_pre_validation(fp8):
    eb = 1 if fp8 else 2
    size = mhc.mhc_coeffs_pre_fp8_workspace_size if fp8 else mhc.mhc_coeffs_pre_workspace_size
    assert _coeffs_pre(B=0, fp8=fp8) == mhc.MHC_OK
    assert _coeffs_pre(B=0, X=None, Fp=None, ws=None, fp8=fp8) == mhc.MHC_OK
    assert _coeffs_pre(n=3, fp8=fp8) == mhc.MHC_ERR_UNSUPPORTED
    assert _coeffs_pre(C=36, fp8=fp8) == mhc.MHC_ERR_UNSUPPORTED              # C % 8 != 0
    assert _coeffs_pre(B=-2, fp8=fp8) == mhc.MHC_ERR_INVALID_ARG
    for k in ("X", "phi", "bp", "bq", "br", "logits", "r", "H", "Fp", "ws"):
        assert _coeffs_pre(fp8=fp8, **{k: None}) == mhc.MHC_ERR_INVALID_ARG, k
    assert _coeffs_pre(Fp=A + 16 * 4 * 64 * eb - 16, fp8=fp8) == mhc.MHC_ERR_INVALID_ARG  # F_pre overlaps X_t
    assert _coeffs_pre(Fp=A + 7 * STEP, fp8=fp8) == mhc.MHC_ERR_INVALID_ARG   # F_pre overlaps H
    assert _coeffs_pre(ws=A + 8 * STEP + 16 * 64 * eb - 16, fp8=fp8) == mhc.MHC_ERR_INVALID_ARG  # ws overlaps F_pre
    assert _coeffs_pre(Fp=A + 8 * STEP + 8, fp8=fp8) == mhc.MHC_ERR_UNSUPPORTED  # F_pre needs 16-byte alignment
    need = size(16, 4, 64)
    assert need > 0 and _coeffs_pre(ws_bytes=need - 1, fp8=fp8) == mhc.MHC_ERR_WORKSPACE
    # C % 32 != 0 is accepted (the two calls): the bf16 call at C = 40, the
    # E4M3 call at C = 48; both sizes are mhc_coeffs's
    C2 = 48 if fp8 else 40
    coeffs_size = mhc.mhc_coeffs_fp8_workspace_size if fp8 else mhc.mhc_coeffs_workspace_size
    assert size(16, 4, C2) == coeffs_size(16, 4, C2) > 0


def test_coeffs_pre_route_and_workspace(tune):
    for k in ("MHC_FUSED_PRE", "MHC_SMALL_MAX_B", "MHC_FUSED_FP8"):
        tune.delenv(k, raising=False)
    for fp8, one, size, coeffs_size in (
            (False, mhc.mhc_coeffs_pre_one_pass, mhc.mhc_coeffs_pre_workspace_size, mhc.mhc_coeffs_workspace_size),
            (True, mhc.mhc_coeffs_pre_fp8_one_pass, mhc.mhc_coeffs_pre_fp8_workspace_size,
             mhc.mhc_coeffs_fp8_workspace_size)):
        assert one(16384, 4, 7168) and one(4096, 4, 4096) and one(1000, 2, 4096) and one(300, 1, 1024)
        assert not one(64, 4, 7168)          # small B: mhc_coeffs then mhc_pre
        # small B, one slice (n*C <= 1024, C % 8 == 0): the single-slice kernel in bf16 only
        for shape in ((64, 4, 256), (7, 4, 48), (256, 1, 1008)):
            assert bool(one(*shape)) == (not fp8)
            assert size(*shape) == coeffs_size(*shape)
        assert not one(64, 4, 264) and not one(64, 8, 64)
        assert not one(8192, 8, 4096)        # n = 8: two calls by default
        assert not one(8192, 8, 4224)        # n = 8 with 33 slices per row
        assert not one(4096, 4, 8704)        # 17 steps of 512 channels per row
        assert not one(4096, 4, 7184)        # C % 32 != 0
        assert not one(0, 4, 7168) and not one(16, 3, 64)
        # one pass: the pre-mix layout of mhc_post_res_coeffs_pre (it also
        # holds mhc_coeffs's workspace, for the two calls)
        B, n, C = 16384, 4, 7168
        assert size(B, n, C) == mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C)
        assert size(B, n, C) >= coeffs_size(B, n, C)
        assert size(8192, 8, 4224) == coeffs_size(8192, 8, 4224)
        assert size(8192, 8, 4096) == coeffs_size(8192, 8, 4096)
        tune.setenv("MHC_PASS8_PRE", 1)      # the n = 8 pass in one pass (bf16 only)
        assert bool(one(8192, 8, 4096)) == (not fp8)
        if not fp8:
            tune.setenv("MHC_FUSED_PRE", 1)
            assert size(8192, 8, 4096) == mhc.mhc_post_res_coeffs_pre_workspace_size(8192, 8, 4096)
            assert size(8192, 8, 4096) >= coeffs_size(8192, 8, 4096)
            tune.delenv("MHC_FUSED_PRE")
        tune.delenv("MHC_PASS8_PRE")
    tune.setenv("MHC_FUSED_PRE", "0")
    assert not mhc.mhc_coeffs_pre_one_pass(16384, 4, 7168)
    assert mhc.mhc_coeffs_pre_workspace_size(16384, 4, 7168) == mhc.mhc_coeffs_workspace_size(16384, 4, 7168)


def test_coeffs_pre_check_host():
    """mhc_coeffs_pre_check answers without a device where no one-pass kernel
    can have run, and rejects bad arguments."""
    assert mhc.mhc_coeffs_pre_check(64, 4, 7168, A, workspace_bytes=1 << 20, stream=0) == mhc.MHC_OK
    assert mhc.mhc_coeffs_pre_check(8192, 8, 4224, A, workspace_bytes=1 << 20, stream=0) == mhc.MHC_OK
    assert mhc.mhc_coeffs_pre_check(4096, 4, 7184, A, workspace_bytes=1 << 30, stream=0) == mhc.MHC_OK
    assert mhc.mhc_coeffs_pre_check(0, 4, 7168, None, stream=0) == mhc.MHC_OK
    assert mhc.mhc_coeffs_pre_check(16384, 3, 7168, A, stream=0) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_coeffs_pre_check(16384, 4, 7168, None, stream=0) == mhc.MHC_ERR_INVALID_ARG
    need = mhc.mhc_coeffs_pre_workspace_size(16384, 4, 7168)
    assert mhc.mhc_coeffs_pre_check(16384, 4, 7168, A, workspace_bytes=need - 1,
                                    stream=0) == mhc.MHC_ERR_WORKSPACE


def test_binding_raises_on_error_status():
    with pytest.raises(mhc.MhcError) as ei:
        mhc.mhc_pre(16, 3, 64, *_addrs(3), stream=0)
    assert ei.value.status == mhc.MHC_ERR_UNSUPPORTED


def test_fp8_validation():
    """The E4M3 calls: same rules as the bf16 ones, with one-byte elements
    (overlap checks in bytes) and C % 16 == 0."""
    X, H, F, Y = _addrs(4)
    assert mhc.mhc_pre_fp8(0, 4, 64, None, None, None, stream=0, check=False) == mhc.MHC_OK
    assert mhc.mhc_pre_fp8(16, 4, 24, X, H, F, stream=0, check=False) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_pre_fp8(16, 4, 64, X, H, None, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    # F_pre right after X_t's 16*4*64 bytes does not overlap; one byte earlier does
    assert mhc.mhc_pre_fp8(16, 4, 64, X, H, X + 16 * 4 * 64 - 16, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    assert mhc.mhc_post_res_fp8(16, 4, 40, X, F, H, Y, stream=0, check=False) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_post_res_fp8(16, 4, 64, X, F, H, X, stream=0, check=False) == mhc.MHC_ERR_INVALID_ARG
    assert mhc.mhc_post_res_fp8(16, 4, 64, X, F, H, Y + 8, stream=0, check=False) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_coeffs_fp8_workspace_size(16, 4, 24) == 0
    assert mhc.mhc_coeffs_fp8_workspace_size(16, 4, 64) > 0
    names = ["X", "phi", "bp", "bq", "br", "logits", "r", "H", "ws"]
    p = dict(zip(names, _addrs(len(names))))

    def coeffs(C=64, ws_bytes=None, **over):
        q = dict(p, **over)
        wb = ws_bytes if ws_bytes is not None else max(mhc.mhc_coeffs_fp8_workspace_size(16, 4, C), 16)
        return mhc.mhc_coeffs_fp8(16, 4, C, q["X"], q["phi"], 0.01, 0.01, 0.01, q["bp"], q["bq"],
                                  q["br"], q["logits"], q["r"], q["H"], q["ws"], wb, stream=0,
                                  check=False)

    assert coeffs(C=24) == mhc.MHC_ERR_UNSUPPORTED
    assert coeffs(X=None) == mhc.MHC_ERR_INVALID_ARG
    assert coeffs(H=A + 1024) == mhc.MHC_ERR_INVALID_ARG               # inside X's 4096 bytes
    assert coeffs(ws_bytes=mhc.mhc_coeffs_fp8_workspace_size(16, 4, 64) - 1) == mhc.MHC_ERR_WORKSPACE
    fnames = ["X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "ws"]
    f = dict(zip(fnames, _addrs(len(fnames))))

    def fused(C=64, ws_bytes=None, **over):
        q = dict(f, **over)
        wb = ws_bytes if ws_bytes is not None else max(mhc.mhc_post_res_coeffs_fp8_workspace_size(16, 4, C), 16)
        return mhc.mhc_post_res_coeffs_fp8(16, 4, C, q["X"], q["F"], q["H"], q["Y"], q["phi"], 0.01,
                                           0.01, 0.01, q["bp"], q["bq"], q["br"], q["logits"],
                                           q["r"], q["Hn"], q["ws"], wb, stream=0, check=False)

    assert fused(C=48) == mhc.MHC_ERR_UNSUPPORTED                      # C % 32 for the fused call
    assert mhc.mhc_post_res_coeffs_fp8_workspace_size(16, 4, 48) == 0
    assert fused(Y=A) == mhc.MHC_ERR_INVALID_ARG
    need = mhc.mhc_post_res_coeffs_fp8_workspace_size(16, 4, 64)
    assert need > 0 and fused(ws_bytes=need - 1) == mhc.MHC_ERR_WORKSPACE


def test_lazy_prenorm_validation():
    """mhc_lazy_prenorm_gemm: K and N multiples of 8, 16-byte aligned operands,
    C and rstd disjoint from the inputs and each other; M == 0 is a no-op."""
    Ap, Wp, Cp, Rp = _addrs(4)

    def call(M=32, N=64, K=64, a=Ap, w=Wp, c=Cp, r=Rp):
        return mhc.mhc_lazy_prenorm_gemm(M, N, K, a, w, c, r, stream=0, check=False)

    assert call(M=0) == mhc.MHC_OK
    assert call(M=0, a=None, w=None, c=None, r=None) == mhc.MHC_OK
    assert call(M=-1) == mhc.MHC_ERR_INVALID_ARG
    assert call(N=0) == mhc.MHC_ERR_INVALID_ARG
    assert call(K=0) == mhc.MHC_ERR_INVALID_ARG
    assert call(K=60) == mhc.MHC_ERR_UNSUPPORTED
    assert call(N=60) == mhc.MHC_ERR_UNSUPPORTED
    for k in ("a", "w", "c"):
        assert call(**{k: None}) == mhc.MHC_ERR_INVALID_ARG, k
    assert call(a=Ap + 8) == mhc.MHC_ERR_UNSUPPORTED
    assert call(c=Cp + 4) == mhc.MHC_ERR_UNSUPPORTED
    assert call(r=Rp + 2) == mhc.MHC_ERR_UNSUPPORTED
    # C right after A's 32*64*2 bytes is fine; one piece earlier overlaps
    assert call(c=Ap + 32 * 64 * 2 - 16) == mhc.MHC_ERR_INVALID_ARG
    assert call(c=Wp + 16) == mhc.MHC_ERR_INVALID_ARG
    assert call(r=Cp + 64) == mhc.MHC_ERR_INVALID_ARG                  # rstd inside C
    assert call(M=1 << 31) == mhc.MHC_ERR_UNSUPPORTED
    assert call(K=(1 << 22) + 8) == mhc.MHC_ERR_UNSUPPORTED


def test_phi32_validation():
    """The fp32-phi calls: the bf16 calls' rules, with phi 4 bytes per element
    (its overlap span is K*N*4 bytes)."""
    B, n, C = 16, 4, 64
    K, N = n * C, n * n + 2 * n
    names = ["X", "phi", "bp", "bq", "br", "logits", "r", "H", "ws"]
    p = dict(zip(names, _addrs(len(names))))

    def coeffs(ws_bytes=None, **over):
        q = dict(p, **over)
        wb = ws_bytes if ws_bytes is not None else max(mhc.mhc_coeffs_phi32_workspace_size(B, n, C), 16)
        return mhc.mhc_coeffs_phi32(B, n, C, q["X"], q["phi"], 0.01, 0.01, 0.01, q["bp"], q["bq"],
                                    q["br"], q["logits"], q["r"], q["H"], q["ws"], wb, stream=0,
                                    check=False)

    assert mhc.mhc_coeffs_phi32_workspace_size(B, n, C) > 0
    assert mhc.mhc_coeffs_phi32_workspace_size(B, 3, C) == 0
    assert mhc.mhc_coeffs_phi32(0, n, C, None, None, 0.01, 0.01, 0.01, None, None, None, None, None,
                                None, None, 0, stream=0, check=False) == mhc.MHC_OK
    assert coeffs(phi=None) == mhc.MHC_ERR_INVALID_ARG
    assert coeffs(phi=p["phi"] + 8) == mhc.MHC_ERR_UNSUPPORTED
    # logits placed after the bf16 size of phi but inside its fp32 size
    assert coeffs(logits=p["phi"] + K * N * 2) == mhc.MHC_ERR_INVALID_ARG
    need = mhc.mhc_coeffs_phi32_workspace_size(B, n, C)
    assert coeffs(ws_bytes=need - 1) == mhc.MHC_ERR_WORKSPACE
    fnames = ["X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "ws"]
    f = dict(zip(fnames, _addrs(len(fnames))))

    def fused(Cc=C, ws_bytes=None, **over):
        q = dict(f, **over)
        wb = ws_bytes if ws_bytes is not None else max(mhc.mhc_post_res_coeffs_phi32_workspace_size(B, n, Cc), 16)
        return mhc.mhc_post_res_coeffs_phi32(B, n, Cc, q["X"], q["F"], q["H"], q["Y"], q["phi"], 0.01,
                                             0.01, 0.01, q["bp"], q["bq"], q["br"], q["logits"],
                                             q["r"], q["Hn"], q["ws"], wb, stream=0, check=False)

    assert fused(Cc=48) == mhc.MHC_ERR_UNSUPPORTED                     # C % 32
    assert mhc.mhc_post_res_coeffs_phi32_workspace_size(B, n, 48) == 0
    assert fused(Y=A) == mhc.MHC_ERR_INVALID_ARG
    assert fused(logits=f["phi"] + K * N * 2) == mhc.MHC_ERR_INVALID_ARG
    need = mhc.mhc_post_res_coeffs_phi32_workspace_size(B, n, C)
    assert need > 0 and fused(ws_bytes=need - 1) == mhc.MHC_ERR_WORKSPACE


def test_tuning_keys_and_no_environment(tune, monkeypatch):
    """Routes change only through mhc_tuning_set: the environment variables
    that once selected them are ignored, and unknown keys are rejected."""
    one = mhc.mhc_post_res_coeffs_pre_one_pass
    ws = mhc.mhc_post_res_coeffs_pre_workspace_size
    base = (one(16384, 4, 7168), ws(16384, 4, 7168), mhc.mhc_coeffs_split_k(16384, 4, 7168),
            mhc.mhc_coeffs_workspace_size(64, 4, 7168))
    for k, v in (("MHC_FUSED_PRE", "0"), ("MHC_SMALL_MAX_B", "0"), ("MHC_SPLIT_K", "5"),
                 ("MHC_GEMM_ALGO", "0")):
        monkeypatch.setenv(k, v)
    assert (one(16384, 4, 7168), ws(16384, 4, 7168), mhc.mhc_coeffs_split_k(16384, 4, 7168),
            mhc.mhc_coeffs_workspace_size(64, 4, 7168)) == base
    # the n = 8 pass's product (MHC_GEMM_ALGO=3): one slice per 128 channels
    tune.setenv("MHC_GEMM_ALGO", 3)
    assert mhc.mhc_coeffs_split_k(8192, 8, 4096) == 32
    # the split-K product's slice count (the default product at n = 8)
    tune.setenv("MHC_GEMM_ALGO", 1)
    s8 = mhc.mhc_coeffs_split_k(8192, 8, 4096)
    tune.setenv("MHC_SPLIT_K", 5)
    assert mhc.mhc_coeffs_split_k(8192, 8, 4096) == 5
    tune.delenv("MHC_GEMM_ALGO")
    assert mhc.mhc_coeffs_split_k(16384, 4, 7168) == base[2]   # the persistent product: one slice per 512 channels
    assert mhc.mhc_coeffs_split_k(8192, 8, 4096) == 5          # the default at n = 8: the split-K product
    tune.setenv("MHC_GEMM_ALGO", 1)
    tune.delenv("MHC_SPLIT_K")
    assert mhc.mhc_coeffs_split_k(8192, 8, 4096) == s8
    assert base[2] == 14
    tune.setenv("MHC_FUSED_PRE", 0)
    assert not one(16384, 4, 7168)
    mhc.mhc_tuning_reset()
    assert one(16384, 4, 7168)
    with pytest.raises(mhc.MhcError) as ei:
        mhc.mhc_tuning_set("MHC_NO_SUCH_KEY", 1)
    assert ei.value.status == mhc.MHC_ERR_INVALID_ARG


def test_every_documented_tuning_key(tune):
    """Each key the header documents is accepted, and the split-K shape keys
    reach the plan: at n = 8 (C = 4096, B = 8192) four waves of one 16-row
    block make 64-row tiles and two K-slices; eight waves, or X through
    registers, make 128-row tiles and four."""
    hdr = open(os.path.join(ROOT, "include", "mhc.h")).read()
    doc = hdr[hdr.index("Testing and tuning."):]
    keys = sorted(set(re.findall(r"\bMHC_[A-Z0-9_]+\b", doc)) - {"MHC_H", "MHC_ERR_INVALID_ARG"})
    assert {"MHC_GEMM_WAVES", "MHC_GEMM_XREG", "MHC_GEMM_KC", "MHC_LPN_ALGO"} <= set(keys)
    for k in keys:
        mhc.mhc_tuning_set(k, -1)
    split = mhc.mhc_coeffs_split_k
    assert split(8192, 8, 4096) == 2      # the split-K product
    tune.setenv("MHC_GEMM_ALGO", 3)       # the n = 8 pass's product
    assert split(8192, 8, 4096) == 32
    tune.setenv("MHC_GEMM_ALGO", 1)       # the split-K product, forced
    assert split(8192, 8, 4096) == 2
    tune.setenv("MHC_GEMM_WAVES", 8)
    assert split(8192, 8, 4096) == 4
    tune.delenv("MHC_GEMM_WAVES")
    tune.setenv("MHC_GEMM_XREG", 2)
    assert split(8192, 8, 4096) == 4
    tune.delenv("MHC_GEMM_XREG")
    assert split(8192, 8, 4096) == 2


def test_binding_checks_tensor_sizes():
    """The binding rejects a tensor of the wrong element size, or smaller
    than the bytes the call touches, before anything reaches the library
    (host tensors suffice: the size check comes before the device check;
    the other arguments are raw addresses, which are passed through)."""
    B, n, C = 16, 4, 64
    X, H, F, Y, W = _addrs(5)
    with pytest.raises(ValueError, match="F_pre: 1792 bytes, the call needs 2048"):
        mhc.mhc_pre(B, n, C, X, H, torch.empty(B, C - 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="X_t: element size 4"):  # fp32 values to a bf16 call
        mhc.mhc_pre(B, n, C, torch.empty(B, n * C, dtype=torch.float32), H, F)
    with pytest.raises(ValueError, match="X_t: 4096 bytes, the call needs 8192"):  # raw bytes: size only
        mhc.mhc_pre(B, n, C, torch.empty(B, n * C, dtype=torch.uint8), H, F)
    with pytest.raises(ValueError, match="X_t: element size 2"):  # a bf16 tensor to an E4M3 call
        mhc.mhc_pre_fp8(B, n, C, torch.empty(B, n * C, dtype=torch.bfloat16), H, F)
    with pytest.raises(ValueError, match="H: "):
        mhc.mhc_post_res(B, n, C, X, F, torch.empty(B - 1, n * n + 2 * n), Y)
    with pytest.raises(ValueError, match="phi: element size 4"):  # fp32 phi to the bf16-phi call
        mhc.mhc_coeffs(B, n, C, X, torch.empty(n * C, 24), 0.01, 0.01, 0.01, *_addrs(6), W,
                       workspace_bytes=1 << 20)
    with pytest.raises(ValueError, match="workspace"):
        mhc.mhc_coeffs(B, n, C, X, H, 0.01, 0.01, 0.01, *_addrs(6), torch.empty(64, dtype=torch.uint8),
                       workspace_bytes=128)
    with pytest.raises(ValueError, match="device tensors"):  # right sizes: then the host-tensor check
        mhc.mhc_pre(B, n, C, X, H, torch.empty(B, C, dtype=torch.bfloat16))


def test_one_pass_grid_and_check():
    """The one-pass grid arithmetic (whole row tiles per round within what is
    resident) is exercised through the route, and the give-up check answers
    without a device where no one-pass kernel can have run."""
    # the shapes that run two calls never give up: no device access needed
    assert mhc.mhc_post_res_coeffs_pre_check(64, 4, 7168, A, workspace_bytes=1 << 20, stream=0) == mhc.MHC_OK
    assert mhc.mhc_post_res_coeffs_pre_check(8192, 8, 4224, A, workspace_bytes=1 << 20, stream=0) == mhc.MHC_OK
    assert mhc.mhc_post_res_coeffs_pre_check(0, 4, 7168, None, stream=0) == mhc.MHC_OK
    # argument errors
    assert mhc.mhc_post_res_coeffs_pre_check(16384, 3, 7168, A, stream=0) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.mhc_post_res_coeffs_pre_check(16384, 4, 7168, None, fp8=True, stream=0) == mhc.MHC_ERR_INVALID_ARG
    # NULL workspace: the no-alloc call's array, which holds at most MHC_NOALLOC_SCRATCH_BYTES
    assert mhc.mhc_post_res_coeffs_pre_check(65536, 4, 7168, None, stream=0) == mhc.MHC_ERR_WORKSPACE
    need = mhc.mhc_post_res_coeffs_pre_workspace_size(16384, 4, 7168)
    assert mhc.mhc_post_res_coeffs_pre_check(16384, 4, 7168, A, workspace_bytes=need - 1,
                                             stream=0) == mhc.MHC_ERR_WORKSPACE
    # the one-pass workspace holds partials, packed phi, records and the give-up word
    assert need % 16 == 0


def _no_device():
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_device(), reason="needs a host without a HIP device (calls use fake addresses)")
def test_no_device_is_mhc_err_hip():
    """Calls that pass validation but cannot launch (no HIP device) report
    MHC_ERR_HIP; nothing aborts."""
    X, H, F, Y = _addrs(4)
    assert mhc.mhc_pre(16, 4, 64, X, H, F, stream=0, check=False) == mhc.MHC_ERR_HIP
    assert mhc.mhc_post_res(16, 4, 64, X, F, H, Y, stream=0, check=False) == mhc.MHC_ERR_HIP
    assert _fused_pre(B=16384, n=4, C=7168, **dict(zip(
        ["X", "F", "H", "Y", "phi", "bp", "bq", "br", "logits", "r", "Hn", "Fp", "ws"],
        [A + k * (1 << 36) for k in range(13)]))) == mhc.MHC_ERR_HIP
    need = mhc.mhc_post_res_coeffs_pre_workspace_size(16384, 4, 7168)
    assert mhc.mhc_post_res_coeffs_pre_check(16384, 4, 7168, A, workspace_bytes=need,
                                             stream=0) == mhc.MHC_ERR_HIP
    assert _coeffs_pre(B=16384, n=4, C=7168, **dict(zip(
        ["X", "phi", "bp", "bq", "br", "logits", "r", "H", "Fp", "ws"],
        [A + k * (1 << 36) for k in range(10)]))) == mhc.MHC_ERR_HIP
    assert mhc.mhc_coeffs_pre_check(16384, 4, 7168, A, workspace_bytes=need, stream=0) == mhc.MHC_ERR_HIP
