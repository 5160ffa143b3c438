"""Host logic of the benchmark: byte and flop accounting, pinned to the
figures printed in the mHC CuTile page (section 4 performance printout; see
tests/golden/page_bench_figures.json), and the one-GPU guard."""

import json
import os
import subprocess
import sys

import pytest

import bench

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "page_bench_figures.json")))


def _fig(name):
    return next(f for f in GOLDEN["figures"] if f["kernel"] == name)


def test_apply_bytes_convention_matches_page():
    g = GOLDEN
    f = _fig("mhc_apply_residual")
    rate = bench.apply_stream_bytes(g["M"], g["n"], g["C"], g["elem_bytes"]) / (f["ms"] * 1e-3) / 1e9
    # the page prints ms to 4 digits: allow that rounding (0.02 %) and a little more
    assert abs(rate - f["rate"]) / f["rate"] < 1e-3


def test_product_flop_convention_matches_page():
    g = GOLDEN
    f = _fig("mhc_gemm_rmsnorm")
    rate = bench.product_flops(g["M"], g["n"], g["C"]) / (f["ms"] * 1e-3) / 1e12
    assert abs(rate - f["rate"]) / f["rate"] < 1e-3


def test_scale_sigmoid_bytes_convention_matches_page():
    g = GOLDEN
    f = _fig("mhc_scale_bias_sigmoid")
    N = g["n"] * g["n"] + 2 * g["n"]
    nbytes = 2 * g["M"] * N * g["elem_bytes"] + g["M"] * 4
    rate = nbytes / (f["ms"] * 1e-3) / 1e9
    assert abs(rate - f["rate"]) / f["rate"] < 2e-3   # ms printed to 2 significant digits


def test_path_bytes_large_workload():
    b = bench.path_bytes(16384, 4, 7168)
    assert (b["mhc_coeffs"], b["mhc_pre"], b["mhc_post_res"]) == (944111712, 1174667264, 2115239936)
    assert b["mhc_coeffs"] + b["mhc_pre"] + b["mhc_post_res"] == 4234018912
    # the fused call moves the apply's bytes plus the next layer's coefficient
    # inputs/outputs, but not X_next a second time
    assert b["mhc_post_res_coeffs"] == b["mhc_post_res"] + (b["mhc_coeffs"] - 16384 * 4 * 7168 * 2)
    assert b["mhc_pre"] + b["mhc_post_res_coeffs"] == 3294494816
    # the one-pass call adds only the next layer's F_pre write: X read once, written once
    assert b["mhc_post_res_coeffs_pre"] == b["mhc_post_res_coeffs"] + 16384 * 7168 * 2
    assert b["mhc_post_res_coeffs_pre"] == 2354708576
    # post_res = page's apply convention at bf16 + the fp32 coefficients it reads
    assert b["mhc_post_res"] == bench.apply_stream_bytes(16384, 4, 7168, 2) + 16384 * 20 * 4


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
