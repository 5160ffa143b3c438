"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's sources with both sanitizers on the host code (the
device code is built as usual, without them), links them with the native
driver tests/host/abi_host_check.cpp, and runs it: every validation branch,
extreme sizes, the tuning keys, the one-pass grid arithmetic and, on a host
without a HIP device, calls that must report MHC_ERR_HIP.  Any sanitizer
report aborts the driver and fails the test."""

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest
import torch

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "manifold_constrained_hyper_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitized")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"

# Sanitizers on the host code only: each -fsanitize= follows -Xarch_host.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src, lang_hip=True):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SAN, *([] if lang_hip else ["-x", "hip"]), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return obj


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANG), reason="needs hipcc and clang++")
def test_abi_layer_under_asan_ubsan():
    shutil.rmtree(OUT, ignore_errors=True)
    os.makedirs(OUT)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs))
    objs.append(_compile(os.path.join(ROOT, "tests", "host", "abi_host_check.cpp"), lang_hip=False))
    exe = os.path.join(OUT, "abi_host_check")
    link = [CLANG, "-fsanitize=address,undefined", "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(link)}\n{r.stdout}\n{r.stderr}"
    # Calls that pass validation would launch on fake addresses: those run
    # only where no HIP device is visible.
    no_device = torch.cuda.device_count() == 0
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "1" if no_device else "0"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, f"driver failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
