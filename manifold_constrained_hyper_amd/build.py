"""Build libmhc.so for gfx950 in-tree with hipcc.

    python -m manifold_constrained_hyper_amd.build

Compiles every HIP source under csrc/ into manifold_constrained_hyper_amd/
libmhc.so, and the benchmark's bandwidth probes (probe/bw_probe.hip, not part
of the library) into probe/libmhc_probe.so.  Packed-fp32 instructions are
disabled for all device code.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmhc.so")
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMPILE_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


PROBE_SRC = os.path.join(PKG, "probe", "bw_probe.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libmhc_probe.so")


def build_probe(verbose=True):
    """The benchmark's bandwidth-probe library (not part of libmhc)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *COMPILE_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


def build(verbose=True):
    """Compile all sources and link libmhc.so (always rebuilds), then the
    benchmark's probe library."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
