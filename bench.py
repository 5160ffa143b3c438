"""Benchmark of the mHC residual-stream forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload large]     (defaults K=100, W=50)

One step = one mHC layer over one batch of synthetic input already resident
in HBM, run as a model runs it: `mhc_coeffs` and `mhc_pre` once before the
loop, then per layer one `mhc_post_res_coeffs_pre` (step 4b of this layer,
then steps 1-3 and 4a of the next, in one pass: the residual stream is read
once and written once per layer).  The residual stream is chained through the
layers (X_{t+1} of one step is X_t of the next); every layer uses the same
synthetic phi and biases, and the layer F between two calls is not mHC
(F_out is a fixed synthetic input).  Also timed: the two-call pipeline
(`mhc_pre` + `mhc_post_res_coeffs` per layer, "two_call_pipeline") and the
three separate calls (`mhc_coeffs`, `mhc_pre`, `mhc_post_res` on a fixed
X_t, "three_call").

Prints ONE JSON line with tokens/s, achieved HBM bandwidth against the
algorithmic byte count, per-call times, the roofline of the dominant call and
the fp64 oracle's throughput on the host as a CPU baseline.

Algorithmic bytes (bf16 X_t, F_out, F_pre, X_next; fp32 coefficients):
  mhc_coeffs               X_t + phi + biases + logits + r + H
  mhc_pre                  X_t + H_pre + F_pre
  mhc_post_res             2 X_t + F_out + (H_post, H_res)
  mhc_post_res_coeffs      mhc_post_res + phi_next + biases + logits + r + H (next layer)
  mhc_post_res_coeffs_pre  mhc_post_res_coeffs + F_pre (next layer)
Split-K partials, the hand-off records of the one-pass call and the packed
copy of phi are implementation traffic and are not counted.

Also reported: the same pipelines on the E4M3 residual stream ("fp8", the
*_fp8 entry points, one byte per stream element in the byte count) and, for
the other workloads (tiny, decode, prefill, wide), both dtypes' one-pass,
two-call and three-call times ("workloads"; decode also cold: the one-pass
call after a 512 MB write; tiny, decode and prefill also with 16 chained
one-pass layers captured in a HIP graph and replayed, "graph_*").

Also reported ("phi32_coeffs"): mhc_coeffs_phi32 (fp32 phi) beside mhc_coeffs
on the same X, decode and headline workloads, mean call time.

Also reported ("lazy_prenorm"): the Lazy Pre-Norm GEMM C = rmsnorm(A) W^T
(mhc_lazy_prenorm_gemm) on its three synthetic workloads, with TFLOP/s
(2 M N K per call; the sums of squares are not counted) against MI355X's
dense bf16 MFMA peak.

Order of the run: the CPU baseline, the three separate calls, the two-call
pipeline, then the headline loop (so the GPU runs at its working clocks when
the timed region starts), then each headline call again between its own
events (per-call mean, median, p10 and p90), the bandwidth probes, and the
other sections.  The headline loop takes exactly W warm-up and K timed
steps; the three-call, two-call and E4M3 loops take at least 40 and 50.  "practical_ceiling" holds the rates of plain HIP read, write
and copy kernels (probe/bw_probe.hip) on 1 GiB buffers, and
frac_of_practical_copy_ceiling relates a leg's bandwidth to the copy rate
(the one-pass call reads and writes about equal bytes).

Other modes:
  --copy-probe   time the probe's copy kernel on 1 GiB (the reference against
                 which rocprofv3 FETCH_SIZE / WRITE_SIZE are scaled);
  --bw-probe     print only the read / write / copy probe rates;
  --three-call-only  run only the three calls' loop (counter runs of their kernels);
  --kernel-only  run only the timed headline loop (for rocprofv3 runs);
  --two-call-only  run only the two-call pipeline's loop (mhc_pre +
                 mhc_post_res_coeffs; for rocprofv3 counter runs of their kernels);
  --lazy-prenorm-only  time only the Lazy Pre-Norm GEMM workloads;
  --lpn-counters  a few launches of each Lazy Pre-Norm kernel layout and of
                 torch's A @ W^T on the square workload (counter runs);
  --shape-sweep  time the one-pass layer call (bf16 and E4M3) over a grid of
                 shapes around the headline one, one JSON line per shape
                 (steady state: ~60 ms of chained layers before ~60 ms timed).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mHC fwd tokens/sec + achieved HBM GB/s (% of peak), n=4 C=7168 B=16384"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
DEFAULT_WORKLOAD = "large"


def apply_stream_bytes(B, n, C, elem_bytes):
    """Residual-stream bytes of the fused post/res apply: X_t read, F_out read,
    X_next written (the convention of the apply figures printed in the mHC
    CuTile page, section 4), without the coefficients."""
    return B * (2 * n * C + C) * elem_bytes


def product_flops(B, n, C):
    """Flops of the fused product + sum of squares, 2 B K (N + 1) (the
    convention of the page's gemm_rmsnorm TFLOPS figure)."""
    N = n * n + 2 * n
    return 2 * B * n * C * (N + 1)


def path_bytes(B, n, C, eb=2):
    """Algorithmic bytes moved by each call for one layer: residual-stream
    tensors (X_t, F_out, F_pre, X_next) of eb bytes per element (2 for bf16, 1
    for the E4M3 calls), bf16 phi, fp32 coefficients and biases."""
    N = n * n + 2 * n
    K = n * C
    x = B * K * eb
    coeff_out = N * 4 + B * N * 4 + B * 4 + B * N * 4   # biases in, logits, H, r out
    post_res = apply_stream_bytes(B, n, C, eb) + B * (n + n * n) * 4
    return {
        "mhc_coeffs": x + K * N * 2 + coeff_out,
        "mhc_pre": x + B * n * 4 + B * C * eb,
        "mhc_post_res": post_res,
        "mhc_post_res_coeffs": post_res + K * N * 2 + coeff_out,
        "mhc_post_res_coeffs_pre": post_res + K * N * 2 + coeff_out + B * C * eb,
        "mhc_coeffs_pre": x + K * N * 2 + coeff_out + B * C * eb,
    }


def path_flops(B, n, C):
    """Algorithmic flops of one forward (product, sum of squares, pre, post/res)."""
    return product_flops(B, n, C) + B * (2 * n * C + 2 * (n * n + n) * C)


# Legs other than the headline (the three-call and two-call pipelines, the
# E4M3 pipelines) take at least this many warm-up and timed steps: the first
# 20-40 back-to-back layers run slower while clocks and caches settle, and
# these legs are reported as steady-state figures.
SECONDARY_WARMUP = 40
SECONDARY_STEPS = 50

# kernels launched by each call (for the roofline record)
KERNELS_OF_CALL = {"mhc_post_res": "post_res_kernel", "mhc_pre": "pre_kernel",
                   "mhc_coeffs": "post_res_next_kernel<n, 3> (product only, fixed-slice layout) + "
                                 "coeff_sinkhorn_kernel",
                   "mhc_post_res_coeffs": "pack_phi_kernel + post_res_next_kernel + coeff_sinkhorn_kernel",
                   "mhc_post_res_coeffs_pre": "zero_kernel (records) + post_res_next_kernel<n, 4> (pre-mix "
                                              "mode) + coeff_sinkhorn_kernel (tree order)",
                   "mhc_coeffs_pre": "zero_kernel (records) + post_res_next_kernel<n, 6> (product-only "
                                     "pre-mix mode) + coeff_sinkhorn_kernel (tree order)"}


class Pipeline:
    """The per-layer pipelines for one input set (X chained through the
    layers): `layer` = mhc_pre + mhc_post_res_coeffs, `onepass` =
    mhc_post_res_coeffs_pre; and `three` = the three separate calls on a
    fixed X_t; in bf16 or E4M3 (fp8=True: the *_fp8 entry points)."""

    def __init__(self, mhc, torch, inp, fp8=False):
        self.torch, self.inp = torch, inp
        B, n, C = inp["B"], inp["n"], inp["C"]
        self.B, self.n, self.C = B, n, C
        N = n * n + 2 * n
        sfx = "_fp8" if fp8 else ""
        self.coeffs = getattr(mhc, "mhc_coeffs" + sfx)
        self.pre = getattr(mhc, "mhc_pre" + sfx)
        self.post_res = getattr(mhc, "mhc_post_res" + sfx)
        self.fused = getattr(mhc, "mhc_post_res_coeffs" + sfx)
        ws_c = getattr(mhc, "mhc_coeffs" + sfx + "_workspace_size")(B, n, C)
        ws_f = getattr(mhc, "mhc_post_res_coeffs" + sfx + "_workspace_size")(B, n, C)
        self.fused_pre = getattr(mhc, "mhc_post_res_coeffs_pre" + sfx)
        ws_f = max(ws_f, getattr(mhc, "mhc_post_res_coeffs_pre" + sfx + "_workspace_size")(B, n, C))
        self.coeffs_pre = getattr(mhc, "mhc_coeffs_pre" + sfx)
        ws_c = max(ws_c, getattr(mhc, "mhc_coeffs_pre" + sfx + "_workspace_size")(B, n, C))
        dev, st = "cuda", torch.uint8 if fp8 else torch.bfloat16
        self.X = [inp["X"], torch.empty_like(inp["X"])]
        self.H = [torch.empty(B, N, device=dev) for _ in range(2)]
        self.logits = torch.empty(B, N, device=dev)
        self.r = torch.empty(B, device=dev)
        self.F_pre = torch.empty(B, C, dtype=st, device=dev)
        self.X_out = torch.empty_like(inp["X"])
        self.ws_c = torch.empty(max(ws_c, 16), dtype=torch.uint8, device=dev)
        self.ws_f = torch.empty(max(ws_f, 16), dtype=torch.uint8, device=dev)
        self.ab = (inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"], inp["b_pre"],
                   inp["b_post"], inp["b_res"])
        self.stream = torch.cuda.current_stream()
        self.coeffs(B, n, C, self.X[0], inp["phi"], *self.ab, self.logits, self.r, self.H[0],
                    self.ws_c, stream=self.stream)
        self.cur = 0

    def layer(self, marks=None):
        B, n, C, a, s = self.B, self.n, self.C, self.cur, self.stream
        if marks is not None:
            marks[0].record(s)
        self.pre(B, n, C, self.X[a], self.H[a], self.F_pre, stream=s)
        if marks is not None:
            marks[1].record(s)
        self.fused(B, n, C, self.X[a], self.inp["F_out"], self.H[a], self.X[1 - a], self.inp["phi"],
                   *self.ab, self.logits, self.r, self.H[1 - a], self.ws_f, stream=s)
        if marks is not None:
            marks[2].record(s)
        self.cur = 1 - a

    def onepass(self, marks=None):
        B, n, C, a, s = self.B, self.n, self.C, self.cur, self.stream
        if marks is not None:
            marks[0].record(s)
        self.fused_pre(B, n, C, self.X[a], self.inp["F_out"], self.H[a], self.X[1 - a], self.inp["phi"],
                       *self.ab, self.logits, self.r, self.H[1 - a], self.F_pre, self.ws_f, stream=s)
        if marks is not None:
            marks[1].record(s)
        self.cur = 1 - a

    def first(self, marks=None):
        """The first layer's call (mhc_coeffs_pre) on the fixed X_t."""
        B, n, C, s, inp = self.B, self.n, self.C, self.stream, self.inp
        if marks is not None:
            marks[0].record(s)
        self.coeffs_pre(B, n, C, inp["X"], inp["phi"], *self.ab, self.logits, self.r, self.H[0],
                        self.F_pre, self.ws_c, stream=s)
        if marks is not None:
            marks[1].record(s)

    def three(self, marks=None):
        B, n, C, s, inp = self.B, self.n, self.C, self.stream, self.inp
        if marks is not None:
            marks[0].record(s)
        self.coeffs(B, n, C, inp["X"], inp["phi"], *self.ab, self.logits, self.r, self.H[0],
                    self.ws_c, stream=s)
        if marks is not None:
            marks[1].record(s)
        self.pre(B, n, C, inp["X"], self.H[0], self.F_pre, stream=s)
        if marks is not None:
            marks[2].record(s)
        self.post_res(B, n, C, inp["X"], inp["F_out"], self.H[0], self.X_out, stream=s)
        if marks is not None:
            marks[3].record(s)

    def time_loop(self, fn, steps, warmup):
        """Mean ms per call of fn over `steps` back-to-back calls between two
        events (no event between calls)."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(self.stream)
        for _ in range(steps):
            fn()
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def time_graph(self, fn, layers=16, reps=20):
        """Mean ms per layer when `layers` chained calls of fn, captured once
        in a HIP graph, are replayed `reps` times back to back (launch
        overhead removed, as a serving loop would run them)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        old = self.stream
        with torch.cuda.stream(side):
            self.stream = side
            for _ in range(layers):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.stream = torch.cuda.current_stream()
            for _ in range(layers):
                fn()
        self.stream = old
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(cur)
        for _ in range(reps):
            g.replay()
        t1.record(cur)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / (reps * layers)

    def per_call(self, fn, names, steps):
        """Mean ms of each call, from events around every call."""
        return {c: sum(v) / len(v) for c, v in self.per_call_all(fn, names, steps).items()}

    def per_call_all(self, fn, names, steps):
        """Every call's ms, from events around every call."""
        torch = self.torch
        marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            fn(marks[k])
        torch.cuda.synchronize()
        return {c: [marks[k][i].elapsed_time(marks[k][i + 1]) for k in range(steps)]
                for i, c in enumerate(names)}

    def flushed(self, fn, reps=20, flush_bytes=512 << 20):
        """Per-call ms of fn with a 512 MB write between calls (outside the
        events), so that no input is left in the MALL or the L2s."""
        torch = self.torch
        scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
        out = []
        for _ in range(reps):
            scratch.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        del scratch
        return out


def _summary(B, n, C, eb, ms_layer, ms_three, per_pipe=None, per_three=None, ms_onepass=None,
             ms_first=None):
    b = path_bytes(B, n, C, eb)
    pipe = b["mhc_pre"] + b["mhc_post_res_coeffs"]
    three = b["mhc_coeffs"] + b["mhc_pre"] + b["mhc_post_res"]
    out = {}
    if ms_first is not None:
        first = b["mhc_coeffs_pre"]
        out.update({"first_layer_us": round(ms_first * 1e3, 2),
                    "first_layer_hbm_gbps": round(first / (ms_first * 1e-3) / 1e9, 1),
                    "first_layer_algorithmic_bytes": first})
    if ms_onepass is not None:
        one = b["mhc_post_res_coeffs_pre"]
        out.update({"onepass_us_per_layer": round(ms_onepass * 1e3, 2),
                    "onepass_tokens_per_s": round(B / (ms_onepass * 1e-3), 1),
                    "onepass_hbm_gbps": round(one / (ms_onepass * 1e-3) / 1e9, 1),
                    "onepass_algorithmic_bytes_per_layer": one})
    out.update({"us_per_layer": round(ms_layer * 1e3, 2), "tokens_per_s": round(B / (ms_layer * 1e-3), 1),
                "hbm_gbps": round(pipe / (ms_layer * 1e-3) / 1e9, 1), "algorithmic_bytes_per_layer": pipe,
                "three_call_us": round(ms_three * 1e3, 2),
                "three_call_hbm_gbps": round(three / (ms_three * 1e-3) / 1e9, 1)})
    if per_pipe:
        out["per_call_us"] = {c: round(v * 1e3, 2) for c, v in per_pipe.items()}
    if per_three:
        out["three_call_per_call_us"] = {c: round(v * 1e3, 2) for c, v in per_three.items()}
    return out


# source files that make up each call's kernels (for the counter-freshness check)
# Sources of the kernels each call runs on the large workload (n=4, C=7168,
# B=16384, bf16): a recorded counter summary is used only while these match.
CALL_SOURCES = {
    "mhc_coeffs": ("mhc_post_res_fused.hip", "mhc_coeff_sinkhorn.hip", "mhc_finish.h", "mhc_device.h"),
    "mhc_pre": ("mhc_stream.hip", "mhc_device.h"),
    "mhc_post_res": ("mhc_stream.hip", "mhc_device.h"),
    "mhc_post_res_coeffs": ("mhc_pack.hip", "mhc_post_res_fused.hip", "mhc_coeff_sinkhorn.hip",
                            "mhc_finish.h", "mhc_device.h"),
    "mhc_post_res_coeffs_pre": ("mhc_pack.hip", "mhc_post_res_fused.hip", "mhc_coeff_sinkhorn.hip",
                                "mhc_finish.h", "mhc_device.h"),
    "mhc_coeffs_pre": ("mhc_pack.hip", "mhc_post_res_fused.hip", "mhc_coeff_sinkhorn.hip",
                       "mhc_finish.h", "mhc_device.h"),
    "mhc_lazy_prenorm_gemm": ("mhc_lazy_prenorm.hip", "mhc_device.h"),
    "mhc_coeffs_phi32": ("mhc_pack.hip", "mhc_gemm_lds.hip", "mhc_coeff_sinkhorn.hip", "mhc_finish.h",
                         "mhc_device.h"),
}


def kernel_source_sha(call):
    """Short hash of the sources of one call's kernels."""
    csrc = os.path.join(ROOT, "manifold_constrained_hyper_amd", "csrc")
    h = hashlib.sha256()
    for f in CALL_SOURCES[call]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _recorded_traffic(call, workload):
    """HBM bytes per launch measured by rocprofv3 counters, from the committed
    summary in profiles/, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{call}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_source_sha(call):
        return None
    return float(val.group(1))


def _cpu_baseline(inp, rows_wanted, budget_s):
    """Time the fp64 oracle (as it stands) on the first rows of the workload."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas_threads = 1
    n, C = inp["n"], inp["C"]
    rows = min(rows_wanted, inp["B"])
    # exact widening bf16 -> fp32 on the device side copy; the oracle widens to fp64
    x = inp["X"][:rows].float().cpu().numpy()
    f = inp["F_out"][:rows].float().cpu().numpy()
    phi = inp["phi"].float().cpu().numpy()
    bp, bq, br = (inp[k].double().cpu().numpy() for k in ("b_pre", "b_post", "b_res"))
    done = 0
    t0 = time.perf_counter()
    while done < rows:
        step = min(256, rows - done)
        oracle.forward(x[done:done + step], phi, inp["alpha_pre"], inp["alpha_post"],
                       inp["alpha_res"], bp, bq, br, f[done:done + step], n, C)
        done += step
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": done / dt, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"first {done} of {inp['B']} rows of the same workload, fp64 numpy oracle, "
                      f"{dt:.1f} s wall; BLAS threads={blas_threads} (elementwise numpy is "
                      f"single-threaded); host cores visible={len(os.sched_getaffinity(0))}; "
                      f"cpu={cpu_model}"}


def _stats(ms):
    """Median and 10th / 90th percentiles (microseconds) of per-call times in ms."""
    v = sorted(ms)
    q = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]  # noqa: E731
    return {"median_us": round(q(0.5) * 1e3, 2), "p10_us": round(q(0.1) * 1e3, 2),
            "p90_us": round(q(0.9) * 1e3, 2), "n": len(v)}


def bandwidth_probe(torch, steps=20, warmup=5, nbytes=1 << 30):
    """Practical HBM ceilings on this device: plain HIP streaming kernels
    (manifold_constrained_hyper_amd/probe/bw_probe.hip, 16-byte non-temporal
    accesses, 8 workgroups per CU) that read, write or copy a 1 GiB buffer,
    far larger than the 256 MB MALL.  Mean GB/s over back-to-back launches
    between two events; a copy counts its reads and its writes."""
    import ctypes
    path = os.path.join(ROOT, "manifold_constrained_hyper_amd", "probe", "libmhc_probe.so")
    lib = ctypes.CDLL(path)
    lib.mhc_probe_bandwidth.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.mhc_probe_bandwidth.restype = ctypes.c_int
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    out, by_variant = {}, {}
    for name, mode, moved in (("copy", 2, 2 * nbytes), ("write", 1, nbytes), ("read", 0, nbytes)):
        for variant, vname in ((0, "grid_stride"), (1, "tiled_nt"), (2, "tiled_plain")):
            if mode == 0 and variant == 2:
                continue  # reads have no store policy

            def fn():
                st = lib.mhc_probe_bandwidth(mode | (variant << 4), src.data_ptr(), dst.data_ptr(), nbytes,
                                             sink.data_ptr(), stream.cuda_stream)
                if st != 0:
                    raise RuntimeError(f"bandwidth probe {name}/{vname}: hipError {st}")
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            by_variant[f"{name}_{vname}"] = round(moved / (ms * 1e-3) / 1e9, 1)
        # the practical ceiling of an access mix: the fastest variant
        out[f"{name}_gbps"] = max(v for k, v in by_variant.items() if k.startswith(name + "_"))
    out["variants_gbps"] = by_variant
    out["buffer_bytes"] = nbytes
    out["kernels"] = "manifold_constrained_hyper_amd/probe/bw_probe.hip"
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def copy_probe(args):
    """One copy kernel of known size (bw_probe.hip, 1 GiB read + 1 GiB
    written per launch): the reference against which rocprofv3 FETCH_SIZE /
    WRITE_SIZE counts are scaled."""
    import torch
    res = bandwidth_probe(torch, args.steps, args.warmup)
    print(json.dumps({"copy_probe_bytes_read": res["buffer_bytes"], "copy_probe_bytes_written": res["buffer_bytes"],
                      "kernel": "copy_kernel (bw_probe.hip)", "copy_gbps": res["copy_gbps"]}), flush=True)


def _variants(args, mhc, torch, synth, stream, ev):
    """The E4M3 pipeline on the headline workload and both dtypes on the
    other workloads (see the module docstring)."""
    B, n, C = (synth.CONFIGS[args.workload][k] for k in ("B", "n", "C"))
    fp8_inp = synth.make_config_fp8(args.workload, device="cuda")
    pf = Pipeline(mhc, torch, fp8_inp, fp8=True)
    steps, warm = max(args.steps, SECONDARY_STEPS), max(args.warmup, SECONDARY_WARMUP)
    fp8_line = _summary(
        B, n, C, 1, pf.time_loop(pf.layer, steps, warm),
        pf.time_loop(pf.three, steps, warm),
        pf.per_call(pf.layer, ("mhc_pre_fp8", "mhc_post_res_coeffs_fp8"), args.steps),
        pf.per_call(pf.three, ("mhc_coeffs_fp8", "mhc_pre_fp8", "mhc_post_res_fp8"), args.steps),
        ms_onepass=pf.time_loop(pf.onepass, steps, warm), ms_first=pf.time_loop(pf.first, steps, warm))
    fp8_line["first_layer_route"] = ("one pass" if mhc.mhc_coeffs_pre_fp8_one_pass(B, n, C)
                                     else "mhc_coeffs_fp8 + mhc_pre_fp8")
    fp8_line["onepass_route"] = ("one pass" if mhc.mhc_post_res_coeffs_pre_fp8_one_pass(B, n, C)
                                 else "mhc_post_res_coeffs_fp8 + mhc_pre_fp8")
    del pf, fp8_inp

    # ---- the other workloads (parity-test shapes), both dtypes: mean over 50
    # back-to-back layers (launch-bound at tiny and decode sizes); decode also
    # "cold", with a 512 MB write between layers and events around each layer.
    workloads = {}
    for wname in synth.CONFIGS:
        if wname == args.workload:
            continue
        wcfg = synth.CONFIGS[wname]
        wsteps = 50
        res = {"shape": f"n={wcfg['n']} C={wcfg['C']} B={wcfg['B']}"}
        for dname, fp8 in (("bf16", False), ("fp8", True)):
            winp = (synth.make_config_fp8 if fp8 else synth.make_config)(wname, device="cuda")
            pw = Pipeline(mhc, torch, winp, fp8=fp8)
            res[dname] = _summary(wcfg["B"], wcfg["n"], wcfg["C"], 1 if fp8 else 2,
                                  pw.time_loop(pw.layer, wsteps, 10), pw.time_loop(pw.three, wsteps, 10),
                                  ms_onepass=pw.time_loop(pw.onepass, wsteps, 10),
                                  ms_first=pw.time_loop(pw.first, wsteps, 10))
            if wname in ("tiny", "decode", "prefill"):  # launch-bound sizes: the same layers replayed from a graph
                res[dname]["graph_onepass_us_per_layer"] = round(pw.time_graph(pw.onepass) * 1e3, 2)
            sfx = "_fp8" if fp8 else ""
            one = getattr(mhc, "mhc_post_res_coeffs_pre" + sfx + "_one_pass")(wcfg["B"], wcfg["n"], wcfg["C"])
            res[dname]["onepass_route"] = ("one pass" if one else
                                           f"mhc_post_res_coeffs{sfx} + mhc_pre{sfx}")
            res[dname]["onepass_per_call"] = _stats(pw.per_call_all(pw.onepass, ("c",), wsteps)["c"])
            if wname in ("tiny", "decode", "prefill"):  # working sets that fit the MALL: also flushed
                res[dname]["flushed_onepass_per_call"] = _stats(pw.flushed(pw.onepass))
            del pw, winp
        workloads[wname] = res

    return fp8_line, workloads


def _phi32(mhc, torch, synth, stream, ev, names, steps=50, warmup=10):
    """mhc_coeffs_phi32 (fp32 phi, hi + lo bf16 product) beside mhc_coeffs on
    the same X: mean time of back-to-back calls, HIP events on the stream."""
    out = {}
    for name in names:
        inp = synth.make_config_phi32(name, device="cuda")
        B, n, C = inp["B"], inp["n"], inp["C"]
        N = n * n + 2 * n
        phi16 = inp["phi"].to(torch.bfloat16)
        lg, r, H = (torch.empty(B, N, device="cuda"), torch.empty(B, device="cuda"),
                    torch.empty(B, N, device="cuda"))
        ws = torch.empty(max(mhc.mhc_coeffs_phi32_workspace_size(B, n, C),
                             mhc.mhc_coeffs_workspace_size(B, n, C), 16), dtype=torch.uint8, device="cuda")
        args = (inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"], inp["b_pre"], inp["b_post"],
                inp["b_res"], lg, r, H, ws)
        res = {"shape": f"n={n} C={C} B={B}"}
        for label, fn in (("phi32_us", lambda: mhc.mhc_coeffs_phi32(B, n, C, inp["X"], inp["phi"], *args,
                                                                    stream=stream)),
                          ("bf16_phi_us", lambda: mhc.mhc_coeffs(B, n, C, inp["X"], phi16, *args,
                                                                 stream=stream))):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            res[label] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
        out[name] = res
        del inp, phi16, lg, r, H, ws
    return out


def _lazy_prenorm(mhc, torch, synth, stream, ev, steps=20, warmup=5):
    """mhc_lazy_prenorm_gemm on its synthetic workloads: mean time of
    back-to-back calls (HIP events on the launch stream), TFLOP/s against the
    dense bf16 MFMA peak, and the algorithmic bytes (A, W, C, rstd) for context."""
    out = {}
    for name, cfg in synth.LPN_CONFIGS.items():
        M, N, K = cfg["M"], cfg["N"], cfg["K"]
        d = synth.make_lpn_inputs(M, N, K, seed=cfg["seed"], device="cuda")
        C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        r = torch.empty(M, dtype=torch.float32, device="cuda")

        def call():
            mhc.mhc_lazy_prenorm_gemm(M, N, K, d["A"], d["W"], C, r, stream=stream)

        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
        nbytes = 2 * (M * K + N * K + M * N) + 4 * M
        # The roof is whichever floor is higher: the flops at the dense bf16
        # MFMA peak or the algorithmic bytes at the HBM peak.
        t_mfma = 2.0 * M * N * K / (BF16_MFMA_PEAK_TFLOPS * 1e12) * 1e6
        t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9) * 1e6
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        out[name] = {"shape": f"M={M} N={N} K={K}", "us_per_call": round(us, 2),
                     "tflops": round(tflops, 1), "bound": bound,
                     "roofline_us": round(max(t_mfma, t_hbm), 2),
                     "frac_of_roofline": round(max(t_mfma, t_hbm) / us, 4),
                     "frac_of_bf16_peak": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "algorithmic_bytes": nbytes,
                     "hbm_gbps_at_algorithmic_bytes": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del d, C, r
    return out


def _lpn_counters(mhc, torch, synth, launches=8):
    """The square Lazy Pre-Norm workload for counter runs: `launches` calls of
    the eight-wave kernel (the default), of the four-wave kernel
    (MHC_LPN_ALGO = 1), then of torch's A @ W^T (the vendor GEMM, no norm) as
    the library reference, each group followed by a device synchronisation."""
    cfg = synth.LPN_CONFIGS["lpn_square"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    d = synth.make_lpn_inputs(M, N, K, seed=cfg["seed"], device="cuda")
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    r = torch.empty(M, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    try:
        for algo in (0, 1):
            mhc.mhc_tuning_set("MHC_LPN_ALGO", algo)
            for _ in range(launches):
                mhc.mhc_lazy_prenorm_gemm(M, N, K, d["A"], d["W"], C, r, stream=s)
            torch.cuda.synchronize()
    finally:
        mhc.mhc_tuning_set("MHC_LPN_ALGO", -1)
    for _ in range(launches):
        torch.matmul(d["A"], d["W"].t())
    torch.cuda.synchronize()
    print(json.dumps({"lpn_counters": {"shape": f"M={M} N={N} K={K}", "launches": launches}}), flush=True)


SWEEP_SHAPES = [(4, 2048, 16384), (4, 4096, 16384), (4, 7168, 1024), (4, 7168, 4096),
                (4, 7168, 16384), (4, 7168, 32768), (4, 7168, 65536), (4, 8192, 16384),
                (2, 7168, 16384), (1, 7168, 16384)]


def _shape_sweep(mhc, torch, synth):
    """mhc_post_res_coeffs_pre(_fp8) chained over layers at each shape of
    SWEEP_SHAPES: mean us per layer and TB/s of its algorithmic bytes."""
    for fp8 in (False, True):
        for n, C, B in SWEEP_SHAPES:
            make = synth.make_inputs_fp8 if fp8 else synth.make_inputs
            inp = make(n, C, B, "normal", seed=7, device="cuda")
            N = n * n + 2 * n
            sfx = "_fp8" if fp8 else ""
            ab = (inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"], inp["b_pre"], inp["b_post"],
                  inp["b_res"])
            H0, lg = torch.empty(B, N, device="cuda"), torch.empty(B, N, device="cuda")
            r = torch.empty(B, device="cuda")
            wsc = torch.empty(max(getattr(mhc, f"mhc_coeffs{sfx}_workspace_size")(B, n, C), 16),
                              dtype=torch.uint8, device="cuda")
            getattr(mhc, f"mhc_coeffs{sfx}")(B, n, C, inp["X"], inp["phi"], *ab, lg, r, H0, wsc)
            X, Hs = [inp["X"], torch.empty_like(inp["X"])], [H0, torch.empty_like(H0)]
            F = torch.empty(B, C, dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
            ws = torch.empty(max(getattr(mhc, f"mhc_post_res_coeffs_pre{sfx}_workspace_size")(B, n, C), 16),
                             dtype=torch.uint8, device="cuda")
            call = getattr(mhc, f"mhc_post_res_coeffs_pre{sfx}")
            cur = [0]

            def layer():
                a = cur[0]
                call(B, n, C, X[a], inp["F_out"], Hs[a], X[1 - a], inp["phi"], *ab, lg, r, Hs[1 - a], F, ws)
                cur[0] = 1 - a

            def timed(k):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(k):
                    layer()
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / k

            layer()
            torch.cuda.synchronize()
            k = max(20, int(60e3 / timed(4)))
            timed(k)  # warm-up
            us = timed(k)
            nbytes = path_bytes(B, n, C, 1 if fp8 else 2)["mhc_post_res_coeffs_pre"]
            one = getattr(mhc, f"mhc_post_res_coeffs_pre{sfx}_one_pass")(B, n, C)
            print(json.dumps({"shape_sweep": {"n": n, "C": C, "B": B, "dtype": "e4m3" if fp8 else "bf16",
                                              "route": "one pass" if one else "two calls", "layers": k,
                                              "us_per_layer": round(us, 1),
                                              "hbm_gbps": round(nbytes / us / 1e3, 1),
                                              "tokens_per_s": round(B / us * 1e6, 1)}}), flush=True)
            del inp, X, Hs, F, ws, wsc, H0, lg, r
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Steady state: the first 20-40 back-to-back layers run slower (clocks and
    # caches settling) unless other loops ran first, as they do here; the
    # default warm-up is 50 layers.  100 timed layers take ~45 ms.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--cpu-budget-s", type=float, default=30.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--bw-probe", action="store_true",
                    help="print only the practical copy / write / read ceilings (plain torch kernels)")
    ap.add_argument("--kernel-only", action="store_true")
    ap.add_argument("--two-call-only", action="store_true",
                    help="run only the two-call pipeline's timed loop (counter runs of its kernels)")
    ap.add_argument("--three-call-only", action="store_true",
                    help="run only the three separate calls' timed loop (counter runs of their kernels)")
    ap.add_argument("--first-layer-only", action="store_true",
                    help="run only the first layer's call (mhc_coeffs_pre) in a timed loop (counter runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the E4M3 and other-workload sections (profiling runs of one workload)")
    ap.add_argument("--lazy-prenorm-only", action="store_true",
                    help="time only mhc_lazy_prenorm_gemm on its workloads (profiling runs)")
    ap.add_argument("--lpn-counters", action="store_true",
                    help="square Lazy Pre-Norm workload: a few launches of each kernel layout and of "
                         "torch's A @ W^T (counter runs)")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="time the one-pass layer call over a grid of shapes (one JSON line each)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the mHC forward shards by rows (tokens) with no "
              "exchange between GPUs, so a multi-GPU figure would be N independent copies of this "
              "one; run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import manifold_constrained_hyper_amd as mhc
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args)
        return
    if args.bw_probe:
        print(json.dumps({"practical_ceiling": bandwidth_probe(torch, args.steps, args.warmup)}), flush=True)
        return

    mhc.load()  # raises if the HIP library is not built
    if args.shape_sweep:
        _shape_sweep(mhc, torch, synth)
        return
    if args.lpn_counters:
        _lpn_counters(mhc, torch, synth)
        return
    if args.lazy_prenorm_only:
        lpn = _lazy_prenorm(mhc, torch, synth, torch.cuda.current_stream(),
                            lambda: torch.cuda.Event(enable_timing=True), args.steps, args.warmup)
        print(json.dumps({"lazy_prenorm": lpn}), flush=True)
        return
    cfg = synth.CONFIGS[args.workload]
    inp = synth.make_config(args.workload, device="cuda")
    B, n, C = inp["B"], inp["n"], inp["C"]
    N = n * n + 2 * n
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # The CPU baseline samples the input before the chained loop overwrites it.
    cpu = None
    if (not args.no_cpu_baseline and not args.kernel_only and not args.two_call_only
            and not args.three_call_only and not args.first_layer_only):
        cpu = _cpu_baseline(inp, args.cpu_rows, args.cpu_budget_s)

    # ---- headline: one call per layer, residual stream chained through layers
    X = [inp["X"], torch.empty_like(inp["X"])]
    Hs = [torch.empty(B, N, device="cuda") for _ in range(2)]
    logits = torch.empty(B, N, device="cuda")
    r = torch.empty(B, device="cuda")
    F_pre = torch.empty(B, C, dtype=torch.bfloat16, device="cuda")
    ws_c = torch.empty(max(mhc.mhc_coeffs_workspace_size(B, n, C), 16), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(max(mhc.mhc_post_res_coeffs_workspace_size(B, n, C),
                           mhc.mhc_post_res_coeffs_pre_workspace_size(B, n, C), 16),
                       dtype=torch.uint8, device="cuda")
    ab = (inp["alpha_pre"], inp["alpha_post"], inp["alpha_res"], inp["b_pre"], inp["b_post"], inp["b_res"])
    # The three separate calls run on a fixed X_t (a copy: the chained layers
    # overwrite inp["X"]).
    X3 = inp["X"].clone()
    mhc.mhc_coeffs(B, n, C, X[0], inp["phi"], *ab, logits, r, Hs[0], ws_c, stream=stream)
    mhc.mhc_pre(B, n, C, X[0], Hs[0], F_pre, stream=stream)
    cur = [0]

    def layer(marks=None):
        a = cur[0]
        if marks is not None:
            marks[0].record(stream)
        mhc.mhc_post_res_coeffs_pre(B, n, C, X[a], inp["F_out"], Hs[a], X[1 - a], inp["phi"], *ab,
                                    logits, r, Hs[1 - a], F_pre, ws_f, stream=stream)
        if marks is not None:
            marks[1].record(stream)
        cur[0] = 1 - a

    def two_call_layer(marks=None):
        a = cur[0]
        if marks is not None:
            marks[0].record(stream)
        mhc.mhc_pre(B, n, C, X[a], Hs[a], F_pre, stream=stream)
        if marks is not None:
            marks[1].record(stream)
        mhc.mhc_post_res_coeffs(B, n, C, X[a], inp["F_out"], Hs[a], X[1 - a], inp["phi"], *ab,
                                logits, r, Hs[1 - a], ws_f, stream=stream)
        if marks is not None:
            marks[2].record(stream)
        cur[0] = 1 - a

    out = mhc.alloc_outputs(B, n, C)

    def three(marks=None):
        if marks is not None:
            marks[0].record(stream)
        mhc.mhc_coeffs(B, n, C, X3, inp["phi"], *ab, out["logits"], out["r"], out["H"],
                       out["workspace"], stream=stream)
        if marks is not None:
            marks[1].record(stream)
        mhc.mhc_pre(B, n, C, X3, out["H"], out["F_pre"], stream=stream)
        if marks is not None:
            marks[2].record(stream)
        mhc.mhc_post_res(B, n, C, X3, inp["F_out"], out["H"], out["X_next"], stream=stream)
        if marks is not None:
            marks[3].record(stream)

    ws_cp = torch.empty(max(mhc.mhc_coeffs_pre_workspace_size(B, n, C), 16), dtype=torch.uint8, device="cuda")

    def first(marks=None):
        if marks is not None:
            marks[0].record(stream)
        mhc.mhc_coeffs_pre(B, n, C, X3, inp["phi"], *ab, out["logits"], out["r"], out["H"], out["F_pre"],
                           ws_cp, stream=stream)
        if marks is not None:
            marks[1].record(stream)

    def timed(fn, warmup=None, steps=None):
        warmup = args.warmup if warmup is None else warmup
        steps = args.steps if steps is None else steps
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - w0

    def per_call(fn, names):
        """Every call's ms, from an event before and after each call."""
        marks = [[ev() for _ in range(len(names) + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            fn(marks[k])
        torch.cuda.synchronize()
        return {c: [marks[k][i].elapsed_time(marks[k][i + 1]) for k in range(args.steps)]
                for i, c in enumerate(names)}

    mean = lambda v: sum(v) / len(v)  # noqa: E731
    sec_warm, sec_steps = max(args.warmup, SECONDARY_WARMUP), max(args.steps, SECONDARY_STEPS)

    if args.two_call_only:  # counter runs of the two-call pipeline's kernels
        timed(two_call_layer)
        print(json.dumps({"two_call_only": True, "steps": args.steps}), flush=True)
        return
    if args.three_call_only:  # counter runs of the three calls' kernels
        timed(three)
        print(json.dumps({"three_call_only": True, "steps": args.steps}), flush=True)
        return
    if args.first_layer_only:  # counter runs of the first layer's call
        timed(first)
        print(json.dumps({"first_layer_only": True, "steps": args.steps}), flush=True)
        return

    ms_three = ms_two = None
    if not args.kernel_only:
        # The other bf16 pipelines first (the GPU is then at its working
        # clocks when the headline loop starts), each with at least
        # SECONDARY_WARMUP warm-up and SECONDARY_STEPS timed steps.
        # Three separate calls on a fixed X_t.
        ms_three, _ = timed(three, sec_warm, sec_steps)
        three_calls = ("mhc_coeffs", "mhc_pre", "mhc_post_res")
        per_call3 = per_call(three, three_calls)
        # The two-call pipeline (mhc_pre + mhc_post_res_coeffs per layer).
        ms_two, _ = timed(two_call_layer, sec_warm, sec_steps)
        per_two = per_call(two_call_layer, ("mhc_pre", "mhc_post_res_coeffs"))
        mhc.mhc_pre(B, n, C, X[cur[0]], Hs[cur[0]], F_pre, stream=stream)
        # The first layer's call on the fixed X_t, against mhc_coeffs +
        # mhc_pre (the three calls' first two).
        ms_first, _ = timed(first, sec_warm, sec_steps)
        per_first = per_call(first, ("mhc_coeffs_pre",))

    # Timed region (the headline number): W warm-up layers, then K
    # back-to-back layers bracketed by two events and a device
    # synchronisation on both sides; no event sits between calls (each
    # recorded event idles the stream a few microseconds).
    ms_step, wall = timed(layer)
    if args.kernel_only:
        print(json.dumps({"kernel_only": True, "steps": args.steps}), flush=True)
        return
    # The same layers with an event before and after each call (per-call
    # durations on the stream the kernels run on).
    pipe_calls = ("mhc_post_res_coeffs_pre",)
    per_call_all = per_call(layer, pipe_calls)
    per_call_ms = {c: mean(v) for c, v in per_call_all.items()}

    del X, Hs, out, X3, ws_cp
    torch.cuda.empty_cache()
    probe = bandwidth_probe(torch)

    # ---- the E4M3 residual-stream variant on the same workload (same shapes
    # and draws, X and F_out rounded to E4M3), the other workloads, the
    # Lazy Pre-Norm GEMM and the fp32-phi product
    fp8_line, workloads, lpn, phi32 = None, None, None, None
    if not args.headline_only:
        fp8_line, workloads = _variants(args, mhc, torch, synth, stream, ev)
        lpn = _lazy_prenorm(mhc, torch, synth, stream, ev)
        phi32 = _phi32(mhc, torch, synth, stream, ev, ("decode", args.workload))

    bytes_call = path_bytes(B, n, C)
    pipe_bytes = bytes_call["mhc_post_res_coeffs_pre"]
    two_bytes = bytes_call["mhc_pre"] + bytes_call["mhc_post_res_coeffs"]
    three_bytes = sum(bytes_call[c] for c in three_calls)
    gbps = pipe_bytes / (ms_step * 1e-3) / 1e9
    tokens_per_s = B / (ms_step * 1e-3)

    dom = max(pipe_calls, key=lambda c: per_call_ms[c])
    dom_gbps = bytes_call[dom] / (per_call_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "call": dom, "kernel": KERNELS_OF_CALL[dom],
                "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dom_gbps / HBM_PEAK_GBPS, 4), "traffic": _recorded_traffic(dom, args.workload),
                "algorithmic_bytes_per_launch": bytes_call[dom],
                "avg_launch_us": round(per_call_ms[dom] * 1e3, 2)}

    def leg(ms, nbytes, per):
        return {"ms_per_step": round(ms, 5), "tokens_per_s": round(B / (ms * 1e-3), 1),
                "hbm_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "hbm_frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "algorithmic_bytes_per_step": nbytes,
                "per_call_us": {c: round(mean(v) * 1e3, 2) for c, v in per.items()},
                "per_call_stats": {c: _stats(v) for c, v in per.items()}}

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; X Student-t(4) for the large workload)",
        "config": {"workload": f"{args.workload}: n={n} C={C} B={B}", "n": n, "C": C, "B": B,
                   "x_dist": cfg["x_dist"], "seed": cfg["seed"],
                   "path": "per layer: mhc_post_res_coeffs_pre (mhc_coeffs and mhc_pre once before the loop)",
                   "one_pass": mhc.mhc_post_res_coeffs_pre_one_pass(B, n, C)},
        # bandwidth of the timed step on the bytes the one-pass call moves
        # (X_t, F_out in; X_next, F_pre_next out; coefficients and phi)
        "hbm_gbps": round(gbps, 1), "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": pipe_bytes,
        "bytes_definition": "one-pass call's own algorithmic bytes (not the three-call definition)",
        # the same step against the three-call algorithmic byte definition:
        # the three calls' bytes moved per second of this step's time would
        # exceed the HBM peak, so only the ratio of tokens/s is reported
        "speedup_vs_three_call": round(ms_three / ms_step, 3),
        "frac_of_practical_copy_ceiling": round(gbps / probe["copy_gbps"], 4),
        "per_call_us": {c: round(v * 1e3, 2) for c, v in per_call_ms.items()},
        "per_call_stats": {c: _stats(v) for c, v in per_call_all.items()},
        "per_call_gbps": {c: round(bytes_call[c] / (per_call_ms[c] * 1e-3) / 1e9, 1) for c in pipe_calls},
        "two_call_pipeline": leg(ms_two, two_bytes, per_two),
        "three_call": dict(leg(ms_three, three_bytes, per_call3), split_k=mhc.mhc_coeffs_split_k(B, n, C),
                           frac_of_practical_copy_ceiling=round(
                               three_bytes / (ms_three * 1e-3) / 1e9 / probe["copy_gbps"], 4)),
        "first_layer": {
            "call": "mhc_coeffs_pre", "kernel": KERNELS_OF_CALL["mhc_coeffs_pre"],
            "route": "one pass" if mhc.mhc_coeffs_pre_one_pass(B, n, C) else "mhc_coeffs + mhc_pre",
            **leg(ms_first, bytes_call["mhc_coeffs_pre"], per_first),
            "vs_mhc_coeffs_plus_mhc_pre_us": round(
                (mean(per_call3["mhc_coeffs"]) + mean(per_call3["mhc_pre"])) * 1e3, 2),
            "frac_of_practical_copy_ceiling": round(
                bytes_call["mhc_coeffs_pre"] / (ms_first * 1e-3) / 1e9 / probe["copy_gbps"], 4)},
        "practical_ceiling": probe,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fp8": None if fp8_line is None else dict(
            fp8_line, note="E4M3 residual stream (X_t, F_out, F_pre, X_next), same workload; "
                           "the *_fp8 entry points"),
        "workloads": workloads,
        "lazy_prenorm": lpn,
        "phi32_coeffs": phi32,
        "kernel_source_sha": {c: kernel_source_sha(c) for c in CALL_SOURCES},
    }
    print(json.dumps(line), flush=True)

if __name__ == "__main__":
    main()
