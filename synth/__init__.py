"""Seeded synthetic inputs for the mHC forward.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  Both the HIP path (through its Python binding) and the
CPU oracle are fed from the same tensors it returns, so both sides see the
identical bf16 bytes.

Workloads (shapes follow the dimensions defined in [mHC-cutile] section 2:
B rows = batch x sequence, n streams, hidden size C; page [mHC-cutile] is
"mHC 算法分析 & cutile 高效实现"):

  name      n  C     B      X distribution
  tiny      4  256   64     N(0, 1)
  prefill   4  4096  4096   N(0, 1)            (batch 1 x sequence 4096)
  decode    4  7168  64     N(0, 1)
  large     4  7168  16384  Student-t, 4 dof   (rows carry outliers)
  wide      8  4096  8192   N(0, 1)

For every workload: phi ~ N(0, sigma = 1/sqrt(nC)) so logits are O(1);
alpha_pre = alpha_post = alpha_res = 0.01; b_pre, b_post ~ N(0, sigma = 0.1);
b_res = 2 * I_n (flattened row-major) + N(0, sigma = 0.1); F_out ~ N(0, 1).
X, phi and F_out are drawn in fp32 and rounded to bf16 (round-to-nearest-even);
biases stay fp32.  The Student-t(4) draw is z / sqrt(chi2_4 / 4) with chi2_4 the
sum of four squared standard normals.
"""

import math

import numpy as np
import torch

CONFIGS = {
    "tiny": dict(n=4, C=256, B=64, x_dist="normal", seed=1000),
    "prefill": dict(n=4, C=4096, B=4096, x_dist="normal", seed=1001),
    "decode": dict(n=4, C=7168, B=64, x_dist="normal", seed=1002),
    "large": dict(n=4, C=7168, B=16384, x_dist="student_t4", seed=1003),
    "wide": dict(n=8, C=4096, B=8192, x_dist="normal", seed=1004),
}

ALPHA = 0.01


def _draw_rows(gen, rows, cols, dist, device):
    z = torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)
    if dist == "normal":
        return z
    if dist == "student_t4":
        chi2 = torch.zeros_like(z)
        for _ in range(4):
            w = torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)
            chi2.addcmul_(w, w)
        return z / torch.sqrt(chi2 / 4.0)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(n, C, B, x_dist="normal", seed=0, device="cpu", row_chunk=512, phi32=False):
    """Draw one seeded input set.  Returns a dict of torch tensors on `device`
    (X bf16 [B, nC], phi bf16 [nC, N], F_out bf16 [B, C], b_pre/b_post fp32 [n],
    b_res fp32 [n*n]) plus the python floats alpha_pre/post/res and the sizes.
    phi32=True keeps phi in fp32 (the same draw, not rounded to bf16)."""
    device = torch.device(device)
    K = n * C
    N = n * n + 2 * n
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    X = torch.empty(B, K, dtype=torch.bfloat16, device=device)
    for lo in range(0, B, row_chunk):
        hi = min(B, lo + row_chunk)
        X[lo:hi] = _draw_rows(gen, hi - lo, K, x_dist, device).to(torch.bfloat16)
    phi = torch.randn(K, N, generator=gen, device=device) / math.sqrt(K)
    phi = phi.contiguous() if phi32 else phi.to(torch.bfloat16)
    b_pre = 0.1 * torch.randn(n, generator=gen, device=device)
    b_post = 0.1 * torch.randn(n, generator=gen, device=device)
    b_res = (2.0 * torch.eye(n, device=device).reshape(-1)
             + 0.1 * torch.randn(n * n, generator=gen, device=device))
    F_out = torch.empty(B, C, dtype=torch.bfloat16, device=device)
    for lo in range(0, B, row_chunk * 4):
        hi = min(B, lo + row_chunk * 4)
        F_out[lo:hi] = torch.randn(hi - lo, C, generator=gen, device=device).to(torch.bfloat16)
    return {
        "n": n, "C": C, "B": B, "seed": int(seed), "x_dist": x_dist,
        "X": X, "phi": phi, "F_out": F_out,
        "b_pre": b_pre.float().contiguous(), "b_post": b_post.float().contiguous(),
        "b_res": b_res.float().contiguous(),
        "alpha_pre": ALPHA, "alpha_post": ALPHA, "alpha_res": ALPHA,
    }


def make_config(name, device="cpu"):
    """Inputs for one named workload of CONFIGS."""
    cfg = CONFIGS[name]
    return make_inputs(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"], device)


def make_config_phi32(name, device="cpu"):
    """Inputs for one named workload of CONFIGS with phi kept in fp32 (the
    bf16 config's phi is this phi rounded to bf16)."""
    cfg = CONFIGS[name]
    return make_inputs(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"], device, phi32=True)


def bf16_bits(t):
    """Raw bf16 bit patterns of a bf16 tensor as a numpy uint16 array (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_e4m3(t):
    """Round a tensor to FP8 E4M3 (the OCP "fn" encoding, round to nearest
    even) after clamping to +-448; returns the raw codes as a uint8 tensor on
    the same device."""
    return t.float().clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def make_inputs_fp8(n, C, B, x_dist="normal", seed=0, device="cpu", row_chunk=512):
    """make_inputs with X and F_out rounded to E4M3 (uint8 codes), for the FP8
    residual-stream variant; phi and the biases are unchanged."""
    inp = make_inputs(n, C, B, x_dist, seed, device, row_chunk)
    for k in ("X", "F_out"):
        src = inp[k]
        out = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
        for lo in range(0, src.shape[0], row_chunk):
            out[lo:lo + row_chunk] = to_e4m3(src[lo:lo + row_chunk])
        inp[k] = out
    inp["fp8"] = True
    return inp


def make_config_fp8(name, device="cpu"):
    """FP8 inputs for one named workload of CONFIGS."""
    cfg = CONFIGS[name]
    return make_inputs_fp8(cfg["n"], cfg["C"], cfg["B"], cfg["x_dist"], cfg["seed"], device)


def e4m3_codes(t):
    """Raw E4M3 codes of a uint8 (or float8_e4m3fn) tensor as a numpy uint8 array."""
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


# Lazy Pre-Norm GEMM workloads (C = rmsnorm(A) @ W^T): A is the pre-mixed
# layer input of the large workload (rows of a fixed scale spread, so rstd
# varies), W a linear layer's weight [N, K].
LPN_CONFIGS = {
    "lpn_proj": dict(M=16384, N=1536, K=7168, seed=2001),
    "lpn_square": dict(M=16384, N=7168, K=7168, seed=2002),
    "lpn_ads": dict(M=262144, N=512, K=512, seed=2003),
}


def make_lpn_inputs(M, N, K, seed=0, device="cpu", row_chunk=2048):
    """A bf16 [M, K] = z * s_row (z ~ N(0, 1), s_row = 2^u, u ~ U(-2, 2) per
    row); W bf16 [N, K] ~ N(0, sigma = 1/sqrt(K))."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    A = torch.empty(M, K, dtype=torch.bfloat16, device=device)
    for lo in range(0, M, row_chunk):
        hi = min(M, lo + row_chunk)
        z = torch.randn(hi - lo, K, generator=gen, device=device)
        u = torch.rand(hi - lo, 1, generator=gen, device=device) * 4.0 - 2.0
        A[lo:hi] = (z * torch.exp2(u)).to(torch.bfloat16)
    W = torch.empty(N, K, dtype=torch.bfloat16, device=device)
    for lo in range(0, N, row_chunk):
        hi = min(N, lo + row_chunk)
        W[lo:hi] = (torch.randn(hi - lo, K, generator=gen, device=device) / math.sqrt(K)).to(torch.bfloat16)
    return {"M": M, "N": N, "K": K, "A": A, "W": W, "seed": int(seed)}
