"""Thin ctypes binding of libmhc (include/mhc.h).

Argument marshalling only: every step of the forward runs in the HIP kernels
of libmhc.  Tensors are torch tensors used as device-memory handles; the
current torch HIP stream is passed unless a stream is given.  There is no CPU
fallback: if the library is missing or fails to load, every call raises.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmhc.so")

MHC_OK = 0
MHC_ERR_INVALID_ARG = 1
MHC_ERR_UNSUPPORTED = 2
MHC_ERR_WORKSPACE = 3
MHC_ERR_HIP = 4
MHC_SINKHORN_ITERS = 20

EXPORTED = ("mhc_status_string", "mhc_coeffs_workspace_size", "mhc_coeffs_split_k",
            "mhc_coeffs", "mhc_pre", "mhc_post_res", "mhc_post_res_coeffs_workspace_size",
            "mhc_post_res_coeffs", "mhc_coeffs_fp8_workspace_size", "mhc_coeffs_fp8",
            "mhc_pre_fp8", "mhc_post_res_fp8", "mhc_post_res_coeffs_fp8_workspace_size",
            "mhc_post_res_coeffs_fp8", "mhc_coeffs_phi32_workspace_size", "mhc_coeffs_phi32",
            "mhc_post_res_coeffs_phi32_workspace_size", "mhc_post_res_coeffs_phi32",
            "mhc_lazy_prenorm_gemm", "mhc_post_res_coeffs_pre_workspace_size",
            "mhc_post_res_coeffs_pre", "mhc_post_res_coeffs_pre_one_pass",
            "mhc_post_res_coeffs_pre_fp8_workspace_size", "mhc_post_res_coeffs_pre_fp8",
            "mhc_post_res_coeffs_pre_fp8_one_pass")

_lib = None


class MhcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {mhc_status_string(status)} (status {status})")


def load():
    """Load libmhc.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m manifold_constrained_hyper_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, f32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.mhc_status_string.argtypes = [ctypes.c_int]
    lib.mhc_status_string.restype = ctypes.c_char_p
    lib.mhc_coeffs_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_coeffs_workspace_size.restype = sz
    lib.mhc_coeffs_split_k.argtypes = [i64, i32, i64]
    lib.mhc_coeffs_split_k.restype = i32
    lib.mhc_coeffs.argtypes = [i64, i32, i64, vp, vp, f32, f32, f32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mhc_coeffs.restype = ctypes.c_int
    lib.mhc_pre.argtypes = [i64, i32, i64, vp, vp, vp, vp]
    lib.mhc_pre.restype = ctypes.c_int
    lib.mhc_post_res.argtypes = [i64, i32, i64, vp, vp, vp, vp, vp]
    lib.mhc_post_res.restype = ctypes.c_int
    lib.mhc_post_res_coeffs_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_post_res_coeffs_workspace_size.restype = sz
    lib.mhc_post_res_coeffs.argtypes = [i64, i32, i64, vp, vp, vp, vp, vp, f32, f32, f32,
                                        vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mhc_post_res_coeffs.restype = ctypes.c_int
    for suffix in ("", "_fp8", "_phi32"):
        if suffix:
            getattr(lib, "mhc_coeffs" + suffix).argtypes = lib.mhc_coeffs.argtypes
            getattr(lib, "mhc_coeffs" + suffix).restype = ctypes.c_int
            if suffix == "_fp8":
                getattr(lib, "mhc_pre" + suffix).argtypes = lib.mhc_pre.argtypes
                getattr(lib, "mhc_pre" + suffix).restype = ctypes.c_int
                getattr(lib, "mhc_post_res" + suffix).argtypes = lib.mhc_post_res.argtypes
                getattr(lib, "mhc_post_res" + suffix).restype = ctypes.c_int
            getattr(lib, "mhc_post_res_coeffs" + suffix).argtypes = lib.mhc_post_res_coeffs.argtypes
            getattr(lib, "mhc_post_res_coeffs" + suffix).restype = ctypes.c_int
    lib.mhc_coeffs_fp8_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_coeffs_fp8_workspace_size.restype = sz
    lib.mhc_post_res_coeffs_fp8_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_post_res_coeffs_fp8_workspace_size.restype = sz
    lib.mhc_coeffs_phi32_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_coeffs_phi32_workspace_size.restype = sz
    lib.mhc_post_res_coeffs_phi32_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_post_res_coeffs_phi32_workspace_size.restype = sz
    lib.mhc_lazy_prenorm_gemm.argtypes = [i64, i64, i64, vp, vp, f32, vp, vp, vp]
    lib.mhc_lazy_prenorm_gemm.restype = ctypes.c_int
    lib.mhc_post_res_coeffs_pre_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_post_res_coeffs_pre_workspace_size.restype = sz
    lib.mhc_post_res_coeffs_pre.argtypes = [i64, i32, i64, vp, vp, vp, vp, vp, f32, f32, f32,
                                            vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mhc_post_res_coeffs_pre.restype = ctypes.c_int
    lib.mhc_post_res_coeffs_pre_one_pass.argtypes = [i64, i32, i64]
    lib.mhc_post_res_coeffs_pre_one_pass.restype = i32
    lib.mhc_post_res_coeffs_pre_fp8_workspace_size.argtypes = [i64, i32, i64]
    lib.mhc_post_res_coeffs_pre_fp8_workspace_size.restype = sz
    lib.mhc_post_res_coeffs_pre_fp8.argtypes = [i64, i32, i64, vp, vp, vp, vp, vp, f32, f32, f32,
                                                vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mhc_post_res_coeffs_pre_fp8.restype = ctypes.c_int
    lib.mhc_post_res_coeffs_pre_fp8_one_pass.argtypes = [i64, i32, i64]
    lib.mhc_post_res_coeffs_pre_fp8_one_pass.restype = i32
    _lib = lib
    return lib


def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Raises on host tensors."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)  # raw address
    if t.numel() > 0 and not t.is_cuda:
        raise ValueError("libmhc takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmhc takes contiguous tensors")
    return t.data_ptr() or None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status, where):
    if status != MHC_OK:
        raise MhcError(status, where)


def mhc_status_string(status):
    return load().mhc_status_string(int(status)).decode()


def mhc_coeffs_workspace_size(B, n, C):
    return int(load().mhc_coeffs_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_split_k(B, n, C):
    return int(load().mhc_coeffs_split_k(int(B), int(n), int(C)))


def mhc_coeffs(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
               logits, r, H, workspace, workspace_bytes=None, stream=None, check=True):
    """Steps (1)-(3): logits, r and H from X_t and phi (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_coeffs(int(B), int(n), int(C), _ptr(X_t), _ptr(phi), float(alpha_pre),
                           float(alpha_post), float(alpha_res), _ptr(b_pre), _ptr(b_post),
                           _ptr(b_res), _ptr(logits), _ptr(r), _ptr(H), _ptr(workspace),
                           int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "mhc_coeffs")
    return st


def mhc_pre(B, n, C, X_t, H, F_pre, stream=None, check=True):
    """Step (4a): F_pre = sum_i H_pre[i] X_t[i] (see include/mhc.h)."""
    st = load().mhc_pre(int(B), int(n), int(C), _ptr(X_t), _ptr(H), _ptr(F_pre), _stream(stream))
    if check:
        _check(st, "mhc_pre")
    return st


def mhc_post_res(B, n, C, X_t, F_out, H, X_next, stream=None, check=True):
    """Step (4b): X_next = H_res X_t + H_post^T F_out (see include/mhc.h)."""
    st = load().mhc_post_res(int(B), int(n), int(C), _ptr(X_t), _ptr(F_out), _ptr(H),
                             _ptr(X_next), _stream(stream))
    if check:
        _check(st, "mhc_post_res")
    return st


def mhc_post_res_coeffs_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                        alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next, workspace,
                        workspace_bytes=None, stream=None, check=True):
    """Step (4b) of this layer fused with steps (1)-(3) of the next (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_post_res_coeffs(int(B), int(n), int(C), _ptr(X_t), _ptr(F_out), _ptr(H),
                                    _ptr(X_next), _ptr(phi_next), float(alpha_pre),
                                    float(alpha_post), float(alpha_res), _ptr(b_pre), _ptr(b_post),
                                    _ptr(b_res), _ptr(logits_next), _ptr(r_next), _ptr(H_next),
                                    _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "mhc_post_res_coeffs")
    return st


def mhc_post_res_coeffs_pre_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_pre_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre_one_pass(B, n, C):
    return bool(load().mhc_post_res_coeffs_pre_one_pass(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                            alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                            F_pre_next, workspace, workspace_bytes=None, stream=None, check=True):
    """Step (4b) of this layer, then steps (1)-(3) and (4a) of the next, in
    one pass where the shape allows (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_post_res_coeffs_pre(int(B), int(n), int(C), _ptr(X_t), _ptr(F_out), _ptr(H),
                                        _ptr(X_next), _ptr(phi_next), float(alpha_pre),
                                        float(alpha_post), float(alpha_res), _ptr(b_pre),
                                        _ptr(b_post), _ptr(b_res), _ptr(logits_next), _ptr(r_next),
                                        _ptr(H_next), _ptr(F_pre_next), _ptr(workspace),
                                        int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "mhc_post_res_coeffs_pre")
    return st


def mhc_post_res_coeffs_pre_fp8_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_pre_fp8_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre_fp8_one_pass(B, n, C):
    return bool(load().mhc_post_res_coeffs_pre_fp8_one_pass(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre_fp8(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                                alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                                F_pre_next, workspace, workspace_bytes=None, stream=None,
                                check=True):
    """mhc_post_res_coeffs_pre on the E4M3 residual stream (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_post_res_coeffs_pre_fp8(int(B), int(n), int(C), _ptr(X_t), _ptr(F_out), _ptr(H),
                                            _ptr(X_next), _ptr(phi_next), float(alpha_pre),
                                            float(alpha_post), float(alpha_res), _ptr(b_pre),
                                            _ptr(b_post), _ptr(b_res), _ptr(logits_next),
                                            _ptr(r_next), _ptr(H_next), _ptr(F_pre_next),
                                            _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "mhc_post_res_coeffs_pre_fp8")
    return st


# FP8 (E4M3) residual-stream variant: same arguments, with X_t, F_out, F_pre
# and X_next as E4M3 tensors (torch.float8_e4m3fn or raw uint8 codes).

def mhc_coeffs_fp8_workspace_size(B, n, C):
    return int(load().mhc_coeffs_fp8_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_fp8(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                   logits, r, H, workspace, workspace_bytes=None, stream=None, check=True):
    """Steps (1)-(3) on an E4M3 X_t (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_coeffs_fp8(int(B), int(n), int(C), _ptr(X_t), _ptr(phi), float(alpha_pre),
                               float(alpha_post), float(alpha_res), _ptr(b_pre), _ptr(b_post),
                               _ptr(b_res), _ptr(logits), _ptr(r), _ptr(H), _ptr(workspace),
                               int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "mhc_coeffs_fp8")
    return st


def mhc_pre_fp8(B, n, C, X_t, H, F_pre, stream=None, check=True):
    """Step (4a) on the E4M3 residual stream (see include/mhc.h)."""
    st = load().mhc_pre_fp8(int(B), int(n), int(C), _ptr(X_t), _ptr(H), _ptr(F_pre), _stream(stream))
    if check:
        _check(st, "mhc_pre_fp8")
    return st


def mhc_post_res_fp8(B, n, C, X_t, F_out, H, X_next, stream=None, check=True):
    """Step (4b) on the E4M3 residual stream (see include/mhc.h)."""
    st = load().mhc_post_res_fp8(int(B), int(n), int(C), _ptr(X_t), _ptr(F_out), _ptr(H),
                                 _ptr(X_next), _stream(stream))
    if check:
        _check(st, "mhc_post_res_fp8")
    return st


def mhc_post_res_coeffs_fp8_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_fp8_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_fp8(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                            alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                            workspace, workspace_bytes=None, stream=None, check=True):
    """mhc_post_res_coeffs on the E4M3 residual stream (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_post_res_coeffs_fp8(int(B), int(n), int(C), _ptr(X_t), _ptr(F_out), _ptr(H),
                                        _ptr(X_next), _ptr(phi_next), float(alpha_pre),
                                        float(alpha_post), float(alpha_res), _ptr(b_pre),
                                        _ptr(b_post), _ptr(b_res), _ptr(logits_next), _ptr(r_next),
                                        _ptr(H_next), _ptr(workspace), int(workspace_bytes),
                                        _stream(stream))
    if check:
        _check(st, "mhc_post_res_coeffs_fp8")
    return st


def mhc_coeffs_phi32_workspace_size(B, n, C):
    return int(load().mhc_coeffs_phi32_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_phi32(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                     logits, r, H, workspace, workspace_bytes=None, stream=None, check=True):
    """Steps (1)-(3) with an fp32 phi (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_coeffs_phi32(int(B), int(n), int(C), _ptr(X_t), _ptr(phi), float(alpha_pre),
                                 float(alpha_post), float(alpha_res), _ptr(b_pre), _ptr(b_post),
                                 _ptr(b_res), _ptr(logits), _ptr(r), _ptr(H), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "mhc_coeffs_phi32")
    return st


def mhc_post_res_coeffs_phi32_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_phi32_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_phi32(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                              alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                              workspace, workspace_bytes=None, stream=None, check=True):
    """mhc_post_res_coeffs with an fp32 phi_next (see include/mhc.h)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().mhc_post_res_coeffs_phi32(int(B), int(n), int(C), _ptr(X_t), _ptr(F_out), _ptr(H),
                                          _ptr(X_next), _ptr(phi_next), float(alpha_pre),
                                          float(alpha_post), float(alpha_res), _ptr(b_pre),
                                          _ptr(b_post), _ptr(b_res), _ptr(logits_next), _ptr(r_next),
                                          _ptr(H_next), _ptr(workspace), int(workspace_bytes),
                                          _stream(stream))
    if check:
        _check(st, "mhc_post_res_coeffs_phi32")
    return st


def mhc_lazy_prenorm_gemm(M, N, K, A, W, C, rstd=None, eps=1e-5, stream=None, check=True):
    """C = rmsnorm(A) @ W^T (A bf16 [M, K], W bf16 [N, K], C bf16 [M, N]); rstd
    fp32 [M] if given (see include/mhc.h)."""
    st = load().mhc_lazy_prenorm_gemm(int(M), int(N), int(K), _ptr(A), _ptr(W), float(eps), _ptr(C),
                                      _ptr(rstd), _stream(stream))
    if check:
        _check(st, "mhc_lazy_prenorm_gemm")
    return st


def alloc_outputs(B, n, C, device="cuda"):
    """Caller-side buffers for one forward of shape (B, n, C): logits, r, H,
    F_pre, X_next and the coefficient workspace (uint8, 16-byte aligned)."""
    N = n * n + 2 * n
    ws_bytes = mhc_coeffs_workspace_size(B, n, C)
    return {
        "logits": torch.empty(B, N, dtype=torch.float32, device=device),
        "r": torch.empty(B, dtype=torch.float32, device=device),
        "H": torch.empty(B, N, dtype=torch.float32, device=device),
        "F_pre": torch.empty(B, C, dtype=torch.bfloat16, device=device),
        "X_next": torch.empty(B, n * C, dtype=torch.bfloat16, device=device),
        "workspace": torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device),
    }
