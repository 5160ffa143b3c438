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
MHC_ERR_INCOMPLETE = 5
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
            "mhc_post_res_coeffs_pre_fp8_one_pass", "mhc_post_res_coeffs_pre_check",
            "mhc_tuning_set", "mhc_tuning_reset", "mhc_post_res_coeffs_pre_noalloc",
            "mhc_coeffs_pre_workspace_size", "mhc_coeffs_pre", "mhc_coeffs_pre_one_pass",
            "mhc_coeffs_pre_check", "mhc_coeffs_pre_fp8_workspace_size", "mhc_coeffs_pre_fp8",
            "mhc_coeffs_pre_fp8_one_pass")

MHC_NOALLOC_SCRATCH_BYTES = 32 << 20

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
    lib.mhc_post_res_coeffs_pre_check.argtypes = [i64, i32, i64, i32, vp, sz, vp]
    lib.mhc_post_res_coeffs_pre_check.restype = ctypes.c_int
    lib.mhc_tuning_set.argtypes = [ctypes.c_char_p, i64]
    lib.mhc_tuning_set.restype = ctypes.c_int
    lib.mhc_post_res_coeffs_pre_noalloc.argtypes = [i64, i32, i64, vp, vp, vp, vp, vp, f32, f32, f32,
                                                    vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mhc_post_res_coeffs_pre_noalloc.restype = ctypes.c_int
    for suffix in ("", "_fp8"):
        getattr(lib, f"mhc_coeffs_pre{suffix}_workspace_size").argtypes = [i64, i32, i64]
        getattr(lib, f"mhc_coeffs_pre{suffix}_workspace_size").restype = sz
        getattr(lib, f"mhc_coeffs_pre{suffix}").argtypes = [i64, i32, i64, vp, vp, f32, f32, f32, vp, vp,
                                                           vp, vp, vp, vp, vp, vp, sz, vp]
        getattr(lib, f"mhc_coeffs_pre{suffix}").restype = ctypes.c_int
        getattr(lib, f"mhc_coeffs_pre{suffix}_one_pass").argtypes = [i64, i32, i64]
        getattr(lib, f"mhc_coeffs_pre{suffix}_one_pass").restype = i32
    lib.mhc_coeffs_pre_check.argtypes = [i64, i32, i64, i32, vp, sz, vp]
    lib.mhc_coeffs_pre_check.restype = ctypes.c_int
    lib.mhc_tuning_reset.argtypes = []
    lib.mhc_tuning_reset.restype = None
    _lib = lib
    return lib


def _ptr(t, nbytes=None, esize=None, name="tensor"):
    """Device pointer of a tensor (None -> NULL; an int is taken as a raw
    address).  Raises ValueError on host or non-contiguous tensors and, when
    the call's sizes are given, on a tensor of another element size (uint8
    tensors are taken as raw bytes) or smaller than the nbytes the library
    will touch, before anything runs."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)  # raw address
    if esize is not None and t.numel() > 0 and t.element_size() != esize and t.dtype != torch.uint8:
        raise ValueError(f"{name}: element size {t.element_size()} bytes, the call takes {esize}")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, the call needs {nbytes}")
    if not t.is_contiguous():
        raise ValueError("libmhc takes contiguous tensors")
    if t.numel() > 0 and not t.is_cuda:
        raise ValueError("libmhc takes device tensors")
    return t.data_ptr() or None


class _Sizes:
    """Byte counts of the tensors of one (B, n, C) call: eb bytes per
    residual-stream element (2 bf16, 1 E4M3), pb per phi element."""

    def __init__(self, B, n, C, eb=2, pb=2):
        B, n, C = int(B), int(n), int(C)
        N = n * n + 2 * n
        self.eb, self.pb = eb, pb
        self.x = max(B, 0) * n * C * eb       # X_t, X_next
        self.f = max(B, 0) * C * eb           # F_out, F_pre
        self.phi = n * C * N * pb
        self.coef = max(B, 0) * N * 4         # logits, H
        self.r = max(B, 0) * 4
        self.nb = n * 4                       # b_pre, b_post
        self.nr = n * n * 4                   # b_res
        if B <= 0:  # B == 0 touches nothing (and B < 0 is the library's error to report)
            self.x = self.f = self.phi = self.coef = self.r = self.nb = self.nr = 0


def _coeff_args(z, phi, b_pre, b_post, b_res, logits, r, H):
    return (_ptr(phi, z.phi, z.pb, "phi"), _ptr(b_pre, z.nb, 4, "b_pre"), _ptr(b_post, z.nb, 4, "b_post"),
            _ptr(b_res, z.nr, 4, "b_res"), _ptr(logits, z.coef, 4, "logits"), _ptr(r, z.r, 4, "r"),
            _ptr(H, z.coef, 4, "H"))


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


def mhc_tuning_set(name, value):
    """Override a route or launch-shape choice process-wide (tests and tuning;
    value < 0 restores the default).  See include/mhc.h."""
    _check(load().mhc_tuning_set(str(name).encode(), int(value)), f"mhc_tuning_set({name})")


def mhc_tuning_reset():
    """Restore every route and launch-shape choice to its default."""
    load().mhc_tuning_reset()


def _ws_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return int(workspace_bytes)
    return workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0


def mhc_coeffs_workspace_size(B, n, C):
    return int(load().mhc_coeffs_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_split_k(B, n, C):
    return int(load().mhc_coeffs_split_k(int(B), int(n), int(C)))


def _coeffs(fn, name, eb, pb, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
            b_res, logits, r, H, workspace, workspace_bytes, stream, check):
    z = _Sizes(B, n, C, eb, pb)
    pp, bp, bq, br, lg, rr, hh = _coeff_args(z, phi, b_pre, b_post, b_res, logits, r, H)
    wb = _ws_bytes(workspace, workspace_bytes)
    st = fn(int(B), int(n), int(C), _ptr(X_t, z.x, eb, "X_t"), pp, float(alpha_pre), float(alpha_post),
            float(alpha_res), bp, bq, br, lg, rr, hh, _ptr(workspace, wb, None, "workspace"), wb,
            _stream(stream))
    if check:
        _check(st, name)
    return st


def mhc_coeffs(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
               logits, r, H, workspace, workspace_bytes=None, stream=None, check=True):
    """Steps (1)-(3): logits, r and H from X_t and phi (see include/mhc.h)."""
    return _coeffs(load().mhc_coeffs, "mhc_coeffs", 2, 2, B, n, C, X_t, phi, alpha_pre, alpha_post,
                   alpha_res, b_pre, b_post, b_res, logits, r, H, workspace, workspace_bytes, stream, check)


def _coeffs_pre(fn, name, eb, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                b_res, logits, r, H, F_pre, workspace, workspace_bytes, stream, check):
    z = _Sizes(B, n, C, eb, 2)
    pp, bp, bq, br, lg, rr, hh = _coeff_args(z, phi, b_pre, b_post, b_res, logits, r, H)
    wb = _ws_bytes(workspace, workspace_bytes)
    st = fn(int(B), int(n), int(C), _ptr(X_t, z.x, eb, "X_t"), pp, float(alpha_pre), float(alpha_post),
            float(alpha_res), bp, bq, br, lg, rr, hh, _ptr(F_pre, z.f, eb, "F_pre"),
            _ptr(workspace, wb, None, "workspace"), wb, _stream(stream))
    if check:
        _check(st, name)
    return st


def mhc_coeffs_pre_workspace_size(B, n, C):
    return int(load().mhc_coeffs_pre_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_pre_one_pass(B, n, C):
    return bool(load().mhc_coeffs_pre_one_pass(int(B), int(n), int(C)))


def mhc_coeffs_pre(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                   logits, r, H, F_pre, workspace, workspace_bytes=None, stream=None, check=True):
    """Steps (1)-(3) and (4a) of one layer: logits, r, H and F_pre from X_t, in
    one pass where the shape allows (see include/mhc.h)."""
    return _coeffs_pre(load().mhc_coeffs_pre, "mhc_coeffs_pre", 2, B, n, C, X_t, phi, alpha_pre,
                       alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, F_pre, workspace,
                       workspace_bytes, stream, check)


def mhc_coeffs_pre_check(B, n, C, workspace, fp8=False, workspace_bytes=None, stream=None):
    """Status of the last one-pass mhc_coeffs_pre(_fp8) call of shape (B, n, C)
    on `workspace`: MHC_OK, or MHC_ERR_INCOMPLETE if one of its waits gave up
    (synchronises the stream).  Returns the status, never raises on it."""
    wb = _ws_bytes(workspace, workspace_bytes)
    return int(load().mhc_coeffs_pre_check(int(B), int(n), int(C), 1 if fp8 else 0,
                                            _ptr(workspace, wb, None, "workspace"), wb, _stream(stream)))


def mhc_coeffs_pre_fp8_workspace_size(B, n, C):
    return int(load().mhc_coeffs_pre_fp8_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_pre_fp8_one_pass(B, n, C):
    return bool(load().mhc_coeffs_pre_fp8_one_pass(int(B), int(n), int(C)))


def mhc_coeffs_pre_fp8(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                       logits, r, H, F_pre, workspace, workspace_bytes=None, stream=None, check=True):
    """mhc_coeffs_pre on an E4M3 X_t (see include/mhc.h)."""
    return _coeffs_pre(load().mhc_coeffs_pre_fp8, "mhc_coeffs_pre_fp8", 1, B, n, C, X_t, phi,
                       alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, F_pre,
                       workspace, workspace_bytes, stream, check)


def _pre(fn, name, eb, B, n, C, X_t, H, F_pre, stream, check):
    z = _Sizes(B, n, C, eb)
    st = fn(int(B), int(n), int(C), _ptr(X_t, z.x, eb, "X_t"), _ptr(H, z.coef, 4, "H"),
            _ptr(F_pre, z.f, eb, "F_pre"), _stream(stream))
    if check:
        _check(st, name)
    return st


def mhc_pre(B, n, C, X_t, H, F_pre, stream=None, check=True):
    """Step (4a): F_pre = sum_i H_pre[i] X_t[i] (see include/mhc.h)."""
    return _pre(load().mhc_pre, "mhc_pre", 2, B, n, C, X_t, H, F_pre, stream, check)


def _post_res(fn, name, eb, B, n, C, X_t, F_out, H, X_next, stream, check):
    z = _Sizes(B, n, C, eb)
    st = fn(int(B), int(n), int(C), _ptr(X_t, z.x, eb, "X_t"), _ptr(F_out, z.f, eb, "F_out"),
            _ptr(H, z.coef, 4, "H"), _ptr(X_next, z.x, eb, "X_next"), _stream(stream))
    if check:
        _check(st, name)
    return st


def mhc_post_res(B, n, C, X_t, F_out, H, X_next, stream=None, check=True):
    """Step (4b): X_next = H_res X_t + H_post^T F_out (see include/mhc.h)."""
    return _post_res(load().mhc_post_res, "mhc_post_res", 2, B, n, C, X_t, F_out, H, X_next, stream, check)


def _fused(fn, name, eb, pb, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
           alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next, F_pre_next, workspace,
           workspace_bytes, stream, check, with_pre):
    z = _Sizes(B, n, C, eb, pb)
    pp, bp, bq, br, lg, rr, hh = _coeff_args(z, phi_next, b_pre, b_post, b_res, logits_next, r_next, H_next)
    wb = _ws_bytes(workspace, workspace_bytes)
    args = [int(B), int(n), int(C), _ptr(X_t, z.x, eb, "X_t"), _ptr(F_out, z.f, eb, "F_out"),
            _ptr(H, z.coef, 4, "H"), _ptr(X_next, z.x, eb, "X_next"), pp, float(alpha_pre),
            float(alpha_post), float(alpha_res), bp, bq, br, lg, rr, hh]
    if with_pre:
        args.append(_ptr(F_pre_next, z.f, eb, "F_pre_next"))
    args += [_ptr(workspace, wb, None, "workspace"), wb, _stream(stream)]
    st = fn(*args)
    if check:
        _check(st, name)
    return st


def mhc_post_res_coeffs_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                        alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next, workspace,
                        workspace_bytes=None, stream=None, check=True):
    """Step (4b) of this layer fused with steps (1)-(3) of the next (see include/mhc.h)."""
    return _fused(load().mhc_post_res_coeffs, "mhc_post_res_coeffs", 2, 2, B, n, C, X_t, F_out, H,
                  X_next, phi_next, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                  logits_next, r_next, H_next, None, workspace, workspace_bytes, stream, check, False)


def mhc_post_res_coeffs_pre_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_pre_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre_one_pass(B, n, C):
    return bool(load().mhc_post_res_coeffs_pre_one_pass(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                            alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                            F_pre_next, workspace, workspace_bytes=None, stream=None, check=True):
    """Step (4b) of this layer, then steps (1)-(3) and (4a) of the next, in
    one pass where the shape allows (see include/mhc.h)."""
    return _fused(load().mhc_post_res_coeffs_pre, "mhc_post_res_coeffs_pre", 2, 2, B, n, C, X_t,
                  F_out, H, X_next, phi_next, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                  logits_next, r_next, H_next, F_pre_next, workspace, workspace_bytes, stream, check,
                  True)


def mhc_post_res_coeffs_pre_noalloc(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre,
                                    alpha_post, alpha_res, b_pre, b_post, b_res, logits_next,
                                    r_next, H_next, F_pre_next, stream=None, check=True):
    """mhc_post_res_coeffs_pre with its workspace in the library's own device
    array (no allocation; see include/mhc.h)."""
    z = _Sizes(B, n, C, 2, 2)
    pp, bp, bq, br, lg, rr, hh = _coeff_args(z, phi_next, b_pre, b_post, b_res, logits_next, r_next, H_next)
    st = load().mhc_post_res_coeffs_pre_noalloc(
        int(B), int(n), int(C), _ptr(X_t, z.x, 2, "X_t"), _ptr(F_out, z.f, 2, "F_out"),
        _ptr(H, z.coef, 4, "H"), _ptr(X_next, z.x, 2, "X_next"), pp, float(alpha_pre),
        float(alpha_post), float(alpha_res), bp, bq, br, lg, rr, hh,
        _ptr(F_pre_next, z.f, 2, "F_pre_next"), _stream(stream))
    if check:
        _check(st, "mhc_post_res_coeffs_pre_noalloc")
    return st


def mhc_post_res_coeffs_pre_check(B, n, C, workspace, fp8=False, workspace_bytes=None, stream=None):
    """Status of the last one-pass call of shape (B, n, C) on `workspace`:
    MHC_OK, or MHC_ERR_INCOMPLETE if one of its waits gave up (synchronises
    the stream; see include/mhc.h).  Returns the status, never raises on it."""
    wb = _ws_bytes(workspace, workspace_bytes)
    return int(load().mhc_post_res_coeffs_pre_check(int(B), int(n), int(C), 1 if fp8 else 0,
                                                     _ptr(workspace, wb, None, "workspace"), wb,
                                                     _stream(stream)))


def mhc_post_res_coeffs_pre_fp8_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_pre_fp8_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre_fp8_one_pass(B, n, C):
    return bool(load().mhc_post_res_coeffs_pre_fp8_one_pass(int(B), int(n), int(C)))


def mhc_post_res_coeffs_pre_fp8(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                                alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                                F_pre_next, workspace, workspace_bytes=None, stream=None,
                                check=True):
    """mhc_post_res_coeffs_pre on the E4M3 residual stream (see include/mhc.h)."""
    return _fused(load().mhc_post_res_coeffs_pre_fp8, "mhc_post_res_coeffs_pre_fp8", 1, 2, B, n, C,
                  X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                  b_res, logits_next, r_next, H_next, F_pre_next, workspace, workspace_bytes, stream,
                  check, True)


# FP8 (E4M3) residual-stream variant: same arguments, with X_t, F_out, F_pre
# and X_next as E4M3 tensors (torch.float8_e4m3fn or raw uint8 codes).

def mhc_coeffs_fp8_workspace_size(B, n, C):
    return int(load().mhc_coeffs_fp8_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_fp8(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                   logits, r, H, workspace, workspace_bytes=None, stream=None, check=True):
    """Steps (1)-(3) on an E4M3 X_t (see include/mhc.h)."""
    return _coeffs(load().mhc_coeffs_fp8, "mhc_coeffs_fp8", 1, 2, B, n, C, X_t, phi, alpha_pre,
                   alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, workspace,
                   workspace_bytes, stream, check)


def mhc_pre_fp8(B, n, C, X_t, H, F_pre, stream=None, check=True):
    """Step (4a) on the E4M3 residual stream (see include/mhc.h)."""
    return _pre(load().mhc_pre_fp8, "mhc_pre_fp8", 1, B, n, C, X_t, H, F_pre, stream, check)


def mhc_post_res_fp8(B, n, C, X_t, F_out, H, X_next, stream=None, check=True):
    """Step (4b) on the E4M3 residual stream (see include/mhc.h)."""
    return _post_res(load().mhc_post_res_fp8, "mhc_post_res_fp8", 1, B, n, C, X_t, F_out, H, X_next,
                     stream, check)


def mhc_post_res_coeffs_fp8_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_fp8_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_fp8(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                            alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                            workspace, workspace_bytes=None, stream=None, check=True):
    """mhc_post_res_coeffs on the E4M3 residual stream (see include/mhc.h)."""
    return _fused(load().mhc_post_res_coeffs_fp8, "mhc_post_res_coeffs_fp8", 1, 2, B, n, C, X_t, F_out,
                  H, X_next, phi_next, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                  logits_next, r_next, H_next, None, workspace, workspace_bytes, stream, check, False)


def mhc_coeffs_phi32_workspace_size(B, n, C):
    return int(load().mhc_coeffs_phi32_workspace_size(int(B), int(n), int(C)))


def mhc_coeffs_phi32(B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                     logits, r, H, workspace, workspace_bytes=None, stream=None, check=True):
    """Steps (1)-(3) with an fp32 phi (see include/mhc.h)."""
    return _coeffs(load().mhc_coeffs_phi32, "mhc_coeffs_phi32", 2, 4, B, n, C, X_t, phi, alpha_pre,
                   alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, workspace,
                   workspace_bytes, stream, check)


def mhc_post_res_coeffs_phi32_workspace_size(B, n, C):
    return int(load().mhc_post_res_coeffs_phi32_workspace_size(int(B), int(n), int(C)))


def mhc_post_res_coeffs_phi32(B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                              alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                              workspace, workspace_bytes=None, stream=None, check=True):
    """mhc_post_res_coeffs with an fp32 phi_next (see include/mhc.h)."""
    return _fused(load().mhc_post_res_coeffs_phi32, "mhc_post_res_coeffs_phi32", 2, 4, B, n, C, X_t,
                  F_out, H, X_next, phi_next, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                  logits_next, r_next, H_next, None, workspace, workspace_bytes, stream, check, False)


def mhc_lazy_prenorm_gemm(M, N, K, A, W, C, rstd=None, eps=1e-5, stream=None, check=True):
    """C = rmsnorm(A) @ W^T (A bf16 [M, K], W bf16 [N, K], C bf16 [M, N]); rstd
    fp32 [M] if given (see include/mhc.h)."""
    M, N, K = int(M), int(N), int(K)
    m = max(M, 0)
    st = load().mhc_lazy_prenorm_gemm(M, N, K, _ptr(A, m * K * 2, 2, "A"), _ptr(W, max(N, 0) * K * 2, 2, "W"),
                                      float(eps), _ptr(C, m * max(N, 0) * 2, 2, "C"),
                                      _ptr(rstd, m * 4, 4, "rstd"), _stream(stream))
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
