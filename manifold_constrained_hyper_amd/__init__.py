"""MI355X-native mHC (manifold-constrained hyper-connections) residual-stream
forward: HIP kernels for gfx950 behind the C ABI of include/mhc.h, with a thin
ctypes binding.  See binding.py for the Python entry points."""

from .binding import (  # noqa: F401
    MHC_OK, MHC_ERR_INVALID_ARG, MHC_ERR_UNSUPPORTED, MHC_ERR_WORKSPACE, MHC_ERR_HIP,
    MHC_ERR_INCOMPLETE, MHC_SINKHORN_ITERS, mhc_tuning_set, mhc_tuning_reset,
    mhc_post_res_coeffs_pre_check, mhc_post_res_coeffs_pre_noalloc, MHC_NOALLOC_SCRATCH_BYTES, MhcError, LIB_PATH, EXPORTED, load, alloc_outputs,
    mhc_status_string, mhc_coeffs_workspace_size, mhc_coeffs_split_k,
    mhc_coeffs, mhc_pre, mhc_post_res, mhc_post_res_coeffs_workspace_size, mhc_post_res_coeffs,
    mhc_coeffs_fp8_workspace_size, mhc_coeffs_fp8, mhc_pre_fp8, mhc_post_res_fp8,
    mhc_post_res_coeffs_fp8_workspace_size, mhc_post_res_coeffs_fp8, mhc_lazy_prenorm_gemm,
    mhc_coeffs_phi32_workspace_size, mhc_coeffs_phi32, mhc_post_res_coeffs_phi32_workspace_size,
    mhc_post_res_coeffs_phi32, mhc_post_res_coeffs_pre_workspace_size, mhc_post_res_coeffs_pre,
    mhc_post_res_coeffs_pre_one_pass, mhc_post_res_coeffs_pre_fp8_workspace_size,
    mhc_post_res_coeffs_pre_fp8, mhc_post_res_coeffs_pre_fp8_one_pass,
    mhc_coeffs_pre_workspace_size, mhc_coeffs_pre, mhc_coeffs_pre_one_pass, mhc_coeffs_pre_check,
    mhc_coeffs_pre_fp8_workspace_size, mhc_coeffs_pre_fp8, mhc_coeffs_pre_fp8_one_pass,
)
