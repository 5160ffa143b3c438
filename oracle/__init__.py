"""fp64 CPU oracle for the mHC residual-stream forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the ``smoke()`` entry of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
call anything in this package.  The HIP library never routes through it and
shares no code with it (no kernels, headers, helpers or constants).

Sources (cited by page title and section throughout):

* [mHC-cutile] -- the blog page "mHC 算法分析 & cutile 高效实现" (edward-lyz,
  2026-02-10), which states the forward computation in its section 2 and shows
  tensor layouts in the kernels of sections 4 and 5.
* [FreeNorm] -- the PyTorch blog "Towards Free Normalization: Fusing
  Normalization into GEMM and Attention Kernels", section 2 (Lazy Pre-Norm),
  used only for the row-scaling identity that lets 1/r be applied after the
  GEMM.
"""

from .mhc_oracle import (  # noqa: F401
    SINKHORN_ITERS,
    bf16_bits_to_f64,
    round_to_bf16,
    coefficient_logits,
    row_sum_squares,
    rms_scale,
    scale_bias,
    sigmoid,
    gate_coefficients,
    sinkhorn_knopp,
    coefficients,
    pre_mix,
    post_res,
    forward,
    split_h,
)

from . import fp8  # noqa: F401,E402  (E4M3 encode / decode for the FP8 variant)
from . import lazy_prenorm  # noqa: F401,E402  (the Lazy Pre-Norm GEMM of [FreeNorm] section 2)
