"""MI355X (gfx950) implicit-GEMM NHWC conv2d: fprop, dgrad and wgrad.

The computation runs in hand-written HIP kernels behind the C ABI declared in
include/conv2d_nhwc.h (libconv2d_nhwc.so, built by
``python -m convolution_nhwc_implicit_amd.build``).  This package is the thin
ctypes binding to it; PyTorch provides device memory and streams.
"""
from .binding import (  # noqa: F401
    CONV2D_DTYPE_BF16, CONV2D_DTYPE_F16, CONV2D_DTYPE_I8, CONV2D_OP_DGRAD, CONV2D_OP_FPROP,
    CONV2D_OP_WGRAD, Conv2dError, conv2d_dgrad, conv2d_fprop, conv2d_output_size,
    conv2d_plan_info, conv2d_status_string, conv2d_wgrad, conv2d_workspace_size, dgrad, fprop,
    load, problem_from, wgrad, workspace_for,
)
