"""The patch kernel (fprop with the workgroup's input patch in LDS, plan
kernel 6) against the fp64 oracle, through the C ABI: exact on integer data,
within max_rel / rms_scaled on Gaussian data.  The cases cover the lattice
reading of strides and dilations (gcd(stride, dil) > 1 on an axis, and 1),
asymmetric strides, dilations and padding, ragged last row and column tiles,
several channel counts per 16-channel step (1, 3, 4, 6 steps per tap), the
three output-channel block widths (32, 64, 96) and patches that limit the
tile's row count."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import check, f64, oracle_fprop_out, run_fprop

pytestmark = pytest.mark.gpu

PATCH_KERNEL = 6


def patch_tile(prob, dtype):
    """1-based algo tile of the patch kernel (the last tile of the table)."""
    info = B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, dtype)
    t = info["num_tiles"]
    assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, dtype, algo=dict(tile=t))["kernel"] == PATCH_KERNEL
    return t


CASES = [
    # (id, problem, dtype, dist, bias, relu)
    ("s2d2_5x5_k96", problem(2, 32, 23, 25, 96, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)), "f16", "int", True, False),
    ("s2d2_5x5_k64_bf16", problem(3, 48, 21, 19, 64, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)), "bf16", "int", True, True),
    ("s2_3x3_k32", problem(2, 64, 28, 28, 32, 3, 3, pad=(1, 1), stride=(2, 2)), "f16", "int", False, True),
    ("s1_3x3_c16", problem(2, 16, 17, 15, 96, 3, 3, pad=(1, 1)), "f16", "int", True, True),
    ("asym", problem(2, 48, 19, 23, 64, 3, 2, pad=(1, 0), stride=(2, 1), dil=(1, 2)), "f16", "int", True, False),
    ("s3_d2", problem(2, 32, 26, 29, 32, 3, 3, pad=(2, 1), stride=(3, 3), dil=(2, 2)), "bf16", "int", False, False),
    ("s2_d4", problem(1, 32, 30, 33, 64, 3, 3, pad=(4, 4), stride=(2, 2), dil=(4, 4)), "f16", "int", True, False),
    ("wide_row", problem(2, 32, 5, 150, 32, 1, 3, pad=(0, 1)), "f16", "int", True, True),
    ("wide_c256", problem(1, 256, 12, 40, 64, 3, 3, pad=(1, 1)), "f16", "int", True, False),
    ("one_by_one_s2", problem(2, 64, 15, 17, 96, 1, 1, stride=(2, 2)), "bf16", "int", True, False),
    ("pad_gt_filter", problem(2, 16, 7, 9, 32, 3, 3, pad=(3, 2)), "f16", "int", True, False),
    ("p_is_1", problem(3, 32, 3, 3, 64, 3, 3), "f16", "int", True, True),
    ("gauss_s2d2", problem(4, 96, 25, 25, 192, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)), "bf16", "gauss", True, False),
    ("gauss_s1", problem(2, 64, 30, 30, 128, 3, 3, pad=(1, 1)), "f16", "gauss", True, True),
]


@pytest.mark.parametrize("cid,prob,dtype,dist,bias,relu", CASES, ids=[c[0] for c in CASES])
def test_patch_fprop(cid, prob, dtype, dist, bias, relu):
    P, Q = oracle.output_hw(prob)
    x, w, b, _ = WL.random_case(prob, dtype, dist, zlib_seed(cid), P, Q, bias=bias)
    ref = oracle.fprop(prob, f64(x), f64(w), bias=None if b is None else f64(b), relu=relu)
    y = run_fprop(prob, dtype, x, w, b, relu, algo=dict(tile=patch_tile(prob, dtype)))
    check(f64(y), ref, dtype, "exact" if dist == "int" else "tol", cid)


def zlib_seed(s):
    import zlib
    return zlib.crc32(s.encode()) & 0x7fffffff


def test_patch_deterministic_and_matches_default_exactly():
    """Two runs give identical bits; on integer data the patch kernel and the
    library's default kernel agree bit for bit."""
    prob = problem(4, 96, 25, 25, 192, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2))
    P, Q = oracle.output_hw(prob)
    x, w, b, _ = WL.random_case(prob, "bf16", "gauss", 7, P, Q, bias=True)
    t = patch_tile(prob, "bf16")
    y1 = run_fprop(prob, "bf16", x, w, b, False, algo=dict(tile=t))
    y2 = run_fprop(prob, "bf16", x, w, b, False, algo=dict(tile=t))
    assert np.array_equal(f64(y1), f64(y2))
    xi, wi, bi, _ = WL.random_case(prob, "f16", "int", 8, P, Q, bias=True)
    ya = run_fprop(prob, "f16", xi, wi, bi, True, algo=dict(tile=t))
    yb = run_fprop(prob, "f16", xi, wi, bi, True, algo=dict(tile=1))
    assert np.array_equal(f64(ya), f64(yb))
