"""The patch kernel (the workgroup's source patch in LDS, plan kernel 6)
against the fp64 oracle, through the C ABI: exact on integer data, within
max_rel / rms_scaled on Gaussian data.

fprop cases cover the lattice reading of strides and dilations
(gcd(stride, dil) > 1 on an axis, and 1), asymmetric strides, dilations and
padding, ragged last row and column tiles, several channel counts per
16-channel step (1, 3, 4, 6 steps per tap), the three output-channel block
widths (32, 64, 96) and patches that limit the tile's row count.  dgrad cases
(stride dividing dilation) cover stride 1 with and without dilation, stride 2
and 3 with the dx rows and columns off the lattice (which the kernel writes
as zeros: dx is pre-filled with NaN), a lattice that starts at row 1, and
asymmetric filters."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import check, f64, oracle_fprop_out, run_dgrad, run_fprop

pytestmark = pytest.mark.gpu

PATCH_KERNEL = 6


def patch_tile(prob, dtype, op=B.CONV2D_OP_FPROP):
    """1-based algo tile of the patch kernel in the pass's table."""
    info = B.conv2d_plan_info(op, prob, dtype)
    tiles = [t for t in range(1, info["num_tiles"] + 1)
             if B.conv2d_plan_info(op, prob, dtype, algo=dict(tile=t))["kernel"] == PATCH_KERNEL]
    assert len(tiles) == 1, tiles
    return tiles[0]


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


DGRAD_CASES = [
    # (id, problem, dtype, dist)
    ("dg_s2d2_5x5", problem(2, 32, 23, 25, 96, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)), "f16", "int"),
    ("dg_s1_5x5", problem(2, 64, 17, 19, 64, 5, 5, pad=(2, 2)), "bf16", "int"),
    ("dg_s1_d2", problem(2, 32, 15, 16, 32, 3, 3, pad=(2, 2), dil=(2, 2)), "f16", "int"),
    ("dg_s2d4_pad3", problem(2, 32, 21, 22, 32, 3, 3, pad=(3, 3), stride=(2, 2), dil=(4, 4)), "f16", "int"),
    ("dg_asym_s3", problem(1, 64, 20, 25, 48, 2, 3, pad=(1, 2), stride=(3, 1), dil=(3, 2)), "f16", "int"),
    ("dg_even_hw", problem(3, 96, 16, 18, 64, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)), "bf16", "int"),
    ("dg_gauss_s2d2", problem(4, 96, 25, 25, 192, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)), "bf16", "gauss"),
    ("dg_gauss_s1", problem(2, 128, 20, 21, 96, 3, 3, pad=(1, 1)), "f16", "gauss"),
]


@pytest.mark.parametrize("cid,prob,dtype,dist", DGRAD_CASES, ids=[c[0] for c in DGRAD_CASES])
def test_patch_dgrad(cid, prob, dtype, dist):
    P, Q = oracle.output_hw(prob)
    _, w, _, dy = WL.random_case(prob, dtype, dist, zlib_seed(cid), P, Q, bias=False)
    ref = oracle.dgrad(prob, f64(dy), f64(w))
    dx = run_dgrad(prob, dtype, dy, w, algo=dict(tile=patch_tile(prob, dtype, B.CONV2D_OP_DGRAD)),
                   fill=float("nan"))
    check(f64(dx), ref, dtype, "exact" if dist == "int" else "tol", cid)


def test_patch_dgrad_refused_where_stride_does_not_divide_dilation():
    """Stride 2 with dilation 1 leaves dx rows of both parities with taps:
    the dgrad table has no patch kernel; fprop still has it."""
    prob = problem(2, 64, 28, 28, 128, 3, 3, pad=(1, 1), stride=(2, 2))
    n = B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, "f16")["num_tiles"]
    assert all(B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, "f16", algo=dict(tile=t))["kernel"] != PATCH_KERNEL
               for t in range(1, n + 1))
    patch_tile(prob, "f16")
