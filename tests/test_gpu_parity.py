"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and medium problems are compared element by element on every output;
they span several tiles in M, N and GEMM-K and end in ragged tails.  The full
workloads are compared on every output too, in the launch configuration the
benchmark uses (the library's default plan).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import DEV, check, f64, gpu, oracle_fprop_out, run_dgrad, run_fprop, run_wgrad

pytestmark = pytest.mark.gpu


def case_inputs(prob, dtype, dist, seed, bias=True):
    P, Q = oracle.output_hw(prob)
    return WL.random_case(prob, dtype, dist, seed, P, Q, bias=bias)


# (id, problem, dtype, dist, bias, relu)
CASES = [
    ("ragged3x3", problem(3, 24, 17, 19, 40, 3, 3, pad=(1, 1)), "f16", "int", True, False),
    ("ragged3x3_relu", problem(2, 32, 15, 13, 72, 3, 3, pad=(1, 1)), "f16", "int", True, True),
    ("strided_dilated", problem(2, 16, 23, 21, 24, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)),
     "f16", "int", False, False),
    ("asym", problem(2, 8, 11, 14, 16, 3, 2, pad=(1, 0), stride=(2, 1), dil=(1, 2)), "f16", "int",
     True, False),
    ("stride3", problem(2, 16, 13, 10, 8, 2, 2, pad=(0, 1), stride=(3, 3)), "f16", "int", False,
     False),
    ("pad_gt_filter", problem(2, 8, 6, 7, 16, 3, 3, pad=(3, 2)), "f16", "int", True, False),
    ("one_by_one", problem(2, 32, 9, 13, 48, 1, 1), "f16", "int", True, True),
    ("one_by_one_s2", problem(2, 16, 9, 13, 24, 1, 1, stride=(2, 2)), "f16", "int", False, False),
    ("tiny_image", problem(3, 8, 1, 1, 8, 1, 1), "f16", "int", True, False),
    ("p_is_1", problem(2, 16, 3, 3, 16, 3, 3), "f16", "int", True, False),
    ("wide_c", problem(1, 256, 7, 6, 32, 3, 3, pad=(1, 1)), "f16", "int", True, False),
    ("bf16_int", problem(2, 24, 12, 11, 40, 3, 3, pad=(1, 1), stride=(2, 1)), "bf16", "int", True,
     True),
    ("bf16_gauss", problem(3, 32, 16, 17, 64, 3, 3, pad=(1, 1)), "bf16", "gauss", True, True),
    ("f16_gauss", problem(2, 64, 20, 18, 136, 3, 3, pad=(1, 1)), "f16", "gauss", True, True),
    ("f16_gauss_s2d2", problem(2, 48, 25, 23, 56, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)),
     "f16", "gauss", False, False),
    ("grouped2", problem(2, 12, 9, 10, 8, 3, 3, pad=(1, 1), groups=2), "bf16", "int", True, True),
    ("grouped4_s2d2", problem(2, 16, 13, 13, 8, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2),
                              groups=4), "f16", "int", False, False),
    ("depthwise", problem(2, 8, 10, 9, 8, 3, 3, pad=(1, 1), groups=8), "f16", "int", True, False),
    # depthwise kernels (groups = C = K, C % 8 == 0): strides and dilation,
    # a ragged last column strip, 24 channels (three 8-channel vectors), 1x3
    ("dw_s2d2", problem(2, 16, 13, 11, 16, 3, 3, pad=(2, 2), stride=(2, 2), dil=(2, 2), groups=16),
     "f16", "int", True, True),
    ("dw_bf16_gauss", problem(3, 32, 15, 17, 32, 3, 3, pad=(1, 1), groups=32), "bf16", "gauss", True, False),
    ("dw_c24_1x3", problem(2, 24, 9, 14, 24, 1, 3, pad=(0, 1), stride=(1, 2), groups=24), "f16", "int",
     False, False),
    ("dw_5x5_fallback", problem(2, 8, 9, 9, 8, 5, 5, pad=(2, 2), groups=8), "f16", "int", True, False),
    # depthwise row kernels (unit column stride and dilation, R, S <= 3):
    # a 3x2 filter with row stride and dilation (dgrad takes the general
    # kernel, stride 2), and a valid 3x3 with row dilation whose stride-1
    # dgrad runs the row kernel with pads (R-1)*dh and S-1; ragged strips
    ("dw_rows_3x2_s21", problem(3, 16, 14, 11, 16, 3, 2, pad=(0, 1), stride=(2, 1), dil=(2, 1), groups=16),
     "f16", "int", True, True),
    ("dw_rows_valid_d2", problem(2, 40, 12, 13, 40, 3, 3, pad=(0, 0), dil=(2, 1), groups=40),
     "bf16", "int", False, False),
    ("dw_rows_2x1_gauss", problem(2, 64, 7, 19, 64, 2, 1, pad=(1, 0), groups=64), "f16", "gauss",
     True, False),
    ("grouped_gauss", problem(2, 24, 11, 11, 24, 3, 3, pad=(1, 1), groups=3), "bf16", "gauss",
     True, False),
    # grouped problems whose channels per group are whole 16-byte vectors
    # (C/G and K/G multiples of 8) run one implicit GEMM per group: strides
    # and dilations, a filter taller than wide
    ("grouped_gemm_s2d2", problem(3, 32, 21, 17, 48, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2),
                                   groups=2), "f16", "int", True, True),
    ("grouped_gemm_asym", problem(2, 48, 13, 21, 48, 3, 2, pad=(1, 0), stride=(1, 2), dil=(2, 1),
                                   groups=3), "bf16", "gauss", True, False),
    ("grouped_gemm_wide", problem(2, 64, 9, 30, 64, 3, 3, pad=(1, 1), groups=2), "f16", "gauss",
     False, False),
    # stride-1 problems with 64 source channels and a 3x3 filter run on the
    # band kernel (filter + ring of input rows in LDS): two column segments,
    # partial N tiles, one-row and multi-group row ranges, padding 0..3
    ("band_two_segments", problem(3, 64, 21, 70, 64, 3, 3, pad=(1, 1)), "f16", "int", True, True),
    ("band_ntail", problem(2, 64, 19, 33, 72, 3, 3, pad=(1, 1)), "bf16", "int", True, False),
    ("band_multigroup", problem(100, 64, 30, 6, 64, 3, 3, pad=(1, 1)), "f16", "int", True, False),
    ("band_pad0", problem(2, 64, 12, 12, 64, 3, 3), "f16", "int", False, False),
    ("band_pad2", problem(2, 64, 9, 9, 64, 3, 3, pad=(2, 2)), "f16", "int", True, False),
    ("band_pad3", problem(2, 64, 8, 8, 64, 3, 3, pad=(3, 3)), "f16", "int", False, False),
    ("band_gauss", problem(8, 64, 28, 28, 64, 3, 3, pad=(1, 1)), "f16", "gauss", True, True),
    ("band_bf16_gauss", problem(4, 64, 17, 23, 64, 3, 3, pad=(1, 1)), "bf16", "gauss", False, False),
    ("band_bf16_relu", problem(3, 64, 13, 40, 64, 3, 3, pad=(1, 1)), "bf16", "int", True, True),
    ("band_one_row", problem(3, 64, 1, 9, 64, 3, 3, pad=(1, 1)), "f16", "int", True, True),
    # wgrad band kernel (stride 1, 3x3, C = K = 64, Q % 4 == 0, Q <= 56):
    # two row groups with a partial last group, and one-row bands whose pixel
    # count is not a multiple of 16; the widest row it takes (Q = 56, several
    # groups per band), and one just past it (Q = 64, generic path)
    ("wband_groups", problem(64, 64, 30, 8, 64, 3, 3, pad=(1, 1)), "f16", "int", False, False),
    ("wband_masked", problem(2, 64, 12, 12, 64, 3, 3, pad=(1, 1)), "f16", "int", False, False),
    ("wband_bf16", problem(16, 64, 20, 20, 64, 3, 3, pad=(1, 1)), "bf16", "gauss", False, False),
    ("wband_q56", problem(2, 64, 23, 56, 64, 3, 3, pad=(1, 1)), "f16", "int", False, False),
    ("wband_wide", problem(4, 64, 9, 64, 64, 3, 3, pad=(1, 1)), "f16", "int", True, True),
    # with at least 8 * 85 output rows over all images the wgrad band kernel
    # splits the columns by filter row over 85 bands of the stacked rows:
    # bands of 8-9 rows across image boundaries, no padding, padding 2, and
    # Gaussian bf16 (the short last groups of 1-3 slots come up per band)
    ("wband3_cross", problem(13, 64, 56, 20, 64, 3, 3, pad=(1, 1)), "f16", "int", False, False),
    ("wband3_pad0", problem(24, 64, 32, 16, 64, 3, 3), "f16", "int", False, False),
    ("wband3_pad2", problem(20, 64, 34, 12, 64, 3, 3, pad=(2, 2)), "f16", "int", False, False),
    ("wband3_bf16", problem(12, 64, 60, 24, 64, 3, 3, pad=(1, 1)), "bf16", "gauss", False, False),
    # 9-row images in bands of 8-9 rows: most bands cross an image boundary;
    # 6-row images in bands of 10-11 rows over two or three images
    ("wband3_short_img", problem(76, 64, 9, 24, 64, 3, 3, pad=(1, 1)), "f16", "int", False, False),
    ("wband3_three_imgs", problem(150, 64, 6, 16, 64, 3, 3, pad=(1, 1)), "f16", "int", False, False),
    # channel counts that are not whole 16-byte vectors run on zero-padded
    # copies: a stem-like C = 3 7x7 stride-2 layer, an odd K, both odd with
    # stride and dilation, and C = 60 whose padded problem takes the band
    # kernels
    ("pad_c3_stem", problem(2, 3, 30, 30, 16, 7, 7, pad=(3, 3), stride=(2, 2)), "f16", "int", True, True),
    ("pad_k13", problem(2, 16, 11, 13, 13, 3, 3, pad=(1, 1)), "bf16", "int", True, False),
    ("pad_both", problem(3, 5, 9, 10, 7, 3, 2, pad=(1, 0), stride=(1, 2), dil=(2, 1)), "f16", "gauss",
     True, True),
    ("pad_c60_band", problem(2, 60, 10, 12, 64, 3, 3, pad=(1, 1)), "f16", "int", True, True),
    # padded problems whose padded copies take the pointwise kernels (1x1,
    # 64 channels) and the patch kernel (dgrad: stride 2 divides dilation 2)
    ("pad_c60_1x1", problem(2, 60, 9, 10, 64, 1, 1), "f16", "int", True, True),
    ("pad_k60_1x1", problem(3, 64, 7, 9, 60, 1, 1), "bf16", "int", True, False),
    ("pad_c29_patch", problem(2, 29, 9, 12, 12, 2, 2, pad=(0, 1), stride=(2, 1), dil=(2, 2)), "f16", "int",
     False, False),
]


@pytest.mark.parametrize("cid,prob,dtype,dist,bias,relu", CASES, ids=[c[0] for c in CASES])
def test_parity_cases(cid, prob, dtype, dist, bias, relu):
    mode = "exact" if dist == "int" else "tol"
    x, w, b, dy = case_inputs(prob, dtype, dist, seed=zlib.crc32(cid.encode()), bias=bias)
    y = run_fprop(prob, dtype, x, w, b, relu)
    check(f64(y), oracle_fprop_out(prob, dtype, x, w, b, relu), dtype, mode, f"{cid} fprop")
    if relu:  # ReLU gives +0, never -0
        assert not bool((y.view(torch.int16) == -32768).any()), f"{cid}: -0 after ReLU"
    dx = run_dgrad(prob, dtype, dy, w, fill=float("nan"))
    check(f64(dx), oracle.dgrad(prob, f64(dy), f64(w)), dtype, mode, f"{cid} dgrad")
    dw = run_wgrad(prob, dtype, x, dy)
    check(f64(dw), oracle.wgrad(prob, f64(x), f64(dy)), dtype, mode, f"{cid} wgrad")


INT8_CASES = [
    ("i8_3x3", problem(2, 32, 11, 13, 48, 3, 3, pad=(1, 1)), True, True),
    ("i8_norelu", problem(2, 16, 9, 9, 32, 3, 3, pad=(1, 1), stride=(2, 2)), True, False),
    ("i8_nobias", problem(1, 64, 8, 7, 16, 1, 1), False, True),
    ("i8_grouped", problem(2, 16, 7, 7, 16, 3, 3, pad=(1, 1), groups=4), True, True),
    ("i8_grouped_gemm", problem(2, 64, 9, 8, 96, 3, 3, pad=(1, 1), stride=(2, 1), groups=2), True, True),
    ("i8_pad_c3", problem(2, 3, 12, 12, 16, 3, 3, pad=(1, 1)), True, True),
    ("i8_pad_k20", problem(2, 32, 9, 8, 20, 3, 3, pad=(1, 1)), True, False),
    # 3x3 stride-1 int8 with 128 channels runs the band kernel: ragged row
    # bands, a K that fills part of a 64-channel slice, two column segments,
    # pads 0 and 2
    ("i8_band", problem(2, 128, 11, 13, 128, 3, 3, pad=(1, 1)), True, True),
    ("i8_band_k48_w70", problem(1, 128, 5, 70, 48, 3, 3, pad=(1, 1)), True, False),
    ("i8_band_pad0_k192", problem(2, 128, 9, 9, 192, 3, 3), False, True),
    ("i8_band_pad2", problem(1, 128, 6, 7, 64, 3, 3, pad=(2, 2)), True, True),
    ("i8_band_two_rows", problem(2, 128, 2, 5, 128, 3, 3, pad=(1, 1)), True, True),
]


@pytest.mark.parametrize("cid,prob,bias,relu", INT8_CASES, ids=[c[0] for c in INT8_CASES])
def test_int8_fprop_exact(cid, prob, bias, relu):
    x, w, b, _ = case_inputs(prob, "i8", "uniform_i8", seed=zlib.crc32(cid.encode()), bias=bias)
    scales = (0.02, 0.01, 0.05)
    y = run_fprop(prob, "i8", x, w, b, relu, scales=scales)
    exp = oracle_fprop_out(prob, "i8", x, w, b, relu, scales=scales)
    got = y.cpu().numpy().reshape(-1)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, f"{bad.size} int8 codes differ, first {bad[:5]}: {got[bad[:5]]} vs {exp[bad[:5]]}"
    if relu:
        assert got.min() >= 0


# ------------------------------------------------------------ tile / split sweeps

def test_int8_every_tile_matches_oracle():
    """Every implicit-GEMM tile and the band kernel give the same int8 codes."""
    prob = problem(2, 128, 10, 12, 64, 3, 3, pad=(1, 1))
    x, w, b, _ = case_inputs(prob, "i8", "uniform_i8", seed=77, bias=True)
    scales = (0.02, 0.01, 0.05)
    exp = oracle_fprop_out(prob, "i8", x, w, b, True, scales=scales)
    info = B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "i8")
    assert info["num_tiles"] == 6 and info["tile"] == 5, info  # the band kernel is the default
    for t in range(1, info["num_tiles"] + 1):
        y = run_fprop(prob, "i8", x, w, b, True, scales=scales, algo=dict(tile=t))
        got = y.cpu().numpy().reshape(-1)
        assert np.array_equal(got, exp), f"tile {t}: {np.count_nonzero(got != exp)} codes differ"


def test_every_fprop_and_dgrad_tile_matches_oracle():
    prob = problem(2, 32, 13, 11, 48, 3, 3, pad=(1, 1), stride=(2, 1))
    x, w, b, dy = case_inputs(prob, "f16", "int", seed=42)
    ref_y = oracle_fprop_out(prob, "f16", x, w, b, True)
    ref_dx = oracle.dgrad(prob, f64(dy), f64(w))
    n = B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16")["num_tiles"]
    for t in range(1, n + 1):
        algo = dict(tile=t)
        check(f64(run_fprop(prob, "f16", x, w, b, True, algo=algo)), ref_y, "f16", "exact", f"tile {t}")
        check(f64(run_dgrad(prob, "f16", dy, w, algo=algo)), ref_dx, "f16", "exact", f"dgrad tile {t}")


@pytest.mark.parametrize("cid,prob,dtype,relayout", [
    # GEMM-K rows of 3200 per stride phase: the filter is re-laid out first
    ("long_k", problem(2, 16, 12, 13, 128, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)), "f16", True),
    # rows of 1152: B read straight from the filter with transposing LDS reads
    ("short_k_grouped", problem(2, 48, 11, 9, 96, 3, 3, pad=(1, 1), stride=(2, 2), groups=2), "bf16", False),
], ids=["long_k", "short_k_grouped"])
def test_dgrad_filter_paths_every_tile(cid, prob, dtype, relayout):
    """The implicit-GEMM dgrad with the filter re-laid out (a workspace) and
    read as it is (none), every tile, integer data: exact."""
    _, w, _, dy = case_inputs(prob, dtype, "int", seed=zlib.crc32(cid.encode()), bias=False)
    ref = oracle.dgrad(prob, f64(dy), f64(w))
    info = B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, dtype)
    assert info["kernel"] == 1 and (info["workspace_bytes"] > 0) == relayout, info
    for t in range(1, info["num_tiles"] + 1):
        dx = run_dgrad(prob, dtype, dy, w, algo=dict(tile=t), fill=float("nan"))
        check(f64(dx), ref, dtype, "exact", f"{cid} dgrad tile {t}")


# 1x1 stride-1 problems without padding run the pointwise kernel (kernel 5):
# GEMM-K 64, 128 and 256, 64 to 256 output channels per workgroup, pixel
# counts that end in a partial sub-tile and a partial workgroup
POINTWISE = [
    ("pw_64_256", problem(3, 64, 9, 13, 256, 1, 1), "f16", "int", True, True),
    ("pw_128_128", problem(2, 128, 17, 11, 128, 1, 1), "bf16", "int", True, False),
    ("pw_256_64", problem(2, 256, 7, 19, 64, 1, 1), "f16", "int", False, True),
    ("pw_64_192", problem(4, 64, 15, 15, 192, 1, 1), "bf16", "gauss", True, True),
    ("pw_128_512", problem(2, 128, 5, 23, 512, 1, 1), "f16", "gauss", True, False),
    ("pw_dil", problem(2, 64, 10, 10, 64, 1, 1, dil=(2, 2)), "f16", "int", True, True),
]


@pytest.mark.parametrize("cid,prob,dtype,dist,bias,relu", POINTWISE, ids=[c[0] for c in POINTWISE])
def test_pointwise(cid, prob, dtype, dist, bias, relu):
    mode = "exact" if dist == "int" else "tol"
    x, w, b, dy = case_inputs(prob, dtype, dist, seed=zlib.crc32(cid.encode()), bias=bias)
    fi = B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, dtype)
    di = B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, dtype)
    fp_pw, dg_pw = fi["kernel"] == 5, di["kernel"] == 5
    assert fp_pw and fi["workspace_bytes"] == 0, fi
    ref_y = oracle_fprop_out(prob, dtype, x, w, b, relu)
    y = run_fprop(prob, dtype, x, w, b, relu)
    check(f64(y), ref_y, dtype, mode, f"{cid} pointwise fprop")
    if relu:
        assert not bool((y.view(torch.int16) == -32768).any()), f"{cid}: -0 after ReLU"
    check(f64(run_fprop(prob, dtype, x, w, b, relu, algo=dict(tile=1))), ref_y, dtype, mode, f"{cid} tile 1")
    ref_dx = oracle.dgrad(prob, f64(dy), f64(w))
    if dg_pw:
        assert di["workspace_bytes"] == 0, di
    dx = run_dgrad(prob, dtype, dy, w, fill=float("nan"))
    check(f64(dx), ref_dx, dtype, mode, f"{cid} pointwise dgrad")
    check(f64(run_dgrad(prob, dtype, dy, w, algo=dict(tile=3))), ref_dx, dtype, mode, f"{cid} dgrad tile 3")


def test_pointwise_plans():
    """Which 1x1 problems the pointwise kernel takes."""
    on = [(64, 256), (256, 64), (128, 128), (64, 64), (128, 512)]
    for c, k in on:
        prob = problem(2, c, 8, 8, k, 1, 1)
        assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16")["kernel"] == 5, (c, k)
    for prob in (problem(2, 64, 8, 8, 256, 1, 1, pad=(1, 1)), problem(2, 64, 8, 8, 256, 1, 1, stride=(2, 2)),
                 problem(2, 32, 8, 8, 256, 1, 1), problem(2, 64, 8, 8, 96, 1, 1),
                 problem(2, 64, 8, 8, 256, 1, 1, groups=2)):
        assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16")["kernel"] != 5, prob
    assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, problem(2, 64, 8, 8, 256, 1, 1), "i8")["kernel"] != 5


# The pointwise wgrad kernel (1x1 stride 1, K and C in {64, 128, 256}, K*C <=
# 16384): every wave layout (one, two and four pixel phases), pixel counts
# that end inside a 64-pixel group, and split counts from one slice to more
# slices than groups (empty slices write zero partials).
PW_WGRAD = [
    ("pww_c64_k256", problem(3, 64, 9, 13, 256, 1, 1), "f16", "int"),
    ("pww_c256_k64", problem(2, 256, 7, 19, 64, 1, 1), "bf16", "int"),
    ("pww_c128_k128", problem(2, 128, 17, 11, 128, 1, 1), "f16", "int"),
    ("pww_c64_k128", problem(2, 64, 11, 9, 128, 1, 1), "bf16", "int"),
    ("pww_c128_k64", problem(2, 128, 9, 9, 64, 1, 1), "f16", "int"),
    ("pww_c64_k64", problem(3, 64, 10, 10, 64, 1, 1), "f16", "int"),
    ("pww_gauss", problem(4, 64, 15, 15, 256, 1, 1), "bf16", "gauss"),
    ("pww_dil_gauss", problem(2, 64, 10, 10, 64, 1, 1, dil=(2, 2)), "f16", "gauss"),
]


@pytest.mark.parametrize("cid,prob,dtype,dist", PW_WGRAD, ids=[c[0] for c in PW_WGRAD])
def test_pointwise_wgrad(cid, prob, dtype, dist):
    info = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, dtype)
    assert info["kernel"] == 5 and info["tile"] == 2, info
    mode = "exact" if dist == "int" else "tol"
    x, _, _, dy = case_inputs(prob, dtype, dist, seed=zlib.crc32(cid.encode()), bias=False)
    ref = oracle.wgrad(prob, f64(x), f64(dy))
    dw = run_wgrad(prob, dtype, x, dy)
    check(f64(dw), ref, dtype, mode, f"{cid} pointwise wgrad")
    again = run_wgrad(prob, dtype, x, dy)
    assert torch.equal(again.view(torch.int16), dw.view(torch.int16)), f"{cid}: repeat differs"
    groups = (prob["N"] * prob["H"] * prob["W"] + 63) // 64
    for s in (1, 3, groups + 5):
        check(f64(run_wgrad(prob, dtype, x, dy, algo=dict(tile=3, split_k=s))), ref, dtype, mode,
              f"{cid} split {s}")
    check(f64(run_wgrad(prob, dtype, x, dy, algo=dict(tile=1))), ref, dtype, mode, f"{cid} generic tile 1")


def test_every_tile_on_band_eligible_problem():
    prob = problem(3, 64, 14, 13, 64, 3, 3, pad=(1, 1))
    x, w, b, dy = case_inputs(prob, "f16", "int", seed=48)
    ref_y = oracle_fprop_out(prob, "f16", x, w, b, False)
    ref_dx = oracle.dgrad(prob, f64(dy), f64(w))
    info = B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16")
    # the band kernel is the default; tile 7 is Winograd F(2x2,3x3), exact
    # here because the transformed integer operands are exact in fp16, and
    # the last fprop tile the patch kernel
    assert info["num_tiles"] == 8 and info["tile"] == 5
    assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16", algo=dict(tile=7))["kernel"] == 3
    assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16", algo=dict(tile=8))["kernel"] == 6
    dinfo = B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, "f16")
    assert dinfo["num_tiles"] == 8 and dinfo["tile"] == 5  # dgrad: Winograd too, then the patch kernel
    assert B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, "f16", algo=dict(tile=7))["kernel"] == 3
    assert B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, "f16", algo=dict(tile=8))["kernel"] == 6
    for t in range(1, info["num_tiles"] + 1):
        check(f64(run_fprop(prob, "f16", x, w, b, False, algo=dict(tile=t))), ref_y, "f16", "exact", f"tile {t}")
    for t in range(1, dinfo["num_tiles"] + 1):
        check(f64(run_dgrad(prob, "f16", dy, w, algo=dict(tile=t))), ref_dx, "f16", "exact", f"dgrad tile {t}")


def test_int8_every_tile():
    prob = problem(2, 32, 9, 10, 48, 3, 3, pad=(1, 1))
    x, w, b, _ = case_inputs(prob, "i8", "uniform_i8", seed=43)
    scales = (0.02, 0.01, 0.05)
    exp = oracle_fprop_out(prob, "i8", x, w, b, True, scales=scales)
    for t in range(1, B.conv2d_plan_info(0, prob, "i8")["num_tiles"] + 1):
        y = run_fprop(prob, "i8", x, w, b, True, scales=scales, algo=dict(tile=t))
        assert np.array_equal(y.cpu().numpy().reshape(-1), exp), f"tile {t}"


def test_wgrad_band_and_generic_agree():
    prob = problem(8, 64, 18, 16, 64, 3, 3, pad=(1, 1))
    x, _, _, dy = case_inputs(prob, "f16", "int", seed=49)
    ref = oracle.wgrad(prob, f64(x), f64(dy))
    info = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")
    assert info["num_tiles"] == 3 and info["tile"] == 2  # band kernel is the default
    for t in (1, 2, 3):
        check(f64(run_wgrad(prob, "f16", x, dy, algo=dict(tile=t))), ref, "f16", "exact", f"wgrad tile {t}")


@pytest.mark.parametrize("prob", [
    problem(2, 16, 11, 9, 32, 3, 3, pad=(1, 1), groups=2),
    problem(3, 64, 14, 13, 96, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2), groups=4),
], ids=["g2", "c4g_like"])
def test_grouped_every_tile(prob):
    """Grouped problems whose channels per group come in 16-byte chunks:
    fprop and dgrad (every stride phase) on every implicit-GEMM tile, wgrad
    on both generic wgrad kernels, one GEMM per group; then the direct
    kernels, which follow the GEMM tiles in the table; against the oracle."""
    x, w, b, dy = case_inputs(prob, "f16", "int", seed=50)
    ref_y = oracle_fprop_out(prob, "f16", x, w, b, True)
    ref_dx = oracle.dgrad(prob, f64(dy), f64(w))
    ref_dw = oracle.wgrad(prob, f64(x), f64(dy))
    for op, n_gemm in ((B.CONV2D_OP_FPROP, 5), (B.CONV2D_OP_DGRAD, 5), (B.CONV2D_OP_WGRAD, 2)):
        info = B.conv2d_plan_info(op, prob, "f16")
        assert info["kernel"] == 1 and n_gemm < info["num_tiles"] <= n_gemm + 2, info
        kinds = [B.conv2d_plan_info(op, prob, "f16", algo=dict(tile=t))["kernel"]
                 for t in range(1, info["num_tiles"] + 1)]
        assert kinds == [1] * n_gemm + [2] * (info["num_tiles"] - n_gemm), kinds
    for t in range(1, B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16")["num_tiles"] + 1):
        algo = dict(tile=t)
        check(f64(run_fprop(prob, "f16", x, w, b, True, algo=algo)), ref_y, "f16", "exact", f"tile {t}")
    for t in range(1, B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, "f16")["num_tiles"] + 1):
        algo = dict(tile=t)
        check(f64(run_dgrad(prob, "f16", dy, w, algo=algo, fill=float("nan"))), ref_dx, "f16", "exact",
              f"dgrad tile {t}")
    for t in range(1, B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")["num_tiles"] + 1):
        algo = dict(tile=t)
        check(f64(run_wgrad(prob, "f16", x, dy, algo=algo)), ref_dw, "f16", "exact", f"wgrad tile {t}")


@pytest.mark.parametrize("groups", [1, 2])
def test_wgrad_split_k_bit_identical(groups):
    prob = problem(2, 16, 14, 12, 24, 3, 3, pad=(1, 1), groups=groups)
    x, _, _, dy = case_inputs(prob, "f16", "int", seed=44)
    ref = oracle.wgrad(prob, f64(x), f64(dy))
    outs = []
    for s in (1, 2, 3, 5, 16, 200):
        dw = run_wgrad(prob, "f16", x, dy, algo=dict(split_k=s))
        check(f64(dw), ref, "f16", "exact", f"split {s}")
        outs.append(dw.cpu())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_deterministic_repeats():
    prob = problem(4, 64, 18, 18, 64, 3, 3, pad=(1, 1))
    x, w, b, dy = case_inputs(prob, "f16", "gauss", seed=45)
    for run in (lambda: run_fprop(prob, "f16", x, w, b, True), lambda: run_dgrad(prob, "f16", dy, w),
                lambda: run_wgrad(prob, "f16", x, dy)):
        a, c = run(), run()
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_nonzero_storage_offsets():
    """Sub-tensors that start inside a larger allocation (16-byte aligned)."""
    prob = problem(3, 16, 9, 9, 24, 3, 3, pad=(1, 1))
    x, w, b, dy = case_inputs(prob, "f16", "int", seed=46)
    P, Q = B.conv2d_output_size(prob)

    def inside(t, off=64):
        buf = torch.zeros(t.numel() + 2 * off, dtype=t.dtype, device="cuda")
        v = buf[off:off + t.numel()].view(t.shape)
        v.copy_(t.to("cuda"))
        return v

    y = inside(torch.zeros(prob["N"], P, Q, prob["K"], dtype=torch.float16))
    B.conv2d_fprop(prob, "f16", inside(x), inside(w), inside(b), 0, 1.0, 1.0, 1.0, y, None)
    torch.cuda.synchronize()
    check(f64(y), oracle_fprop_out(prob, "f16", x, w, b, False), "f16", "exact", "offset fprop")


def test_error_leaves_output_untouched():
    # wgrad split four ways needs room for its fp32 partials
    prob = problem(2, 16, 8, 8, 16, 3, 3, pad=(1, 1))
    x, w, b, dy = case_inputs(prob, "f16", "int", seed=47)
    dw = torch.full((16, 3, 3, 16), 7.0, dtype=torch.float16, device="cuda")
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.Conv2dError) as e:
        B.conv2d_wgrad(prob, "f16", x.cuda(), dy.cuda(), dw, small, algo=dict(split_k=4))
    assert e.value.status == B.CONV2D_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(dw == 7.0)


# ------------------------------------------- the LDS-tiled direct kernels
# Grouped problems whose channels per group are not whole 16-byte vectors run
# the direct kernels.  fprop and wgrad take the LDS-tiled kernel when C/G is
# a multiple of 8 and K/G of 4 (here K/G = 4 or 12, so not the grouped GEMM);
# dgrad takes it when K/G is a multiple of 8 and C/G of 4.  Each case asserts
# the plan (kernel 2 = direct, tile 1 = tiled) so that the kernel under test
# is the one that runs.
DIRECT_TILED = [
    # (id, problem, dtype, dist, bias, relu, tiled passes)
    ("dt_fw_small", problem(2, 16, 9, 10, 8, 3, 3, pad=(1, 1), groups=2), "f16", "int", True, False,
     ("fprop", "wgrad")),
    ("dt_fw_s2d2", problem(3, 48, 21, 17, 24, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2), groups=2),
     "bf16", "int", True, True, ("fprop", "wgrad")),
    ("dt_d_small", problem(2, 8, 11, 9, 16, 3, 3, pad=(1, 1), groups=2), "f16", "int", False, False,
     ("dgrad",)),
    ("dt_d_asym", problem(3, 24, 13, 21, 48, 3, 2, pad=(1, 0), stride=(1, 2), dil=(2, 1), groups=2),
     "bf16", "int", True, True, ("dgrad",)),
    ("dt_d_gauss", problem(2, 12, 10, 14, 24, 3, 3, pad=(1, 1), groups=3), "f16", "gauss", True, False,
     ("dgrad",)),
    ("dt_fw_gauss_g3", problem(2, 24, 12, 13, 12, 3, 3, pad=(1, 1), groups=3), "bf16", "gauss", True, True,
     ("fprop", "wgrad")),
]


@pytest.mark.parametrize("cid,prob,dtype,dist,bias,relu,tiled", DIRECT_TILED, ids=[c[0] for c in DIRECT_TILED])
def test_direct_tiled_kernels(cid, prob, dtype, dist, bias, relu, tiled):
    ops = dict(fprop=B.CONV2D_OP_FPROP, dgrad=B.CONV2D_OP_DGRAD, wgrad=B.CONV2D_OP_WGRAD)
    for name in tiled:
        info = B.conv2d_plan_info(ops[name], prob, dtype)
        assert info["kernel"] == 2 and info["tile"] == 1 and info["num_tiles"] == 2, (name, info)
    mode = "exact" if dist == "int" else "tol"
    x, w, b, dy = case_inputs(prob, dtype, dist, seed=zlib.crc32(cid.encode()), bias=bias)
    ref_y = oracle_fprop_out(prob, dtype, x, w, b, relu)
    ref_dx = oracle.dgrad(prob, f64(dy), f64(w))
    ref_dw = oracle.wgrad(prob, f64(x), f64(dy))
    # the default plan, then both direct tiles explicitly
    for algo in (None, dict(tile=1), dict(tile=2)):
        if algo is not None and B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, dtype)["num_tiles"] < algo["tile"]:
            continue
        tag = f"{cid} tile {algo['tile'] if algo else 'default'}"
        check(f64(run_fprop(prob, dtype, x, w, b, relu, algo=algo)), ref_y, dtype, mode, f"{tag} fprop")
    for algo in (None, dict(tile=1)) + ((dict(tile=2),) if "dgrad" in tiled else ()):
        tag = f"{cid} tile {algo['tile'] if algo else 'default'}"
        check(f64(run_dgrad(prob, dtype, dy, w, algo=algo, fill=float("nan"))), ref_dx, dtype, mode,
              f"{tag} dgrad")
    for algo in (None, dict(tile=1)) + ((dict(tile=2), dict(tile=2, split_k=3)) if "wgrad" in tiled else ()):
        tag = f"{cid} tile {algo['tile'] if algo else 'default'}"
        check(f64(run_wgrad(prob, dtype, x, dy, algo=algo)), ref_dw, dtype, mode, f"{tag} wgrad")


# ---------------------------------------------------- few input channels

# C not a multiple of 8 with stride_w*C even, W*C a multiple of 8 and K = 32
# or 64: the few-channel fprop kernel (the default), each filter row's S*C
# taps read as one window of the input row.  Window lengths 8..32 (reduction
# steps 1..14 of the built 4, 8, 11, 12, 16), odd and even pads (the window
# starts one element early when pad_w*C is odd), row dilation, 1x1, and a
# ragged last band (P = 25 over bands of 3 rows).
FEW_CASES = [
    ("few_stem", problem(2, 3, 32, 32, 64, 7, 7, pad=(3, 3), stride=(2, 2)), "f16", "int", True, True),
    ("few_stem_ragged", problem(64, 3, 50, 32, 64, 7, 7, pad=(3, 3), stride=(2, 2)), "f16", "gauss", True, True),
    ("few_c4_k32", problem(2, 4, 17, 22, 32, 3, 3, pad=(1, 1)), "bf16", "gauss", True, False),
    ("few_c2_dil", problem(2, 2, 19, 20, 64, 5, 5, pad=(2, 2), dil=(2, 1)), "f16", "int", False, False),
    ("few_c1_s2", problem(3, 1, 25, 24, 32, 3, 3, stride=(2, 2)), "f16", "int", True, True),
    ("few_c6", problem(3, 6, 9, 12, 64, 3, 3, pad=(1, 1)), "bf16", "int", True, False),
    ("few_c5_1x1", problem(2, 5, 8, 16, 32, 1, 1, stride=(2, 2)), "f16", "int", True, False),
    ("few_c3_asym", problem(2, 3, 11, 40, 64, 2, 5, pad=(0, 2), stride=(1, 2)), "f16", "int", True, True),
    ("few_c4_7x7", problem(2, 4, 20, 22, 64, 7, 7, pad=(3, 3)), "f16", "int", True, True),
    ("few_c3_8x7", problem(2, 3, 21, 24, 32, 8, 7, pad=(3, 3), stride=(2, 2)), "bf16", "int", True, False),
]


@pytest.mark.parametrize("cid,prob,dtype,dist,bias,relu", FEW_CASES, ids=[c[0] for c in FEW_CASES])
def test_fewchan_fprop(cid, prob, dtype, dist, bias, relu):
    info = B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, dtype)
    assert info["kernel"] == 4 and info["tile"] == 0 and info["workspace_bytes"] == 0, info
    mode = "exact" if dist == "int" else "tol"
    x, w, b, _ = case_inputs(prob, dtype, dist, seed=zlib.crc32(cid.encode()), bias=bias)
    ref = oracle_fprop_out(prob, dtype, x, w, b, relu)
    P, Q = B.conv2d_output_size(prob)
    y = torch.full((prob["N"], P, Q, prob["K"]), float("nan"), dtype=x.dtype, device=DEV)
    B.conv2d_fprop(prob, dtype, gpu(x), gpu(w), gpu(b), relu, 1.0, 1.0, 1.0, y, None)
    torch.cuda.synchronize()
    check(f64(y), ref, dtype, mode, f"{cid} few-channel")
    if relu:
        assert not bool((y.view(torch.int16) == -32768).any()), f"{cid}: -0 after ReLU"
    # the padded path's first tile gives the same answer
    yp = run_fprop(prob, dtype, x, w, b, relu, algo=dict(tile=2))
    check(f64(yp), ref, dtype, mode, f"{cid} padded tile")
    if mode == "exact":
        assert torch.equal(y.view(torch.int16), yp.view(torch.int16))


def test_fewchan_bias_at_2_byte_offset():
    """The bias may start at any 2-byte boundary (the boundary's own rule);
    the few-channel kernel reads it from the 16-byte boundary below."""
    prob = problem(2, 3, 20, 32, 64, 7, 7, pad=(3, 3), stride=(2, 2))
    x, w, b, _ = case_inputs(prob, "f16", "int", seed=4711, bias=True)
    ref = oracle_fprop_out(prob, "f16", x, w, b, True)
    P, Q = B.conv2d_output_size(prob)
    for off in (1, 3, 7):
        buf = torch.zeros(prob["K"] + 16, dtype=torch.float16, device=DEV)
        bv = buf[off:off + prob["K"]]
        bv.copy_(b.to(DEV))
        y = torch.full((prob["N"], P, Q, prob["K"]), float("nan"), dtype=torch.float16, device=DEV)
        B.conv2d_fprop(prob, "f16", gpu(x), gpu(w), bv, 1, 1.0, 1.0, 1.0, y, None)
        torch.cuda.synchronize()
        check(f64(y), ref, "f16", "exact", f"bias at element offset {off}")


# The few-channel wgrad kernel (K = 64): window columns read with transposing
# LDS reads; when stride_w*C is 2 mod 4 the odd pixels come from the rows'
# copy shifted by 4 bytes.  Both alignments, one to three steps per pixel
# class, row dilation, bands of 3 rows (groups of 2 and 1), bf16 Gaussian.
FEW_WGRAD_CASES = [
    ("fw_c4_s1", problem(2, 4, 15, 18, 64, 3, 3, pad=(1, 1)), "f16", "int"),
    ("fw_c2_s2_wide", problem(2, 2, 9, 80, 64, 3, 3, pad=(1, 1), stride=(2, 2)), "f16", "int"),
    ("fw_c3_wide_s2", problem(3, 3, 11, 136, 64, 7, 7, pad=(3, 3), stride=(2, 2)), "f16", "int"),
    ("fw_c6_dil_bf16", problem(2, 6, 13, 20, 64, 3, 2, pad=(2, 1), dil=(2, 1)), "bf16", "gauss"),
    ("fw_c1_s4", problem(2, 1, 17, 64, 64, 5, 5, pad=(2, 2), stride=(4, 4)), "f16", "int"),
    ("fw_c3_bands3", problem(24, 3, 66, 32, 64, 7, 7, pad=(3, 3), stride=(2, 2)), "f16", "gauss"),
] + [(c[0], c[1], c[2], c[3]) for c in FEW_CASES if c[1]["K"] == 64 and c[0] != "few_c4_7x7"]


@pytest.mark.parametrize("cid,prob,dtype,dist", FEW_WGRAD_CASES, ids=[c[0] for c in FEW_WGRAD_CASES])
def test_fewchan_wgrad(cid, prob, dtype, dist):
    info = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, dtype)
    assert info["kernel"] == 4 and info["tile"] == 0, info
    mode = "exact" if dist == "int" else "tol"
    x, _, _, dy = case_inputs(prob, dtype, dist, seed=zlib.crc32(cid.encode()), bias=False)
    ref = oracle.wgrad(prob, f64(x), f64(dy))
    dw = run_wgrad(prob, dtype, x, dy)
    check(f64(dw), ref, dtype, mode, f"{cid} few-channel wgrad")
    again = run_wgrad(prob, dtype, x, dy)
    assert torch.equal(again.view(torch.int16), dw.view(torch.int16)), f"{cid}: repeat differs"
    # the padded path's first tile gives the same answer
    dwp = run_wgrad(prob, dtype, x, dy, algo=dict(tile=2))
    check(f64(dwp), ref, dtype, mode, f"{cid} padded tile")


def test_fewchan_wgrad_epilogue():
    """alpha/beta with C and an fp32 dw, and the bias gradient, on the
    few-channel wgrad plan (the epilogue runs in the split-K reduce, the bias
    gradient as its own column sums)."""
    prob = problem(2, 3, 20, 32, 64, 7, 7, pad=(3, 3), stride=(2, 2))
    x, _, _, dy = case_inputs(prob, "f16", "int", seed=4242, bias=False)
    assert B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")["kernel"] == 4
    ref = oracle.wgrad(prob, f64(x), f64(dy))
    c = torch.randint(-3, 4, ref.shape, dtype=torch.float32)
    dw = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=DEV)
    db = torch.full((prob["K"],), float("nan"), dtype=torch.float32, device=DEV)
    epi = dict(alpha=2.0, beta=-1.0, c=c.to(DEV), out_f32=1, db=db)
    n = B.conv2d_workspace_size_ex(B.CONV2D_OP_WGRAD, prob, "f16", epi=epi)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
    B.conv2d_wgrad_ex(prob, "f16", gpu(x), gpu(dy), epi, dw, ws)
    torch.cuda.synchronize()
    assert np.array_equal(f64(dw), 2.0 * ref - c.numpy().astype(np.float64))
    assert np.array_equal(f64(db), f64(dy).reshape(-1, prob["K"]).sum(axis=0))


# The few-channel dgrad kernel (C <= 4, stride 2, K = 64): 2x2 output blocks
# as GEMM rows.  Filters that read 2, 3 and 4 dy offsets per axis, an odd H
# (the last block row half outside), a last block of 16 super-pixels that
# ends inside the row, bands of several row pairs, bf16 Gaussian.
FEW_DGRAD_CASES = [
    ("fd_c4_3x3", problem(2, 4, 18, 20, 64, 3, 3, pad=(1, 1), stride=(2, 2)), "f16", "int"),
    ("fd_c2_5x5_oddH", problem(2, 2, 17, 24, 64, 5, 5, pad=(2, 2), stride=(2, 2)), "f16", "int"),
    ("fd_c1_4x4_p0", problem(3, 1, 16, 32, 64, 4, 4, stride=(2, 2)), "f16", "int"),
    ("fd_c3_wide_bf16", problem(2, 3, 12, 72, 64, 7, 7, pad=(3, 3), stride=(2, 2)), "bf16", "gauss"),
    ("fd_c3_bands", problem(40, 3, 26, 16, 64, 7, 7, pad=(3, 3), stride=(2, 2)), "f16", "gauss"),
] + [(c[0], c[1], c[2], c[3]) for c in FEW_CASES if c[0] in ("few_stem", "few_stem_ragged")]


@pytest.mark.parametrize("cid,prob,dtype,dist", FEW_DGRAD_CASES, ids=[c[0] for c in FEW_DGRAD_CASES])
def test_fewchan_dgrad(cid, prob, dtype, dist):
    info = B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, dtype)
    assert info["kernel"] == 4 and info["tile"] == 0 and info["workspace_bytes"] == 0, info
    mode = "exact" if dist == "int" else "tol"
    _, w, _, dy = case_inputs(prob, dtype, dist, seed=zlib.crc32(cid.encode()), bias=False)
    ref = oracle.dgrad(prob, f64(dy), f64(w))
    dx = run_dgrad(prob, dtype, dy, w, fill=float("nan"))
    check(f64(dx), ref, dtype, mode, f"{cid} few-channel dgrad")
    again = run_dgrad(prob, dtype, dy, w)
    assert torch.equal(again.view(torch.int16), dx.view(torch.int16)), f"{cid}: repeat differs"
    # the padded path's first tile gives the same answer
    dxp = run_dgrad(prob, dtype, dy, w, algo=dict(tile=2), fill=float("nan"))
    check(f64(dxp), ref, dtype, mode, f"{cid} padded tile")


# ------------------------------------------------------------- the workloads

def _workload_inputs(name):
    wl = WL.WORKLOADS[name]
    prob = wl["prob"]
    P, Q = B.conv2d_output_size(prob)
    x, w = WL.make_x(name), WL.make_w(name)
    b = WL.make_bias(name) if wl["bias"] else None
    dy = WL.make_dy(name, P, Q) if wl["dtype"] != "i8" else None
    return wl, prob, x, w, b, dy


@pytest.mark.parametrize("name", ["c1_tiny", "c2_strided", "c3a_resnet3x3", "c3b_resnet1x1", "c4_awkward",
                                  "c4g_grouped", "n1_stem", "d1_depthwise"])
def test_workload_full(name):
    """Every output of the three passes at the workload's full size, in the
    launch configuration the benchmark times (the library's default plan),
    against the oracle; plus, for workloads without bias and ReLU, the
    adjoint identity <y, dy> = <x, dx> = <w, dw> on the GPU's own results."""
    wl, prob, x, w, b, dy = _workload_inputs(name)
    dt, mode = wl["dtype"], wl["check"]
    y = run_fprop(prob, dt, x, w, b, wl["relu"])
    yr = f64(y)
    check(yr, oracle_fprop_out(prob, dt, x, w, b, wl["relu"]), dt, mode, f"{name} fprop")
    dx = f64(run_dgrad(prob, dt, dy, w, fill=float("nan")))
    xb, wb, dyb = f64(x), f64(w), f64(dy)
    check(dx, oracle.dgrad(prob, dyb, wb), dt, mode, f"{name} dgrad")
    dw = f64(run_wgrad(prob, dt, x, dy))
    check(dw, oracle.wgrad(prob, xb, dyb), dt, mode, f"{name} wgrad")
    if not wl["relu"] and b is None:
        a1 = float(np.dot(yr.reshape(-1), dyb.reshape(-1)))
        a2 = float(np.dot(xb.reshape(-1), dx.reshape(-1)))
        a3 = float(np.dot(wb.reshape(-1), dw.reshape(-1)))
        scale = np.linalg.norm(yr) * np.linalg.norm(dyb)
        assert abs(a1 - a2) <= 2e-3 * scale and abs(a1 - a3) <= 2e-3 * scale, (a1, a2, a3, scale)


def test_workload_c4g_direct_full():
    """The grouped variant of the awkward workload (16x57x57x96 -> 96, 5x5
    s2 p2 d2, groups 4, bf16) runs on the grouped implicit GEMM by default;
    here every pass runs it on the direct kernels (the last tile of each
    table), every output against the oracle."""
    name = "c4g_grouped"
    wl, prob, x, w, b, dy = _workload_inputs(name)
    dt, mode = wl["dtype"], wl["check"]
    algos = {}
    for op in (B.CONV2D_OP_FPROP, B.CONV2D_OP_DGRAD, B.CONV2D_OP_WGRAD):
        n = B.conv2d_plan_info(op, prob, dt)["num_tiles"]
        algos[op] = dict(tile=n)
        assert B.conv2d_plan_info(op, prob, dt, algo=algos[op])["kernel"] == 2
    y = run_fprop(prob, dt, x, w, b, wl["relu"], algo=algos[B.CONV2D_OP_FPROP])
    check(f64(y), oracle_fprop_out(prob, dt, x, w, b, wl["relu"]), dt, mode, "c4g direct fprop")
    dx = run_dgrad(prob, dt, dy, w, algo=algos[B.CONV2D_OP_DGRAD], fill=float("nan"))
    check(f64(dx), oracle.dgrad(prob, f64(dy), f64(w)), dt, mode, "c4g direct dgrad")
    dw = run_wgrad(prob, dt, x, dy, algo=algos[B.CONV2D_OP_WGRAD])
    check(f64(dw), oracle.wgrad(prob, f64(x), f64(dy)), dt, mode, "c4g direct wgrad")


def test_workload_int8_full():
    """Every int8 code of the c5 workload (32x56x56x128 -> 128, 3x3,
    requantised with ReLU), bit-exact, on the benchmark's launch plan."""
    name = "c5_int8"
    wl, prob, x, w, b, _ = _workload_inputs(name)
    y = run_fprop(prob, "i8", x, w, b, wl["relu"], scales=wl["scales"]).cpu().numpy().reshape(-1)
    exp = oracle_fprop_out(prob, "i8", x, w, b, wl["relu"], scales=wl["scales"])
    bad = np.nonzero(y != exp)[0]
    assert bad.size == 0, f"{bad.size} of {y.size} codes differ, first at {bad[:5]}"
    assert y.min() >= 0 and y.max() <= 127
