"""GPU parity of the linear-combination epilogue (out = alpha * result +
beta * C, and wgrad's fp32 output) against the oracle, through the C ABI, on
every kernel family: the implicit GEMM (fprop, strided dgrad phases, generic
wgrad), shapes the band kernels would take (fprop/dgrad then run on the
implicit GEMM; wgrad keeps the band kernel and applies the epilogue in its
reduction), the pointwise wgrad kernel (1x1), the grouped implicit GEMM, the LDS-tiled and
one-thread-per-output direct kernels, and the zero-padded channel path.  Integer-valued data with alpha = 2, beta = -1 is
exact in fp32, so those outputs must equal the oracle's rounded once."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import DEV, check, f64, gpu

pytestmark = pytest.mark.gpu

CASES = [
    ("igemm", problem(2, 32, 13, 11, 48, 3, 3, pad=(1, 1), stride=(2, 1)), "f16", "int"),
    ("band_shape", problem(3, 64, 12, 14, 64, 3, 3, pad=(1, 1)), "f16", "int"),
    # the wgrad band kernel (Q a multiple of 4): the bias gradient is summed
    # inside it and reduced with the weight gradient
    ("wband_shape", problem(2, 64, 10, 12, 64, 3, 3, pad=(1, 1)), "bf16", "int"),
    ("wband_gauss", problem(3, 64, 9, 16, 64, 3, 3, pad=(1, 1)), "f16", "gauss"),
    ("grouped_gemm", problem(2, 32, 11, 9, 48, 3, 3, pad=(1, 1), groups=2), "f16", "int"),
    # LDS-tiled direct kernels: fprop and wgrad (C/G = 8, K/G = 4), dgrad (C/G = 4, K/G = 8)
    ("direct_tiled_fw", problem(2, 16, 9, 10, 8, 3, 3, pad=(1, 1), groups=2), "f16", "int"),
    ("direct_tiled_d", problem(2, 8, 11, 9, 16, 3, 3, pad=(1, 1), groups=2), "bf16", "int"),
    ("direct_tiled_gauss", problem(2, 24, 12, 13, 12, 3, 3, pad=(1, 1), groups=3), "bf16", "gauss"),
    ("grouped_naive", problem(2, 12, 9, 10, 8, 3, 3, pad=(1, 1), groups=2), "bf16", "int"),
    ("padded_c3_k13", problem(2, 3, 17, 15, 13, 5, 5, pad=(2, 2), stride=(2, 2)), "f16", "int"),
    ("gauss", problem(2, 24, 12, 11, 40, 3, 3, pad=(1, 1)), "bf16", "gauss"),
    # 1x1 stride 1: wgrad on the pointwise wgrad kernel (bias gradient in its
    # slices, the epilogue in the reduce); one and four pixel phases
    ("pointwise_k256", problem(3, 64, 9, 13, 256, 1, 1), "f16", "int"),
    ("pointwise_k64_gauss", problem(2, 64, 12, 11, 64, 1, 1), "bf16", "gauss"),
]


def inputs(cid, prob, dtype, dist):
    P, Q = oracle.output_hw(prob)
    x, w, b, dy = WL.random_case(prob, dtype, dist, zlib.crc32(cid.encode()), P, Q, bias=True)
    # C tensors with the distribution of the data
    cy = WL.random_case(prob, dtype, dist, zlib.crc32(cid.encode()) + 1, P, Q, bias=False)[3]
    cx = WL.random_case(prob, dtype, dist, zlib.crc32(cid.encode()) + 2, P, Q, bias=False)[0]
    cw = WL.random_case(prob, dtype, dist, zlib.crc32(cid.encode()) + 3, P, Q, bias=False)[1]
    return x, w, b, dy, cy, cx, cw


def coefs(dist):
    return (2.0, -1.0) if dist == "int" else (0.5, 0.25)


def ws_for(op, prob, dtype, epi):
    n = B.conv2d_workspace_size_ex(op, prob, dtype, epi=epi)
    return torch.empty(n, dtype=torch.uint8, device=DEV) if n else None


@pytest.mark.parametrize("cid,prob,dtype,dist", CASES, ids=[c[0] for c in CASES])
def test_epilogue_all_passes(cid, prob, dtype, dist):
    if cid.startswith("direct_tiled"):  # the kernels under test are the ones planned
        ops = (B.CONV2D_OP_DGRAD,) if cid == "direct_tiled_d" else (B.CONV2D_OP_FPROP, B.CONV2D_OP_WGRAD)
        for op in ops:
            info = B.conv2d_plan_info(op, prob, dtype)
            assert info["kernel"] == 2 and info["tile"] == 1, (op, info)
    mode = "exact" if dist == "int" else "tol"
    alpha, beta = coefs(dist)
    x, w, b, dy, cy, cx, cw = inputs(cid, prob, dtype, dist)
    P, Q = oracle.output_hw(prob)
    # fprop, with bias and ReLU after the combination
    epi = dict(alpha=alpha, beta=beta, c=gpu(cy))
    y = torch.empty((prob["N"], P, Q, prob["K"]), dtype=x.dtype, device=DEV)
    B.conv2d_fprop_ex(prob, dtype, gpu(x), gpu(w), gpu(b), True, epi, y,
                      ws_for(B.CONV2D_OP_FPROP, prob, dtype, epi))
    torch.cuda.synchronize()
    ref = oracle.linear_combination(oracle.fprop(prob, f64(x), f64(w)), alpha, beta, f64(cy),
                                    bias=f64(b), relu=True)
    check(f64(y), ref, dtype, mode, f"{cid} fprop")
    # dgrad
    epi = dict(alpha=alpha, beta=beta, c=gpu(cx))
    dx = torch.full_like(gpu(x), float("nan"))
    B.conv2d_dgrad_ex(prob, dtype, gpu(dy), gpu(w), epi, dx, ws_for(B.CONV2D_OP_DGRAD, prob, dtype, epi))
    torch.cuda.synchronize()
    ref = oracle.linear_combination(oracle.dgrad(prob, f64(dy), f64(w)), alpha, beta, f64(cx))
    check(f64(dx), ref, dtype, mode, f"{cid} dgrad")
    # wgrad, rounded to the filter type, with the bias gradient beside it
    db = torch.full((prob["K"],), float("nan"), dtype=x.dtype, device=DEV)
    epi = dict(alpha=alpha, beta=beta, c=gpu(cw), db=db)
    dw = torch.empty_like(gpu(w))
    B.conv2d_wgrad_ex(prob, dtype, gpu(x), gpu(dy), epi, dw, ws_for(B.CONV2D_OP_WGRAD, prob, dtype, epi))
    torch.cuda.synchronize()
    dw_ref = oracle.wgrad(prob, f64(x), f64(dy))
    db_ref = oracle.bias_grad(prob, f64(dy))
    check(f64(dw), oracle.linear_combination(dw_ref, alpha, beta, f64(cw)), dtype, mode, f"{cid} wgrad")
    check(f64(db), db_ref, dtype, mode, f"{cid} db")  # alpha and beta do not apply to db
    # wgrad kept in fp32, with an fp32 C (and an fp32 db)
    cw32 = gpu(cw).float()
    db32 = torch.full((prob["K"],), float("nan"), dtype=torch.float32, device=DEV)
    epi = dict(alpha=alpha, beta=beta, c=cw32, out_f32=True, db=db32)
    dw32 = torch.empty(dw.shape, dtype=torch.float32, device=DEV)
    B.conv2d_wgrad_ex(prob, dtype, gpu(x), gpu(dy), epi, dw32, ws_for(B.CONV2D_OP_WGRAD, prob, dtype, epi))
    torch.cuda.synchronize()
    g = dw32.cpu().numpy().astype(np.float64).reshape(-1)
    r = oracle.linear_combination(dw_ref, alpha, beta, f64(cw)).reshape(-1)
    gb = db32.cpu().numpy().astype(np.float64)
    if mode == "exact":  # integer partial sums below 2^24: exact in fp32
        assert np.array_equal(g, r), f"{cid} wgrad fp32: {np.count_nonzero(g != r)} differ"
        assert np.array_equal(gb, db_ref), f"{cid} db fp32"
    else:
        assert np.max(np.abs(g - r)) <= 1e-5 * np.max(np.abs(r)), f"{cid} wgrad fp32"
        assert np.max(np.abs(gb - db_ref)) <= 1e-5 * np.max(np.abs(db_ref)), f"{cid} db fp32"


def test_epilogue_in_place_and_plain():
    """C may be the output itself (D += conv with beta = 1); alpha = 1,
    beta = 0 (and a NULL epilogue) is the plain pass, bit for bit."""
    prob = problem(2, 16, 10, 9, 24, 3, 3, pad=(1, 1))
    x, w, b, dy, cy, cx, cw = inputs("inplace", prob, "f16", "int")
    P, Q = oracle.output_hw(prob)
    y = gpu(cy).clone()
    epi = dict(alpha=1.0, beta=1.0, c=y)
    B.conv2d_fprop_ex(prob, "f16", gpu(x), gpu(w), None, False, epi, y,
                      ws_for(B.CONV2D_OP_FPROP, prob, "f16", epi))
    torch.cuda.synchronize()
    ref = oracle.linear_combination(oracle.fprop(prob, f64(x), f64(w)), 1.0, 1.0, f64(cy))
    check(f64(y), ref, "f16", "exact", "fprop in place")
    dw = gpu(cw).clone()
    epi = dict(alpha=1.0, beta=1.0, c=dw)
    B.conv2d_wgrad_ex(prob, "f16", gpu(x), gpu(dy), epi, dw, ws_for(B.CONV2D_OP_WGRAD, prob, "f16", epi))
    torch.cuda.synchronize()
    ref = oracle.linear_combination(oracle.wgrad(prob, f64(x), f64(dy)), 1.0, 1.0, f64(cw))
    check(f64(dw), ref, "f16", "exact", "wgrad in place")
    # plain: identical bits to conv2d_fprop / conv2d_dgrad
    y0 = torch.empty((prob["N"], P, Q, prob["K"]), dtype=torch.float16, device=DEV)
    y1 = torch.empty_like(y0)
    B.conv2d_fprop(prob, "f16", gpu(x), gpu(w), gpu(b), True, 1.0, 1.0, 1.0, y0,
                   B.workspace_for(B.CONV2D_OP_FPROP, prob, "f16", DEV))
    epi = dict(alpha=1.0, beta=0.0)
    B.conv2d_fprop_ex(prob, "f16", gpu(x), gpu(w), gpu(b), True, epi, y1,
                      ws_for(B.CONV2D_OP_FPROP, prob, "f16", epi))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
