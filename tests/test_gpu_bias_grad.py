"""GPU parity of the bias gradient, db[k] = sum of dy[n,p,q,k] over n, p, q,
against the oracle, through the C ABI: the 16-byte path (K % 8 == 0) on the
benchmark's full-size dy, a K that is not a multiple of 8 (element loads),
more than 256 eight-channel vectors (two column blocks), fewer rows than one
slice, a strided problem, fp32 output, and bit-identical repeats.  Integer
data sums exactly in fp32 (every partial sum is an integer below 2^24), so
those results must equal the oracle's rounded once."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import DEV, check, f64

pytestmark = pytest.mark.gpu

C3A = WL.WORKLOADS["c3a_resnet3x3"]["prob"]
CASES = [
    ("c3a_gauss", C3A, "f16", "gauss"),
    ("c3a_int", C3A, "f16", "int"),
    ("k13_bf16", problem(3, 8, 9, 10, 13, 3, 3, pad=(1, 1)), "bf16", "int"),
    ("k2056_two_blocks", problem(1, 8, 8, 8, 2056, 1, 1), "f16", "gauss"),
    ("rows_lt_64", problem(1, 8, 5, 6, 40, 3, 3, pad=(1, 1)), "f16", "int"),
    ("strided_bf16", problem(4, 16, 23, 19, 72, 3, 3, pad=(1, 1), stride=(2, 2)), "bf16", "gauss"),
]


def make_dy(cid, prob, dtype, dist):
    P, Q = oracle.output_hw(prob)
    rng = np.random.Generator(np.random.PCG64(zlib.crc32(cid.encode())))
    return WL.draw((prob["N"], P, Q, prob["K"]), dtype, dist, rng)


def run(prob, dtype, dy, out_f32=False):
    db = torch.empty((prob["K"],), dtype=torch.float32 if out_f32 else dy.dtype, device=DEV)
    n = B.conv2d_bias_grad_workspace_size(prob, dtype)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
    B.conv2d_bias_grad(prob, dtype, dy, db, ws, out_f32=out_f32)
    torch.cuda.synchronize()
    return db


@pytest.mark.parametrize("cid,prob,dtype,dist", CASES, ids=[c[0] for c in CASES])
def test_bias_grad(cid, prob, dtype, dist):
    dy = make_dy(cid, prob, dtype, dist)
    ref = oracle.bias_grad(prob, f64(dy))
    dyg = dy.to(DEV)
    db = run(prob, dtype, dyg)
    check(f64(db), ref, dtype, "exact" if dist == "int" else "tol", f"{cid} db")
    db32 = run(prob, dtype, dyg, out_f32=True)
    g = db32.cpu().numpy().astype(np.float64)
    if dist == "int":
        assert np.array_equal(g, ref), f"{cid} db fp32: {np.count_nonzero(g != ref)} differ"
    else:
        assert np.max(np.abs(g - ref)) <= 1e-5 * np.max(np.abs(ref)), f"{cid} db fp32"
    assert torch.equal(run(prob, dtype, dyg), db), f"{cid}: repeat differs"


def test_wgrad_with_fused_bias_grad_full_size():
    """On the benchmark shape the wgrad band kernel sums dy in its own slices:
    dw stays bit-identical to the plain pass, db matches the oracle."""
    prob = C3A
    assert B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")["tile"] == 2  # the wgrad band kernel
    x = WL.make_x("c3a_resnet3x3").to(DEV)
    dy = WL.make_dy("c3a_resnet3x3", 56, 56).to(DEV)
    dw0 = torch.empty((64, 3, 3, 64), dtype=torch.float16, device=DEV)
    B.conv2d_wgrad(prob, "f16", x, dy, dw0, B.workspace_for(B.CONV2D_OP_WGRAD, prob, "f16", DEV))
    db = torch.full((64,), float("nan"), dtype=torch.float16, device=DEV)
    epi = dict(db=db)
    n = B.conv2d_workspace_size_ex(B.CONV2D_OP_WGRAD, prob, "f16", epi=epi)
    dw = torch.empty_like(dw0)
    B.conv2d_wgrad_ex(prob, "f16", x, dy, epi, dw, torch.empty(n, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(dw, dw0), "dw changed by the fused bias gradient"
    check(f64(db), oracle.bias_grad(prob, f64(dy)), "f16", "tol", "fused db")


@pytest.mark.parametrize("prob", [
    problem(2, 64, 10, 12, 64, 3, 3, pad=(1, 1)),                       # all three wgrad kernels
    problem(76, 64, 9, 24, 64, 3, 3, pad=(1, 1)),                       # band kernel by filter rows
    problem(3, 32, 11, 9, 136, 5, 3, pad=(2, 1), stride=(2, 1), dil=(1, 2)),
], ids=["wband_shape", "wband_rows", "strided"])
def test_wgrad_db_every_tile(prob):
    """db beside wgrad on every wgrad kernel (fused into the 128x128 and band
    kernels, a second launch after the 64x64 one): dw is bit-identical to the
    plain pass of the same tile, db equals the oracle's (integer data)."""
    P, Q = oracle.output_hw(prob)
    x, _, _, dy = WL.random_case(prob, "f16", "int", zlib.crc32(b"db-tiles"), P, Q, bias=False)
    x, dy = x.to(DEV), dy.to(DEV)
    ref = oracle.bias_grad(prob, f64(dy))
    wshape = (prob["K"], prob["R"], prob["S"], prob["C"])
    for t in range(1, B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")["num_tiles"] + 1):
        algo = dict(tile=t)
        dw0 = torch.empty(wshape, dtype=torch.float16, device=DEV)
        B.conv2d_wgrad(prob, "f16", x, dy, dw0, B.workspace_for(B.CONV2D_OP_WGRAD, prob, "f16", DEV, algo), algo)
        db = torch.full((prob["K"],), float("nan"), dtype=torch.float16, device=DEV)
        epi = dict(db=db)
        n = B.conv2d_workspace_size_ex(B.CONV2D_OP_WGRAD, prob, "f16", algo=algo, epi=epi)
        dw = torch.empty_like(dw0)
        B.conv2d_wgrad_ex(prob, "f16", x, dy, epi, dw, torch.empty(max(n, 1), dtype=torch.uint8, device=DEV), algo)
        torch.cuda.synchronize()
        assert torch.equal(dw, dw0), f"tile {t}: dw changed"
        check(f64(db), ref, "f16", "exact", f"tile {t} db")
