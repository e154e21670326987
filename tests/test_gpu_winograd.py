"""GPU parity of the Winograd F(2x2, 3x3) fprop and dgrad (the last tile on
stride-1 3x3 fp16 problems with 64 source channels), through the C ABI.

Integer-valued inputs in [-4, 4]: the transformed filter values are
quarter-integers below 10 and the transformed input values integers below 17,
all exact in fp16, and every later sum is exact in fp32, so the result must
equal the direct definition rounded once (the oracle's fprop).

Gaussian inputs: the kernel rounds U = G g G^T and V = B^T d B once to fp16
(unit roundoff u_op) before the products; everything else runs in fp32, then
one rounding to the output type.  Every output must lie within
oracle.winograd.error_bound (2 u_op + u_op^2 + (2C+40) 2^-24 times the sum of
the absolute values of the terms) of the exact value, plus the output
rounding, and the whole output must also meet the max_rel <= 5e-3 and
rms_scaled <= 1e-3 every other path meets.  bf16 problems are refused."""
import numpy as np
import pytest
import torch

import oracle
from oracle import winograd as WGO
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import MAX_REL, RMS_SCALED, check, f64, run_dgrad, run_fprop

pytestmark = pytest.mark.gpu

U_TYPE = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def wino_tile(prob, dtype, op=B.CONV2D_OP_FPROP):
    """The Winograd tile of a pass: the one plan kernel 3 runs (the patch
    kernel's tile follows it where that kernel applies)."""
    info = B.conv2d_plan_info(op, prob, dtype)
    tiles = [t for t in range(1, info["num_tiles"] + 1)
             if B.conv2d_plan_info(op, prob, dtype, algo=dict(tile=t))["kernel"] == 3]
    assert len(tiles) == 1, tiles
    return dict(tile=tiles[0])


EXACT = [
    # partial 2x2 blocks (odd P, Q), two 64-column segments, bias + ReLU
    ("odd_two_segments", problem(2, 64, 13, 71, 64, 3, 3, pad=(1, 1)), "f16", True, True),
    ("pad0_k16", problem(3, 64, 9, 10, 16, 3, 3), "f16", True, False),
    ("pad2_k48", problem(2, 64, 7, 8, 48, 3, 3, pad=(2, 2)), "f16", False, True),
    ("k128_two_slices", problem(2, 64, 12, 20, 128, 3, 3, pad=(1, 1)), "f16", True, True),
    ("one_row", problem(3, 64, 1, 5, 32, 3, 3, pad=(1, 1)), "f16", True, False),
    ("many_batches", problem(40, 64, 10, 12, 64, 3, 3, pad=(1, 1)), "f16", True, True),
]


@pytest.mark.parametrize("cid,prob,dtype,bias,relu", EXACT, ids=[c[0] for c in EXACT])
def test_winograd_exact_on_integers(cid, prob, dtype, bias, relu):
    P, Q = oracle.output_hw(prob)
    x, w, b, _ = WL.random_case(prob, dtype, "int", 7000 + len(cid), P, Q, bias=bias)
    y = run_fprop(prob, dtype, x, w, b, relu, algo=wino_tile(prob, dtype))
    ref = oracle.fprop(prob, f64(x), f64(w), bias=None if b is None else f64(b), relu=relu)
    check(f64(y), ref, dtype, "exact", cid)


def within_bound(g, prob, x, w, b, relu, dtype, what):
    """Every output within the derived bound; returns (max_rel, rms_scaled)."""
    xf, wf = f64(x), f64(w)
    bf = None if b is None else f64(b)
    y = oracle.fprop(prob, xf, wf, bias=bf, relu=relu)
    E = WGO.error_bound(prob, xf, wf, U_TYPE[dtype])
    u_out = U_TYPE[dtype]
    babs = 0.0 if bf is None else np.abs(bf)
    tol = E * 1.001 + u_out * (np.abs(y) + E) + 2.0 ** -23 * (np.abs(y) + babs) + 1e-7
    err = np.abs(f64(g) - y)
    bad = np.nonzero(err > tol)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} outputs outside the bound; worst err/tol "
                              f"{np.max(err / tol):.3f}")
    ref_out = oracle.bits_to_f64(oracle.round_to(y, dtype), dtype)
    max_rel = float(np.max(err) / np.max(np.abs(y)))
    rms = float(np.linalg.norm(f64(g) - ref_out) / np.linalg.norm(ref_out))
    return max_rel, rms, float(np.max(err / tol))


GAUSS = [
    ("gauss_f16", problem(4, 64, 17, 23, 64, 3, 3, pad=(1, 1)), "f16", True, True),
    ("gauss_f16_nobias", problem(4, 64, 17, 23, 64, 3, 3, pad=(1, 1)), "f16", True, False),
    ("gauss_f16_k96_pad0", problem(2, 64, 15, 66, 96, 3, 3), "f16", False, False),
]


@pytest.mark.parametrize("cid,prob,dtype,bias,relu", GAUSS, ids=[c[0] for c in GAUSS])
def test_winograd_within_derived_bound(cid, prob, dtype, bias, relu):
    P, Q = oracle.output_hw(prob)
    x, w, b, _ = WL.random_case(prob, dtype, "gauss", 7100 + len(cid), P, Q, bias=bias)
    y = run_fprop(prob, dtype, x, w, b, relu, algo=wino_tile(prob, dtype))
    max_rel, rms, worst = within_bound(y, prob, x, w, b, relu, dtype, cid)
    print(f"{cid}: max_rel {max_rel:.2e} rms_scaled {rms:.2e} worst err/bound {worst:.3f}")
    assert max_rel <= MAX_REL and rms <= RMS_SCALED, (max_rel, rms)


def test_winograd_full_size_c3a():
    """The benchmark shape (64x56x56x64 -> 64, Gaussian, bias + ReLU) on the
    Winograd tile: two whole images against the bound (the first and the
    last, so the first and last batches of the persistent grid), and the
    same inputs' direct-kernel result for comparison."""
    name = "c3a_resnet3x3"
    prob = WL.WORKLOADS[name]["prob"]
    x, w, b = WL.make_x(name), WL.make_w(name), WL.make_bias(name)
    y = run_fprop(prob, "f16", x, w, b, True, algo=wino_tile(prob, "f16"))
    sub = dict(prob, N=1)
    for n in (0, prob["N"] - 1):
        mr, rms, worst = within_bound(y[n:n + 1], sub, x[n:n + 1], w, b, True, "f16", f"image {n}")
        print(f"c3a image {n}: max_rel {mr:.2e} rms_scaled {rms:.2e} worst err/bound {worst:.3f}")
    yd = run_fprop(prob, "f16", x, w, b, True)
    d = (y.float() - yd.float()).abs()
    assert torch.isfinite(y.float()).all()
    print(f"c3a Winograd vs band kernel: max |diff| {d.max().item():.3e}, "
          f"rms {d.pow(2).mean().sqrt().item():.3e}")


# ---- dgrad: the forward Winograd kernel on dy (K = 64 channels) with the
# filter's taps reversed and channel axes swapped, padded by 2 - pad
def dgrad_as_fprop(prob, w):
    """The forward problem and filter w'[c][r][s][k] = w[k][2-r][2-s][c] whose
    fprop of dy is dgrad(dy, w) for a stride-1 3x3 problem."""
    P, Q = oracle.output_hw(prob)
    fp = problem(prob["N"], prob["K"], P, Q, prob["C"], 3, 3, pad=(2 - prob["pad_h"], 2 - prob["pad_w"]))
    wf = np.ascontiguousarray(np.transpose(f64(w)[:, ::-1, ::-1, :], (3, 1, 2, 0)))
    return fp, torch.from_numpy(wf)


def run_dgrad_wino(prob, dtype, dy, w):
    return run_dgrad(prob, dtype, dy, w, algo=wino_tile(prob, dtype, B.CONV2D_OP_DGRAD), fill=float("nan"))


EXACT_D = [
    ("d_odd_two_segments", problem(2, 64, 13, 71, 64, 3, 3, pad=(1, 1)), "f16"),
    ("d_pad0_c16", problem(3, 16, 9, 10, 64, 3, 3), "f16"),
    ("d_pad2_c48", problem(2, 48, 7, 8, 64, 3, 3, pad=(2, 2)), "f16"),
    ("d_c128_two_slices", problem(2, 128, 12, 20, 64, 3, 3, pad=(1, 1)), "f16"),
]


@pytest.mark.parametrize("cid,prob,dtype", EXACT_D, ids=[c[0] for c in EXACT_D])
def test_winograd_dgrad_exact_on_integers(cid, prob, dtype):
    P, Q = oracle.output_hw(prob)
    _, w, _, dy = WL.random_case(prob, dtype, "int", 7200 + len(cid), P, Q, bias=False)
    dx = run_dgrad_wino(prob, dtype, dy, w)
    check(f64(dx), oracle.dgrad(prob, f64(dy), f64(w)), dtype, "exact", cid)


def test_winograd_dgrad_within_derived_bound():
    dtype = "f16"
    prob = problem(4, 64, 17, 23, 64, 3, 3, pad=(1, 1))
    P, Q = oracle.output_hw(prob)
    _, w, _, dy = WL.random_case(prob, dtype, "gauss", 7300, P, Q, bias=False)
    dx = run_dgrad_wino(prob, dtype, dy, w)
    fp, wf = dgrad_as_fprop(prob, w)
    # the equivalent forward problem reproduces the direct dgrad
    ref = oracle.dgrad(prob, f64(dy), f64(w))
    assert np.max(np.abs(oracle.fprop(fp, f64(dy), f64(wf)) - ref)) <= 1e-12 * np.max(np.abs(ref))
    max_rel, rms, worst = within_bound(dx, fp, dy, wf, None, False, dtype, f"dgrad {dtype}")
    print(f"dgrad {dtype}: max_rel {max_rel:.2e} rms_scaled {rms:.2e} worst err/bound {worst:.3f}")
    assert max_rel <= MAX_REL and rms <= RMS_SCALED, (max_rel, rms)


def test_winograd_refuses_bf16():
    prob = problem(2, 64, 10, 12, 64, 3, 3, pad=(1, 1))
    for op in (B.CONV2D_OP_FPROP, B.CONV2D_OP_DGRAD):
        n = B.conv2d_plan_info(op, prob, "bf16")["num_tiles"]
        assert all(B.conv2d_plan_info(op, prob, "bf16", algo=dict(tile=t))["kernel"] != 3 for t in range(1, n + 1))
        with pytest.raises(B.Conv2dError) as e:
            B.conv2d_plan_info(op, prob, "bf16", algo=dict(tile=n + 1))
        assert e.value.status == B.CONV2D_ERR_UNSUPPORTED
