"""Seeded sweep of random small problems through every kernel family: the
band kernels, the implicit GEMM (every tile and stride phase), the wgrad band
and generic wgrad with several split counts, the zero-padded channel path,
the grouped direct kernels and the depthwise kernels.  Every pass is compared
with the oracle on integer-valued data, where every partial sum is an exact
fp32 integer, so the outputs must equal the oracle's rounded once."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import check, f64, run_dgrad, run_fprop, run_wgrad

pytestmark = pytest.mark.gpu

NCASES = 126
KINDS = ("dense", "dense_odd", "grouped", "depthwise", "band", "wband", "stem")


def draw_problem(rng, kind):
    """A valid problem of the given kind, small enough for the oracle."""
    N = int(rng.integers(1, 3))
    R, S = (int(v) for v in rng.choice([1, 2, 3, 5], size=2))
    sh, sw = (int(v) for v in rng.integers(1, 4, size=2))
    dh, dw = (int(v) for v in rng.integers(1, 3, size=2))
    G = 1
    if kind == "dense":
        C, K = (8 * int(v) for v in rng.integers(1, 13, size=2))
    elif kind == "dense_odd":
        C, K = (int(v) for v in rng.integers(1, 41, size=2))
    elif kind == "grouped":
        # a third each: whole 16-byte channel vectors per group (one implicit
        # GEMM per group); 8-channel vectors on one side and an odd multiple
        # of 4 channels on the other (the LDS-tiled direct kernels); any
        # counts (the one-thread-per-output kernel)
        G = int(rng.integers(2, 5))
        mode = int(rng.integers(0, 3))
        if mode == 0:
            C, K = (G * 8 * int(v) for v in rng.integers(1, 5, size=2))
        elif mode == 1:
            a, b = 8 * int(rng.integers(1, 4)), 4 * (2 * int(rng.integers(0, 3)) + 1)
            C, K = (G * a, G * b) if rng.integers(0, 2) == 0 else (G * b, G * a)
        else:
            C, K = (G * int(v) for v in rng.integers(1, 25, size=2))
    elif kind == "stem":  # few input channels, a wide filter, stride 2 (zero-padded channels)
        C, K = int(rng.integers(1, 8)), 8 * int(rng.integers(1, 9))
        R = S = int(rng.choice([3, 5, 7]))
        sh = sw = 2
        dh = dw = 1
    elif kind == "depthwise":  # most with unit column stride and dilation (row kernels)
        C = K = G = 8 * int(rng.integers(1, 9))
        R, S = (int(v) for v in rng.integers(1, 4, size=2))
        if rng.integers(0, 5) < 3:
            sw = dw = 1
    else:  # band shapes: stride 1, 3x3, 64 source channels
        C, K = 64, 64
        R = S = 3
        sh = sw = 1
        dh = dw = 1 if kind == "wband" else int(rng.integers(1, 3))
    ph, pw = (int(v) for v in rng.integers(0, 4, size=2))
    H = int(rng.integers(1, 15 if kind != "stem" else 30))
    W = int(rng.integers(1, 15 if kind != "stem" else 30))
    if kind == "wband":
        W = 4 * int(rng.integers(1, 4)) + 2 - 2 * 1  # Q = W + 2p - 2, a multiple of 4 with p = 1
        ph = pw = 1
    # grow the input until the dilated filter fits the padded extent
    H = max(H, dh * (R - 1) + 1 - 2 * ph)
    W = max(W, dw * (S - 1) + 1 - 2 * pw)
    return problem(N, C, H, W, K, R, S, pad=(ph, pw), stride=(sh, sw), dil=(dh, dw), groups=G)


@pytest.mark.parametrize("case", range(NCASES))
def test_random_problem(case):
    rng = np.random.default_rng(1000 + case)
    kind = KINDS[case % len(KINDS)]
    prob = draw_problem(rng, kind)
    dtype = "f16" if rng.integers(0, 2) == 0 else "bf16"
    bias, relu = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    P, Q = oracle.output_hw(prob)
    x, w, b, dy = WL.random_case(prob, dtype, "int", 5000 + case, P, Q, bias=bias)
    what = f"case {case} {kind} {dtype} {prob}"
    print(what, flush=True)
    # a random tile of the plan for fprop and dgrad, a random split for wgrad
    algos = []
    for op in (B.CONV2D_OP_FPROP, B.CONV2D_OP_DGRAD):
        n = B.conv2d_plan_info(op, prob, dtype)["num_tiles"]
        algos.append(None if rng.integers(0, 2) == 0 else dict(tile=int(rng.integers(1, n + 1))))
    wal = None if rng.integers(0, 2) == 0 else dict(split_k=int(rng.choice([1, 3, 7])))

    y = run_fprop(prob, dtype, x, w, b, relu, algo=algos[0])
    ref = oracle.fprop(prob, f64(x), f64(w), bias=None if b is None else f64(b), relu=relu)
    check(f64(y), ref, dtype, "exact", f"{what} fprop {algos[0]}")
    dx = run_dgrad(prob, dtype, dy, w, algo=algos[1], fill=float("nan"))
    check(f64(dx), oracle.dgrad(prob, f64(dy), f64(w)), dtype, "exact", f"{what} dgrad {algos[1]}")
    dwt = run_wgrad(prob, dtype, x, dy, algo=wal)
    check(f64(dwt), oracle.wgrad(prob, f64(x), f64(dy)), dtype, "exact", f"{what} wgrad {wal}")
