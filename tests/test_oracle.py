"""Pins of the fp64 CPU oracle against facts fixed outside it.

None of these tests touches the GPU or the HIP library.  Each checks the oracle
against something it does not share code with: page-printed output sizes, brute
force on tiny shapes, closed forms (1x1 == matmul, stride == subsampling,
dilation == zero-inserted filter, groups == block-diagonal), the adjoint
identities, torch's CPU float64 convolution routines, exact rational
arithmetic for the int8 requantisation, and numpy / bit-level enumeration for
the fp16 / bf16 rounding.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from convolution_nhwc_implicit_amd.workloads import problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ints(rng, shape, lo=-4, hi=4):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def rand_problem_inputs(prob, rng):
    P, Q = oracle.output_hw(prob)
    x = ints(rng, (prob["N"], prob["H"], prob["W"], prob["C"]))
    w = ints(rng, (prob["K"], prob["R"], prob["S"], prob["C"] // prob["groups"]))
    dy = ints(rng, (prob["N"], P, Q, prob["K"]))
    return x, w, dy


# ---------------------------------------------------------------- output size

def brute_out_size(inp, pad, k, stride, dil):
    """Count window placements whose every tap lies inside the padded input."""
    span = dil * (k - 1) + 1
    n = 0
    o = 0
    while True:
        start = o * stride  # in padded coordinates
        if start + span > inp + 2 * pad:
            break
        n += 1
        o += 1
    return n if n > 0 else -1


def test_out_size_matches_enumeration():
    for inp in range(1, 24):
        for pad in range(0, 4):
            for k in range(1, 7):
                for stride in range(1, 4):
                    for dil in range(1, 4):
                        assert oracle.out_size(inp, pad, k, stride, dil) == \
                            brute_out_size(inp, pad, k, stride, dil), (inp, pad, k, stride, dil)


def test_out_size_golden_from_pages():
    n = 0
    with open(os.path.join(GOLDEN, "output_sizes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            nums, _src = line.split("|", 1)
            inp, pad, k, stride, dil, out = (int(v) for v in nums.split())
            assert oracle.out_size(inp, pad, k, stride, dil) == out, line
            n += 1
    assert n >= 3


def test_out_size_invalid():
    assert oracle.out_size(2, 0, 3, 1, 1) == -1
    assert oracle.out_size(5, 0, 3, 1, 3) == -1  # dilated span 7 > 5
    assert oracle.out_size(0, 1, 1, 1, 1) == -1
    assert oracle.out_size(8, 1, 3, 0, 1) == -1


# ----------------------------------------------------------- fprop definition

def test_fprop_is_cross_correlation_not_convolution():
    # A one-hot filter at tap (r0, s0) shifts the input by (r0 - pad, s0 - pad):
    # y[p, q] = x[p + r0 - 1, q + s0 - 1].  A flipped (true) convolution would
    # give x[p - r0 + 1, q - s0 + 1] instead.
    prob = problem(1, 1, 6, 7, 1, 3, 3, pad=(1, 1))
    rng = np.random.default_rng(0)
    x = ints(rng, (1, 6, 7, 1))
    for r0, s0 in [(0, 2), (2, 0), (0, 0), (1, 2)]:
        w = np.zeros((1, 3, 3, 1))
        w[0, r0, s0, 0] = 1.0
        y = oracle.fprop(prob, x, w)
        for p in range(6):
            for q in range(7):
                h, ww = p + r0 - 1, q + s0 - 1
                exp = x[0, h, ww, 0] if (0 <= h < 6 and 0 <= ww < 7) else 0.0
                assert y[0, p, q, 0] == exp


def test_identity_filter_gives_input():
    C = 5
    prob = problem(2, C, 5, 4, C, 3, 3, pad=(1, 1))
    rng = np.random.default_rng(1)
    x = ints(rng, (2, 5, 4, C))
    w = np.zeros((C, 3, 3, C))
    for c in range(C):
        w[c, 1, 1, c] = 1.0
    assert np.array_equal(oracle.fprop(prob, x, w), x)


def test_one_by_one_is_matmul():
    rng = np.random.default_rng(2)
    prob = problem(3, 6, 5, 7, 4, 1, 1)
    x = rng.standard_normal((3, 5, 7, 6))
    w = rng.standard_normal((4, 1, 1, 6))
    y = oracle.fprop(prob, x, w)
    ref = x.reshape(-1, 6) @ w.reshape(4, 6).T
    np.testing.assert_allclose(y.reshape(-1, 4), ref, rtol=1e-13, atol=1e-13)
    # strided 1x1: subsample then matmul
    prob2 = problem(3, 6, 5, 7, 4, 1, 1, stride=(2, 3))
    y2 = oracle.fprop(prob2, x, w)
    ref2 = x[:, ::2, ::3, :].reshape(-1, 6) @ w.reshape(4, 6).T
    np.testing.assert_allclose(y2.reshape(-1, 4), ref2, rtol=1e-13, atol=1e-13)


def test_stride_is_subsampled_stride_one():
    rng = np.random.default_rng(3)
    for sh, sw in [(2, 2), (3, 2), (2, 3)]:
        p1 = problem(2, 3, 11, 9, 4, 3, 2, pad=(1, 0))
        ps = dict(p1, stride_h=sh, stride_w=sw)
        x, w, _ = rand_problem_inputs(p1, rng)
        y1 = oracle.fprop(p1, x, w)
        ys = oracle.fprop(ps, x, w)
        assert np.array_equal(ys, y1[:, ::sh, ::sw, :][:, :ys.shape[1], :ys.shape[2], :])


def test_dilation_is_zero_inserted_filter():
    rng = np.random.default_rng(4)
    for dh, dw in [(2, 2), (3, 1), (1, 2)]:
        pd = problem(2, 3, 13, 12, 4, 3, 3, pad=(2, 1), dil=(dh, dw))
        x, w, _ = rand_problem_inputs(pd, rng)
        Re, Se = dh * 2 + 1, dw * 2 + 1
        we = np.zeros((4, Re, Se, 3))
        we[:, ::dh, ::dw, :] = w
        pe = dict(pd, R=Re, S=Se, dil_h=1, dil_w=1)
        assert np.array_equal(oracle.fprop(pd, x, w), oracle.fprop(pe, x, we))


def test_groups_are_independent_dense_convs():
    rng = np.random.default_rng(5)
    G, Cg, Kg = 3, 4, 2
    pg = problem(2, G * Cg, 7, 6, G * Kg, 3, 3, pad=(1, 1), groups=G)
    x, w, dy = rand_problem_inputs(pg, rng)
    y = oracle.fprop(pg, x, w)
    dx = oracle.dgrad(pg, dy, w)
    dw = oracle.wgrad(pg, x, dy)
    for g in range(G):
        pd = dict(pg, C=Cg, K=Kg, groups=1)
        xs = x[..., g * Cg:(g + 1) * Cg]
        ws = w[g * Kg:(g + 1) * Kg]
        dys = dy[..., g * Kg:(g + 1) * Kg]
        assert np.array_equal(y[..., g * Kg:(g + 1) * Kg], oracle.fprop(pd, xs, ws))
        assert np.array_equal(dx[..., g * Cg:(g + 1) * Cg], oracle.dgrad(pd, dys, ws))
        assert np.array_equal(dw[g * Kg:(g + 1) * Kg], oracle.wgrad(pd, xs, dys))


def test_bias_and_relu_epilogue():
    rng = np.random.default_rng(6)
    prob = problem(2, 4, 6, 6, 5, 3, 3, pad=(1, 1))
    x, w, _ = rand_problem_inputs(prob, rng)
    b = ints(rng, (5,))
    y0 = oracle.fprop(prob, x, w)
    yb = oracle.fprop(prob, x, w, bias=b)
    assert np.array_equal(yb, y0 + b)
    yr = oracle.fprop(prob, x, w, bias=b, relu=True)
    assert np.array_equal(yr, np.maximum(y0 + b, 0.0))
    assert not np.any(np.signbit(yr))  # ReLU yields +0, never -0


def test_linear_combination_epilogue():
    """D = alpha*conv + beta*C (the CUTLASS notebook's epilogue): the plain
    pass at (1, 0), beta*C alone at alpha = 0, linear in (alpha, beta), bias
    and ReLU in the plain epilogue's order (exact on integer data)."""
    rng = np.random.default_rng(16)
    prob = problem(2, 4, 7, 6, 5, 3, 3, pad=(1, 1))
    x, w, dy = rand_problem_inputs(prob, rng)
    y = oracle.fprop(prob, x, w)
    c = ints(rng, y.shape)
    b = ints(rng, (5,))
    assert np.array_equal(oracle.linear_combination(y), y)
    assert np.array_equal(oracle.linear_combination(y, bias=b, relu=True),
                          oracle.fprop(prob, x, w, bias=b, relu=True))
    assert np.array_equal(oracle.linear_combination(y, 0.0, 3.0, c), 3.0 * c)
    assert np.array_equal(oracle.linear_combination(y, 0.0, 3.0, c, bias=b), 3.0 * c + b)
    l1 = oracle.linear_combination(y, 2.0, -1.0, c)
    l2 = oracle.linear_combination(y, -0.5, 4.0, c)
    assert np.array_equal(l1 + l2, oracle.linear_combination(y, 1.5, 3.0, c))
    assert np.array_equal(oracle.linear_combination(y, 2.0, 0.0, c), 2.0 * y)
    # ReLU after the sum: where beta*C turns the sign, the result follows the sum
    v = oracle.linear_combination(y, 1.0, -1.0, c, relu=True)
    assert np.array_equal(v > 0, (y - c) > 0)
    assert not np.any(np.signbit(v))
    # dgrad / wgrad results take the same epilogue elementwise
    dx = oracle.dgrad(prob, dy, w)
    cx = ints(rng, dx.shape)
    assert np.array_equal(oracle.linear_combination(dx, 1.0, 1.0, cx) - cx, dx)


# ------------------------------------------------------------ adjoint pins

ADJ_PROBLEMS = [
    problem(2, 3, 7, 6, 4, 3, 3, pad=(1, 1)),
    problem(2, 4, 9, 8, 3, 3, 2, pad=(1, 0), stride=(2, 3)),
    problem(1, 6, 11, 10, 4, 5, 3, pad=(2, 2), stride=(2, 2), dil=(2, 1), groups=2),
    problem(3, 2, 5, 5, 2, 1, 1),
    problem(1, 4, 8, 8, 4, 3, 3, pad=(3, 0), stride=(3, 1), dil=(1, 2), groups=4),
]


@pytest.mark.parametrize("prob", ADJ_PROBLEMS)
def test_adjoint_identities_exact(prob):
    rng = np.random.default_rng(7)
    x, w, dy = rand_problem_inputs(prob, rng)
    y = oracle.fprop(prob, x, w)
    dx = oracle.dgrad(prob, dy, w)
    dw = oracle.wgrad(prob, x, dy)
    a = float(np.sum(y * dy))
    b = float(np.sum(x * dx))
    c = float(np.sum(w * dw))
    assert a == b == c


@pytest.mark.parametrize("prob", ADJ_PROBLEMS)
def test_bias_grad_adjoint_exact(prob):
    """db is the adjoint of the bias add: with a zero filter fprop is the
    broadcast of the bias, so <fprop(x, 0, b), dy> = <b, db>, exactly on
    integer data."""
    rng = np.random.default_rng(9)
    x, w, dy = rand_problem_inputs(prob, rng)
    b = rng.integers(-4, 5, size=prob["K"]).astype(np.float64)
    y = oracle.fprop(prob, x, np.zeros_like(w), bias=b)
    db = oracle.bias_grad(prob, dy)
    assert float(np.sum(y * dy)) == float(np.sum(b * db))


@pytest.mark.parametrize("prob", ADJ_PROBLEMS[:3])
def test_bias_grad_brute_force(prob):
    """The map bias -> fprop(x, 0, bias), built column by column from unit
    bias vectors; bias_grad must be its exact transpose."""
    rng = np.random.default_rng(10)
    x, w, dy = rand_problem_inputs(prob, rng)
    K = prob["K"]
    V = np.empty((dy.size, K))
    for k in range(K):
        e = np.zeros(K)
        e[k] = 1.0
        V[:, k] = oracle.fprop(prob, x, np.zeros_like(w), bias=e).reshape(-1)
    assert np.array_equal(oracle.bias_grad(prob, dy), V.T @ dy.reshape(-1))


@pytest.mark.parametrize("prob", ADJ_PROBLEMS[:3])
def test_dense_operator_brute_force(prob):
    """Build the linear maps x -> fprop(x, w) and w -> fprop(x, w) column by
    column from unit vectors; dgrad and wgrad must be their exact transposes."""
    rng = np.random.default_rng(8)
    x, w, dy = rand_problem_inputs(prob, rng)
    nx, nw = x.size, w.size
    T = np.empty((dy.size, nx))
    for i in range(nx):
        e = np.zeros(nx)
        e[i] = 1.0
        T[:, i] = oracle.fprop(prob, e.reshape(x.shape), w).reshape(-1)
    U = np.empty((dy.size, nw))
    for j in range(nw):
        e = np.zeros(nw)
        e[j] = 1.0
        U[:, j] = oracle.fprop(prob, x, e.reshape(w.shape)).reshape(-1)
    assert np.array_equal(oracle.dgrad(prob, dy, w).reshape(-1), T.T @ dy.reshape(-1))
    assert np.array_equal(oracle.wgrad(prob, x, dy).reshape(-1), U.T @ dy.reshape(-1))
    # fprop itself is linear in x with that operator
    assert np.array_equal(oracle.fprop(prob, x, w).reshape(-1), T @ x.reshape(-1))


# -------------------------------------------------- library cross-check (torch)

TORCH_PROBLEMS = ADJ_PROBLEMS + [
    problem(2, 8, 8, 8, 16, 3, 3, pad=(1, 1)),
    problem(2, 16, 14, 13, 8, 3, 3, pad=(1, 1), stride=(2, 2)),
    problem(2, 8, 17, 17, 12, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)),
    problem(2, 8, 17, 17, 8, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2), groups=4),
]


@pytest.mark.parametrize("prob", TORCH_PROBLEMS)
def test_matches_torch_cpu_float64(prob):
    rng = np.random.default_rng(9)
    x, w, dy = rand_problem_inputs(prob, rng)
    kw = dict(stride=(prob["stride_h"], prob["stride_w"]), padding=(prob["pad_h"], prob["pad_w"]),
              dilation=(prob["dil_h"], prob["dil_w"]), groups=prob["groups"])
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w).permute(0, 3, 1, 2)
    dyt = torch.from_numpy(dy).permute(0, 3, 1, 2)
    y_t = torch.nn.functional.conv2d(xt, wt, **kw).permute(0, 2, 3, 1).numpy()
    dx_t = torch.nn.grad.conv2d_input(xt.shape, wt, dyt, **kw).permute(0, 2, 3, 1).numpy()
    dw_t = torch.nn.grad.conv2d_weight(xt, wt.shape, dyt, **kw).permute(0, 2, 3, 1).numpy()
    assert np.array_equal(oracle.fprop(prob, x, w), y_t)
    assert np.array_equal(oracle.dgrad(prob, dy, w), dx_t)
    assert np.array_equal(oracle.wgrad(prob, x, dy), dw_t)


def test_sampled_equals_full():
    rng = np.random.default_rng(10)
    prob = problem(2, 6, 9, 8, 4, 3, 3, pad=(1, 2), stride=(2, 1), dil=(1, 2), groups=2)
    x, w, dy = rand_problem_inputs(prob, rng)
    b = ints(rng, (4,))
    y = oracle.fprop(prob, x, w, bias=b, relu=True).reshape(-1)
    dx = oracle.dgrad(prob, dy, w).reshape(-1)
    dw = oracle.wgrad(prob, x, dy).reshape(-1)
    for full, fn in [(y, lambda i: oracle.fprop_sampled(prob, x, w, i, bias=b, relu=True)),
                     (dx, lambda i: oracle.dgrad_sampled(prob, dy, w, i)),
                     (dw, lambda i: oracle.wgrad_sampled(prob, x, dy, i))]:
        idx = rng.integers(0, full.size, size=50)
        assert np.array_equal(fn(idx), full[idx])


# ------------------------------------------------------------ int8 requant

def rne_rational(v, num, den):
    """Round v*num/den half to even with exact integer arithmetic."""
    q, r = divmod(v * num, den)
    if 2 * r > den or (2 * r == den and q % 2 == 1):
        q += 1
    return q


def test_requant_multiplier_is_double_product():
    m = oracle.requant_multiplier(0.02, 0.01, 0.05)
    assert m == 0.02 * 0.01 / 0.05


def test_requant_matches_exact_rational_rounding():
    # scales act 0.02, w 0.01, out 0.05 -> exact multiplier 1/250.  Every value
    # of the unsaturated band and all ties v = 250n + 125 lie in this range.
    m = oracle.requant_multiplier(0.02, 0.01, 0.05)
    v = np.arange(-40000, 40000, dtype=np.int64)
    for relu in (False, True):
        got = oracle.requant(v.astype(np.float64), K=1, relu=relu, multiplier=m)
        frac = Fraction(2, 100) * Fraction(1, 100) / Fraction(5, 100)
        assert frac == Fraction(1, 250)
        exp = np.array([rne_rational(max(int(t), 0) if relu else int(t), 1, 250) for t in v])
        exp = np.clip(exp, -128, 127)
        assert np.array_equal(got.astype(np.int64), exp)


def test_requant_bias_relu_saturation():
    rng = np.random.default_rng(11)
    K = 7
    acc = rng.integers(-200000, 200000, size=K * 50).astype(np.float64)
    bias = rng.integers(-(1 << 15), 1 << 15, size=K).astype(np.int32)
    m = oracle.requant_multiplier(0.02, 0.01, 0.05)
    q = oracle.requant(acc, K, bias=bias, relu=True, multiplier=m)
    v = acc.astype(np.int64) + np.tile(bias.astype(np.int64), 50)
    assert q.min() >= 0 and q.max() <= 127
    assert np.all(q[v >= 127 * 250 + 125] == 127)
    assert np.all(q[v <= 0] == 0)
    q2 = oracle.requant(acc, K, bias=bias, relu=False, multiplier=m)
    assert np.all(q2[v <= -128 * 250 - 125] == -128)
    # the idx form picks the same bias channel as the dense form
    idx = np.arange(acc.size)
    assert np.array_equal(oracle.requant(acc, K, bias=bias, relu=True, multiplier=m, idx=idx), q)


# ------------------------------------------------------------- rounding

def test_round_f16_matches_numpy():
    rng = np.random.default_rng(12)
    v = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e-8, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, np.inf, -np.inf, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0]),
    ])
    got = oracle.round_f16(v)
    exp = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, exp)


def bf16_value(bits):
    return oracle.bits_to_f64(np.asarray(bits, dtype=np.uint16), "bf16")


def test_round_bf16_is_nearest_even():
    rng = np.random.default_rng(13)
    v = rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)
    # exact ties between neighbours: midpoints of random bf16 pairs
    b = rng.integers(0, 0x7F7F, size=2000).astype(np.uint16)
    mid = (bf16_value(b) + bf16_value(b + 1)) / 2.0
    v = np.concatenate([v, mid, -mid, [0.0, 2.0 ** -133, 2.0 ** -134, 3.0 * 2.0 ** -135]])
    got = oracle.round_bf16(v)
    gv = bf16_value(got)
    a = np.abs(v)
    mag = got & 0x7FFF
    lo = bf16_value(np.maximum(mag.astype(np.int64) - 1, 0).astype(np.uint16))
    hi = bf16_value((mag + 1).astype(np.uint16))
    # |v| lies between the neighbours of the chosen value and is no closer to either
    assert np.all(np.abs(np.abs(gv) - a) <= np.abs(lo - a))
    assert np.all(np.abs(np.abs(gv) - a) <= np.abs(hi - a))
    # ties go to the even mantissa
    tie = (np.abs(np.abs(gv) - a) == np.abs(lo - a)) | (np.abs(np.abs(gv) - a) == np.abs(hi - a))
    tie &= a > 0
    assert np.all(mag[tie] % 2 == 0)
    assert np.all(np.signbit(gv) == np.signbit(v))


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(14)
    v32 = (rng.standard_normal(200000) * 10.0 ** rng.integers(-20, 20, 200000)).astype(np.float32)
    v32 = v32[np.isfinite(v32)]
    exp = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(v32.astype(np.float64))
    assert np.array_equal(got, exp)


def test_round_overflow_to_inf():
    got = oracle.round_bf16(np.array([3.4e38, 3.39e38, -1e39]))
    assert math.isinf(bf16_value(got[2])) and bf16_value(got[2]) < 0
    assert np.isfinite(bf16_value(got[1]))


# ---- Winograd F(2x2, 3x3) (oracle.winograd), pinned to the direct definition
WINO_CASES = [(2, 5, 7, 9, 3, 1), (1, 3, 6, 6, 4, 0), (2, 4, 5, 8, 2, 2), (1, 2, 1, 1, 3, 1), (3, 8, 12, 11, 5, 1)]


@pytest.mark.parametrize("N,C,H,W,K,pad", WINO_CASES)
def test_winograd_matches_direct(N, C, H, W, K, pad):
    """The transforms, products and inverse transform reproduce the direct
    convolution (odd P and Q leave partial 2x2 blocks; pads 0, 1, 2)."""
    from oracle import winograd as WG
    prob = problem(N, C, H, W, K, 3, 3, pad=(pad, pad))
    rng = np.random.default_rng(N * 1000 + C * 100 + H)
    x, w, b = rng.standard_normal((N, H, W, C)), rng.standard_normal((K, 3, 3, C)), rng.standard_normal(K)
    yd = oracle.fprop(prob, x, w, bias=b, relu=True)
    yw = WG.fprop(prob, x, w, bias=b, relu=True)
    assert yw.shape == yd.shape
    assert np.max(np.abs(yw - yd)) <= 1e-12 * np.max(np.abs(yd))
    # every output is a signed sum of the terms S adds up in absolute value
    assert np.all(np.abs(oracle.fprop(prob, x, w)) <= WG.abs_terms(prob, x, w) * (1 + 1e-12))


def test_winograd_single_tap_and_errors():
    """A filter with one nonzero tap gives the shifted input times that tap;
    other problem shapes are refused."""
    from oracle import winograd as WG
    prob = problem(1, 2, 5, 6, 2, 3, 3, pad=(1, 1))
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 5, 6, 2))
    w = np.zeros((2, 3, 3, 2))
    w[0, 2, 0, 1] = 3.0  # y[p, q, 0] = 3 x[p + 1, q - 1, 1]
    y = WG.fprop(prob, x, w)
    want = np.zeros((1, 5, 6))
    want[0, :4, 1:] = 3.0 * x[0, 1:, :5, 1]
    assert np.allclose(y[..., 0], want, rtol=0, atol=1e-13)
    assert np.all(y[..., 1] == 0)
    with pytest.raises(ValueError):
        WG.fprop(problem(1, 2, 5, 6, 2, 3, 3, pad=(1, 1), stride=(2, 2)), x, w)


# ---- oracle.winograd.error_bound pinned from both sides by a simulation of
# the rounded arithmetic: U = G g G^T and V = B^T d B formed in fp32 and
# rounded once to the 16-bit type, fp32 products and sums over the channels
# in order, the inverse transform in fp32 (no output rounding).  The bound must
# hold for every output, and must not be loose: with one channel (few terms,
# little cancellation of rounding errors) the worst output reaches a quarter of
# it, with 64 channels (the kernel's shape) a twenty-fifth.
def _wino_rounded_sim(prob, x, w, dtype):
    from oracle import winograd as WG
    f32 = np.float32

    def r16(a):
        return oracle.bits_to_f64(oracle.round_to(np.asarray(a, dtype=np.float64), dtype), dtype).astype(f32)

    d, P, Q = WG._tiles(prob, x)
    G, BT, AT = WG.G.astype(f32), WG.BT.astype(f32), WG.AT.astype(f32)
    U = np.einsum("kasc,bs->kabc", np.einsum("ar,krsc->kasc", G, w.astype(f32)).astype(f32), G).astype(f32)
    V = np.einsum("ntqajc,bj->ntqabc", np.einsum("ai,ntqijc->ntqajc", BT, d.astype(f32)).astype(f32),
                  BT).astype(f32)
    U, V = r16(U), r16(V)
    M = np.zeros(V.shape[:5] + (w.shape[0],), dtype=f32)
    for c in range(x.shape[-1]):
        M = (M + np.einsum("kab,ntqab->ntqabk", U[..., c], V[..., c]).astype(f32)).astype(f32)
    Yb = np.einsum("ntqybk,xb->ntqyxk", np.einsum("ya,ntqabk->ntqybk", AT, M).astype(f32), AT).astype(f32)
    N, TP, TQ = Yb.shape[:3]
    return Yb.transpose(0, 1, 3, 2, 4, 5).reshape(N, 2 * TP, 2 * TQ, -1)[:, :P, :Q, :].astype(np.float64)


@pytest.mark.parametrize("dtype,u", [("f16", 2.0 ** -11), ("bf16", 2.0 ** -8)])
@pytest.mark.parametrize("C,floor", [(1, 0.25), (64, 0.04)])
def test_winograd_error_bound_holds_and_is_tight(dtype, u, C, floor):
    from oracle import winograd as WG
    from convolution_nhwc_implicit_amd.workloads import draw
    prob = problem(2, C, 9, 11, 8, 3, 3, pad=(1, 1))
    rng = np.random.default_rng(900 + C)
    x = draw((2, 9, 11, C), dtype, "gauss", rng).to(torch.float64).numpy()
    w = draw((8, 3, 3, C), dtype, "gauss", rng, std=1.0 / np.sqrt(9 * C)).to(torch.float64).numpy()
    y = oracle.fprop(prob, x, w)
    ratio = np.abs(_wino_rounded_sim(prob, x, w, dtype) - y) / WG.error_bound(prob, x, w, u)
    assert ratio.max() <= 1.0, f"simulated rounding exceeds the bound: {ratio.max():.3f}"
    assert ratio.max() >= floor, f"bound loose: worst simulated error is {ratio.max():.3f} of it"


def test_winograd_error_bound_catches_a_dropped_rounding():
    """The simulation must separate a right bound from a wrong one: rounding
    only V (the filter transform left exact) gives a bound that the full
    rounding exceeds on some output."""
    from oracle import winograd as WG
    from convolution_nhwc_implicit_amd.workloads import draw
    prob = problem(2, 1, 9, 11, 8, 3, 3, pad=(1, 1))
    rng = np.random.default_rng(901)
    x = draw((2, 9, 11, 1), "f16", "gauss", rng).to(torch.float64).numpy()
    w = draw((8, 3, 3, 1), "f16", "gauss", rng, std=1.0 / 3).to(torch.float64).numpy()
    u = 2.0 ** -11
    y = oracle.fprop(prob, x, w)
    err = np.abs(_wino_rounded_sim(prob, x, w, "f16") - y)
    half = 1.01 * (u + 42 * 2.0 ** -24) * WG.abs_terms(prob, x, w)  # one operand's rounding only
    assert np.any(err > half)
    assert np.all(err <= WG.error_bound(prob, x, w, u))
