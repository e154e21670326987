"""Synthetic conv2d workloads and their seeded input generators.

This module holds data only: problem sizes, value distributions and seeded
random draws.  It contains no convolution arithmetic, so both the HIP library's
tests and the independent CPU oracle can take their inputs from it.

Workloads (sizes and distributions follow the pages' own examples):
  c1_tiny        fp16 integer-valued, 2x8x8x8 -> 16, 3x3 s1 p1, bias
  c2_strided     fp16 integer-valued, 32x28x28x64 -> 128, 3x3 s2 p1, bias
                 (the shape of the CUTLASS Python Conv2d notebook, "General setup")
  c3a_resnet3x3  fp16 Gaussian, 64x56x56x64 -> 64, 3x3 s1 p1, bias + ReLU
  c3b_resnet1x1  fp16 Gaussian, same input, 64 -> 256, 1x1, bias + ReLU
  c4_awkward     bf16 Gaussian, 16x57x57x96 -> 192, 5x5 s2 p2 d2
  c4g_grouped    bf16 Gaussian, same input, groups 4, 96 -> 96 (24 per group)
  c5_int8        int8 uniform, 32x56x56x128 -> 128, 3x3 s1 p1, int32 bias, ReLU,
                 requantised with scales act 0.02, w 0.01, out 0.05
  n1_stem        fp16 Gaussian, 32x224x224x3 -> 64, 7x7 s2 p3, bias + ReLU (a
                 three-channel image stem, the small-C case; cfg 5)
  d1_depthwise   fp16 Gaussian, 32x56x56x128 -> 128, 3x3 s1 p1, groups 128
                 (depthwise), bias + ReLU (cfg 6)

Integer-valued data is ceil(U(-4.5, 3.5)), the draw the CUTLASS notebook uses
so that fp16 products and fp32 sums are exact.  Its values are -4..4.

Seeds: numpy PCG64(1234 + 16*cfg + tensor_index), cfg = 0..4 for c1..c5 (5 for n1_stem, 6 for d1_depthwise),
tensor_index x=0, w=1, bias=2, dy=3, and 4/5/6 for the filter, bias and dy of
the variant that shares its input with the base config (c3b, c4g).

Gaussian values are drawn in float64, scaled, rounded to float32 and then to
the element type (round to nearest even at each step).  Filters have standard
deviation 1/sqrt(C/G*R*S) so outputs have about unit variance.
"""
import math

import numpy as np
import torch


def problem(N, C, H, W, K, R, S, pad=(0, 0), stride=(1, 1), dil=(1, 1), groups=1):
    """A conv2d problem as the plain mapping the binding and the oracle take."""
    return dict(N=N, C=C, H=H, W=W, K=K, R=R, S=S,
                pad_h=pad[0], pad_w=pad[1], stride_h=stride[0], stride_w=stride[1],
                dil_h=dil[0], dil_w=dil[1], groups=groups)


WORKLOADS = {
    "c1_tiny": dict(
        prob=problem(2, 8, 8, 8, 16, 3, 3, pad=(1, 1)),
        dtype="f16", dist="int", cfg=0, idx=dict(x=0, w=1, bias=2, dy=3),
        bias=True, relu=False, check="exact"),
    "c2_strided": dict(
        prob=problem(32, 64, 28, 28, 128, 3, 3, pad=(1, 1), stride=(2, 2)),
        dtype="f16", dist="int", cfg=1, idx=dict(x=0, w=1, bias=2, dy=3),
        bias=True, relu=False, check="exact"),
    "c3a_resnet3x3": dict(
        prob=problem(64, 64, 56, 56, 64, 3, 3, pad=(1, 1)),
        dtype="f16", dist="gauss", cfg=2, idx=dict(x=0, w=1, bias=2, dy=3),
        bias=True, relu=True, check="tol"),
    "c3b_resnet1x1": dict(
        prob=problem(64, 64, 56, 56, 256, 1, 1),
        dtype="f16", dist="gauss", cfg=2, idx=dict(x=0, w=4, bias=5, dy=6),
        bias=True, relu=True, check="tol"),
    "c4_awkward": dict(
        prob=problem(16, 96, 57, 57, 192, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2)),
        dtype="bf16", dist="gauss", cfg=3, idx=dict(x=0, w=1, bias=2, dy=3),
        bias=False, relu=False, check="tol"),
    "c4g_grouped": dict(
        prob=problem(16, 96, 57, 57, 96, 5, 5, pad=(2, 2), stride=(2, 2), dil=(2, 2), groups=4),
        dtype="bf16", dist="gauss", cfg=3, idx=dict(x=0, w=4, bias=5, dy=6),
        bias=False, relu=False, check="tol"),
    "c5_int8": dict(
        prob=problem(32, 128, 56, 56, 128, 3, 3, pad=(1, 1)),
        dtype="i8", dist="uniform_i8", cfg=4, idx=dict(x=0, w=1, bias=2, dy=3),
        bias=True, relu=True, check="exact", scales=(0.02, 0.01, 0.05)),
    "n1_stem": dict(
        prob=problem(32, 3, 224, 224, 64, 7, 7, pad=(3, 3), stride=(2, 2)),
        dtype="f16", dist="gauss", cfg=5, idx=dict(x=0, w=1, bias=2, dy=3),
        bias=True, relu=True, check="tol"),
    "d1_depthwise": dict(
        prob=problem(32, 128, 56, 56, 128, 3, 3, pad=(1, 1), groups=128),
        dtype="f16", dist="gauss", cfg=6, idx=dict(x=0, w=1, bias=2, dy=3),
        bias=True, relu=True, check="tol"),
}

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}


def rng_for(cfg, tensor_index):
    return np.random.Generator(np.random.PCG64(1234 + 16 * cfg + tensor_index))


def _to_dtype(a64, dtype):
    if dtype == "i8":
        return torch.from_numpy(np.ascontiguousarray(a64.astype(np.int8)))
    t32 = torch.from_numpy(np.ascontiguousarray(a64.astype(np.float32)))
    return t32.to(TORCH_DTYPE[dtype]).contiguous()


def draw(shape, dtype, dist, rng, std=1.0):
    """One seeded tensor (torch, CPU, contiguous) of the given distribution."""
    shape = tuple(int(s) for s in shape)
    if dist == "int":
        return _to_dtype(np.ceil(rng.uniform(-4.5, 3.5, size=shape)), dtype)
    if dist == "gauss":
        return _to_dtype(rng.standard_normal(size=shape) * std, dtype)
    if dist == "uniform_i8":
        return torch.from_numpy(rng.integers(-128, 128, size=shape, dtype=np.int8))
    if dist == "bias_i32":
        return torch.from_numpy(rng.integers(-(1 << 15), 1 << 15, size=shape, dtype=np.int32))
    raise ValueError(dist)


def filter_std(prob):
    return 1.0 / math.sqrt(prob["C"] // prob["groups"] * prob["R"] * prob["S"])


def make_x(name):
    wl = WORKLOADS[name]
    p = wl["prob"]
    return draw((p["N"], p["H"], p["W"], p["C"]), wl["dtype"], wl["dist"],
                rng_for(wl["cfg"], wl["idx"]["x"]))


def make_w(name):
    wl = WORKLOADS[name]
    p = wl["prob"]
    return draw((p["K"], p["R"], p["S"], p["C"] // p["groups"]), wl["dtype"], wl["dist"],
                rng_for(wl["cfg"], wl["idx"]["w"]), std=filter_std(p))


def make_bias(name):
    wl = WORKLOADS[name]
    p = wl["prob"]
    rng = rng_for(wl["cfg"], wl["idx"]["bias"])
    if wl["dtype"] == "i8":
        return draw((p["K"],), "i8", "bias_i32", rng)
    return draw((p["K"],), wl["dtype"], wl["dist"], rng)


def make_dy(name, P, Q):
    """Output gradient [N,P,Q,K]; P and Q are supplied by the caller."""
    wl = WORKLOADS[name]
    p = wl["prob"]
    return draw((p["N"], P, Q, p["K"]), wl["dtype"], wl["dist"],
                rng_for(wl["cfg"], wl["idx"]["dy"]))


def random_case(prob, dtype, dist, seed, P, Q, bias=True):
    """Inputs for an ad-hoc problem (parity sweeps): x, w, bias, dy."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = draw((prob["N"], prob["H"], prob["W"], prob["C"]), dtype, dist, rng)
    w = draw((prob["K"], prob["R"], prob["S"], prob["C"] // prob["groups"]), dtype, dist, rng,
             std=filter_std(prob))
    if not bias:
        b = None
    elif dtype == "i8":
        b = draw((prob["K"],), "i8", "bias_i32", rng)
    else:
        b = draw((prob["K"],), dtype, dist, rng)
    dy = draw((prob["N"], P, Q, prob["K"]), dtype, dist, rng)
    return x, w, b, dy
