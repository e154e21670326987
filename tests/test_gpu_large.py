"""Tensors past 2^31 bytes: the buffer and element offsets of the band kernels
(per image), the pointwise kernel and the implicit GEMM (whole tensor) near
the 32-bit limits the host plan allows.  x is 8 x 1536 x 1536 x 64 fp16 (2.4 GB, 1.2e9 elements);
integer-valued data in -4..4, so every sum is exact.  Outputs are checked at
sampled points against the oracle run on the sampled point's receptive field
(a 3x3 patch, zero outside the image) as a one-pixel problem."""
import numpy as np
import pytest
import torch

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd.workloads import problem

from parity import check

pytestmark = pytest.mark.gpu

N, H, W, C, K = 8, 1536, 1536, 64, 64


def big_int_tensor(shape, seed):
    """Seeded integers in -4..4, drawn as int8 on the host, widened to fp16 on the GPU."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.integers(-4, 5, size=shape, dtype=np.int8)
    return torch.from_numpy(a).to("cuda").to(torch.float16)


def patch(t, n, h, w):
    """t[n, h-1..h+1, w-1..w+1, :] as fp64, zero outside the image."""
    out = np.zeros((1, 3, 3, t.shape[3]), dtype=np.float64)
    for dr in range(3):
        for ds in range(3):
            hh, ww = h - 1 + dr, w - 1 + ds
            if 0 <= hh < t.shape[1] and 0 <= ww < t.shape[2]:
                out[0, dr, ds] = t[n, hh, ww].float().cpu().numpy()
    return out


def sample_points(seed, count=24):
    rng = np.random.default_rng(seed)
    pts = [(0, 0, 0), (N - 1, H - 1, W - 1), (N - 1, 0, W - 1), (N // 2, H // 2, W // 2)]
    pts += [(int(rng.integers(0, N)), int(rng.integers(0, H)), int(rng.integers(0, W))) for _ in range(count)]
    return pts


def test_large_tensors_band_and_igemm():
    prob = problem(N, C, H, W, K, 3, 3, pad=(1, 1))
    assert 2 * N * H * W * C > 2 ** 31
    print("drawing x", flush=True)
    x = big_int_tensor((N, H, W, C), 901)
    rng = np.random.default_rng(902)
    w = torch.from_numpy(rng.integers(-4, 5, size=(K, 3, 3, C)).astype(np.float16)).cuda()
    w1 = torch.from_numpy(rng.integers(-4, 5, size=(K, 1, 1, C)).astype(np.float16)).cuda()
    w64, w164 = w.double().cpu().numpy(), w1.double().cpu().numpy()
    assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, prob, "f16")["tile"] == 5  # band kernel
    print("fprop 3x3 (band)", flush=True)
    y = torch.empty((N, H, W, K), dtype=torch.float16, device="cuda")
    B.conv2d_fprop(prob, "f16", x, w, None, False, 1.0, 1.0, 1.0, y, None)
    torch.cuda.synchronize()
    one = problem(1, C, 3, 3, K, 3, 3)
    for (n, h, ww) in sample_points(903):
        ref = oracle.fprop(one, patch(x, n, h, ww), w64).reshape(-1)
        check(y[n, h, ww].double().cpu().numpy(), ref, "f16", "exact", f"fprop band at {(n, h, ww)}")
    del y
    p1 = problem(N, C, H, W, K, 1, 1)
    assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, p1, "f16")["kernel"] == 5  # pointwise
    y1 = torch.empty((N, H, W, K), dtype=torch.float16, device="cuda")
    for algo, name in ((None, "pointwise"), (dict(tile=1), "implicit GEMM")):
        print(f"fprop 1x1 ({name})", flush=True)
        y1.fill_(float("nan"))
        B.conv2d_fprop(p1, "f16", x, w1, None, False, 1.0, 1.0, 1.0, y1, None, algo)
        torch.cuda.synchronize()
        for (n, h, ww) in sample_points(904):
            ref = oracle.fprop(problem(1, C, 1, 1, K, 1, 1),
                               x[n, h, ww].double().cpu().numpy().reshape(1, 1, 1, C), w164).reshape(-1)
            check(y1[n, h, ww].double().cpu().numpy(), ref, "f16", "exact", f"fprop 1x1 {name} at {(n, h, ww)}")
    del y1, x
    print("drawing dy, dgrad 3x3 (band)", flush=True)
    dy = big_int_tensor((N, H, W, K), 905)
    assert B.conv2d_plan_info(B.CONV2D_OP_DGRAD, prob, "f16")["tile"] == 5
    dx = torch.empty((N, H, W, C), dtype=torch.float16, device="cuda")
    B.conv2d_dgrad(prob, "f16", dy, w, dx, None)
    torch.cuda.synchronize()
    onep = problem(1, C, 3, 3, K, 3, 3, pad=(1, 1))
    for (n, h, ww) in sample_points(906):
        ref = oracle.dgrad(onep, patch(dy, n, h, ww), w64)[0, 1, 1]
        check(dx[n, h, ww].double().cpu().numpy(), ref, "f16", "exact", f"dgrad band at {(n, h, ww)}")


def test_large_wgrad_far_rows():
    """wgrad over the same 2.4 GB x with dy zero except in the last three
    output rows of the last image: every slice runs, the only non-zero terms
    sit at the far end of both tensors, and dw equals the oracle's wgrad of
    the 4-row strip those rows read (exact on integer data)."""
    prob = problem(N, C, H, W, K, 3, 3, pad=(1, 1))
    x = big_int_tensor((N, H, W, C), 901)
    rng = np.random.Generator(np.random.PCG64(907))
    dy = torch.zeros((N, H, W, K), dtype=torch.float16, device="cuda")
    dy[N - 1, H - 3:] = torch.from_numpy(rng.integers(-4, 5, size=(3, W, K)).astype(np.float16)).cuda()
    strip = problem(1, C, 4, W, K, 3, 3, pad=(1, 1))
    ref = oracle.wgrad(strip, x[N - 1:, H - 4:].double().cpu().numpy(), dy[N - 1:, H - 4:].double().cpu().numpy())
    info = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")
    assert info["num_tiles"] == 2, info
    for t in (1, 2):
        algo = dict(tile=t)
        print(f"wgrad tile {t}", flush=True)
        ws = B.workspace_for(B.CONV2D_OP_WGRAD, prob, "f16", "cuda", algo)
        dw = torch.empty((K, 3, 3, C), dtype=torch.float16, device="cuda")
        B.conv2d_wgrad(prob, "f16", x, dy, dw, ws, algo)
        torch.cuda.synchronize()
        check(dw.double().cpu().numpy(), ref, "f16", "exact", f"wgrad tile {t}")
