"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, and compare.

Comparison rules:
  exact  -- integer-valued fp16/bf16 data and int8: every partial sum is an
            exact integer below 2^24 in the fp32/int32 accumulator, so the one
            rounding at the end is unique; the GPU must equal the oracle's
            fp64 result rounded once to the output type (numeric equality,
            so -0 == +0).
  tol    -- Gaussian data: max_rel = max|g - ref_hi| / max|ref_hi| <= 5e-3 and
            rms_scaled = ||g - ref_out|| / ||ref_out|| <= 1e-3, where ref_hi is
            the oracle's fp64 value and ref_out that value rounded once to the
            output type.
"""
import numpy as np
import torch

import oracle
from convolution_nhwc_implicit_amd import binding as B

MAX_REL = 5e-3
RMS_SCALED = 1e-3
DEV = "cuda"


def f64(t):
    """Exact float64 copy of a CPU or GPU tensor."""
    t = t.detach().cpu()
    if t.dtype in (torch.int8, torch.int32):
        return t.numpy().astype(np.float64)
    return t.to(torch.float64).numpy()


def rounded(ref_hi, dtype):
    return oracle.bits_to_f64(oracle.round_to(ref_hi, dtype), dtype)


def check(g, ref_hi, dtype, mode, what=""):
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    ref_hi = np.asarray(ref_hi, dtype=np.float64).reshape(-1)
    assert g.shape == ref_hi.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    ref_out = rounded(ref_hi, dtype)
    if mode == "exact":
        bad = np.nonzero(g != ref_out)[0]
        assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ; first at {bad[:5]}: "
                               f"gpu {g[bad[:5]]} oracle {ref_out[bad[:5]]}")
        return 0.0, 0.0
    scale = np.max(np.abs(ref_hi))
    max_rel = float(np.max(np.abs(g - ref_hi)) / scale) if scale > 0 else float(np.max(np.abs(g)))
    den = np.linalg.norm(ref_out)
    rms = float(np.linalg.norm(g - ref_out) / den) if den > 0 else float(np.linalg.norm(g))
    assert max_rel <= MAX_REL, f"{what}: max_rel {max_rel:.3e} > {MAX_REL}"
    assert rms <= RMS_SCALED, f"{what}: rms_scaled {rms:.3e} > {RMS_SCALED}"
    return max_rel, rms


def gpu(t):
    return None if t is None else t.to(DEV).contiguous()


def run_fprop(prob, dtype, x, w, bias, relu, scales=None, algo=None):
    P, Q = B.conv2d_output_size(prob)
    y = torch.empty((prob["N"], P, Q, prob["K"]), dtype=x.dtype, device=DEV)
    ws = B.workspace_for(B.CONV2D_OP_FPROP, prob, dtype, DEV, algo)
    act, wsc, out = scales if scales else (1.0, 1.0, 1.0)
    B.conv2d_fprop(prob, dtype, gpu(x), gpu(w), gpu(bias), relu, act, wsc, out, y, ws, algo)
    torch.cuda.synchronize()
    return y


def run_dgrad(prob, dtype, dy, w, algo=None, fill=None):
    dx = torch.empty((prob["N"], prob["H"], prob["W"], prob["C"]), dtype=dy.dtype, device=DEV)
    if fill is not None:
        dx.fill_(fill)
    ws = B.workspace_for(B.CONV2D_OP_DGRAD, prob, dtype, DEV, algo)
    B.conv2d_dgrad(prob, dtype, gpu(dy), gpu(w), dx, ws, algo)
    torch.cuda.synchronize()
    return dx


def run_wgrad(prob, dtype, x, dy, algo=None):
    dw = torch.empty((prob["K"], prob["R"], prob["S"], prob["C"] // prob["groups"]), dtype=x.dtype,
                     device=DEV)
    ws = B.workspace_for(B.CONV2D_OP_WGRAD, prob, dtype, DEV, algo)
    B.conv2d_wgrad(prob, dtype, gpu(x), gpu(dy), dw, ws, algo)
    torch.cuda.synchronize()
    return dw


def oracle_fprop_out(prob, dtype, x, w, bias, relu, scales=None, idx=None):
    """Oracle fprop (fp64 ref_hi, or int8 codes for dtype i8), full or at idx."""
    xb, wb = f64(x), f64(w)
    if dtype == "i8":
        acc = oracle.fprop(prob, xb, wb) if idx is None else oracle.fprop_sampled(prob, xb, wb, idx)
        m = oracle.requant_multiplier(*scales)
        b = None if bias is None else bias.numpy()
        return oracle.requant(acc.reshape(-1), prob["K"], bias=b, relu=relu, multiplier=m, idx=idx)
    bb = None if bias is None else f64(bias)
    if idx is None:
        return oracle.fprop(prob, xb, wb, bias=bb, relu=relu)
    return oracle.fprop_sampled(prob, xb, wb, idx, bias=bb, relu=relu)


def sample_indices(total, n, seed):
    rng = np.random.default_rng(seed)
    edge = np.array([0, 1, total // 2, total - 2, total - 1], dtype=np.int64)
    return np.unique(np.concatenate([edge[(edge >= 0) & (edge < total)],
                                     rng.integers(0, total, size=n)]))
