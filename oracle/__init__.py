"""fp64 CPU oracle for NHWC conv2d -- TEST INFRASTRUCTURE ONLY.

This package is the checker of the HIP library, not part of it.  Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the library never does, and the two share no code.

The arithmetic lives in ``conv2d_oracle.c`` (plain C, double precision, one
output element at a time).  This module only marshals numpy arrays to it.
``oracle.winograd`` (numpy, fp64) writes out the Winograd F(2x2, 3x3) steps
for stride-1 3x3 layers and the per-output bound on its rounding error.

A problem is a mapping with the keys N, C, H, W, K, R, S, pad_h, pad_w,
stride_h, stride_w, dil_h, dil_w, groups.  Tensors are float64 numpy arrays in
the layouts x/dx [N,H,W,C], w/dw [K,R,S,C/G], y/dy [N,P,Q,K].
"""
import ctypes

import numpy as np

from . import build as _build

_KEYS = ("N", "C", "H", "W", "K", "R", "S", "pad_h", "pad_w",
         "stride_h", "stride_w", "dil_h", "dil_w", "groups")

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_out_size.restype = ctypes.c_int
        lib.oracle_out_size.argtypes = [ctypes.c_int] * 5
        lib.oracle_threads.restype = ctypes.c_int
        for name in ("oracle_fprop",):
            getattr(lib, name).argtypes = [ip, dp, dp, dp, ctypes.c_int, dp]
        lib.oracle_dgrad.argtypes = [ip, dp, dp, dp]
        lib.oracle_wgrad.argtypes = [ip, dp, dp, dp]
        lib.oracle_bias_grad.argtypes = [ip, dp, dp]
        lib.oracle_fprop_sampled.argtypes = [ip, dp, dp, dp, ctypes.c_int, i64p, ctypes.c_long, dp]
        lib.oracle_dgrad_sampled.argtypes = [ip, dp, dp, i64p, ctypes.c_long, dp]
        lib.oracle_wgrad_sampled.argtypes = [ip, dp, dp, i64p, ctypes.c_long, dp]
        lib.oracle_linear_combination.argtypes = [dp, dp, ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                                   ctypes.c_double, dp, ctypes.c_int, dp]
        lib.oracle_requant_multiplier.restype = ctypes.c_double
        lib.oracle_requant_multiplier.argtypes = [ctypes.c_double] * 3
        lib.oracle_requant.argtypes = [dp, i64p, ctypes.c_long, ctypes.c_long,
                                       ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                       ctypes.c_double, ctypes.POINTER(ctypes.c_int8)]
        u16p = ctypes.POINTER(ctypes.c_uint16)
        lib.oracle_round_f16.argtypes = [dp, ctypes.c_long, u16p]
        lib.oracle_round_bf16.argtypes = [dp, ctypes.c_long, u16p]
        for name in ("oracle_fprop", "oracle_dgrad", "oracle_wgrad", "oracle_fprop_sampled",
                     "oracle_dgrad_sampled", "oracle_wgrad_sampled", "oracle_bias_grad"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _dims(prob):
    arr = (ctypes.c_int * 14)(*[int(prob[k]) for k in _KEYS])
    return arr


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def threads():
    """OpenMP threads the oracle runs on."""
    return _load().oracle_threads()


def out_size(inp, pad, k, stride, dil):
    """Output extent along one axis, or -1 when the problem is invalid."""
    return _load().oracle_out_size(int(inp), int(pad), int(k), int(stride), int(dil))


def output_hw(prob):
    return (out_size(prob["H"], prob["pad_h"], prob["R"], prob["stride_h"], prob["dil_h"]),
            out_size(prob["W"], prob["pad_w"], prob["S"], prob["stride_w"], prob["dil_w"]))


def _check(rc):
    if rc != 0:
        raise ValueError("oracle: invalid problem")


def fprop(prob, x, w, bias=None, relu=False):
    """y = conv(x, w) (+ bias) (ReLU), exact fp64 sums, shape [N,P,Q,K]."""
    P, Q = output_hw(prob)
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    y = np.empty((prob["N"], P, Q, prob["K"]), dtype=np.float64)
    dp = ctypes.c_double
    _check(_load().oracle_fprop(_dims(prob), _ptr(x, dp), _ptr(w, dp),
                                None if b is None else _ptr(b, dp), int(bool(relu)), _ptr(y, dp)))
    return y


def dgrad(prob, dy, w):
    """dx = adjoint of fprop in x, applied to dy; shape [N,H,W,C]."""
    dy, w = _f64(dy), _f64(w)
    dx = np.empty((prob["N"], prob["H"], prob["W"], prob["C"]), dtype=np.float64)
    dp = ctypes.c_double
    _check(_load().oracle_dgrad(_dims(prob), _ptr(dy, dp), _ptr(w, dp), _ptr(dx, dp)))
    return dx


def wgrad(prob, x, dy):
    """dw = adjoint of fprop in w, applied to dy; shape [K,R,S,C/G]."""
    x, dy = _f64(x), _f64(dy)
    dw = np.empty((prob["K"], prob["R"], prob["S"], prob["C"] // prob["groups"]), dtype=np.float64)
    dp = ctypes.c_double
    _check(_load().oracle_wgrad(_dims(prob), _ptr(x, dp), _ptr(dy, dp), _ptr(dw, dp)))
    return dw


def bias_grad(prob, dy):
    """db[k] = sum of dy[n,p,q,k] over n, p, q (adjoint of the bias add); shape [K]."""
    dy = _f64(dy)
    db = np.empty((prob["K"],), dtype=np.float64)
    dp = ctypes.c_double
    _check(_load().oracle_bias_grad(_dims(prob), _ptr(dy, dp), _ptr(db, dp)))
    return db


def _idx(idx):
    return np.ascontiguousarray(idx, dtype=np.int64)


def fprop_sampled(prob, x, w, idx, bias=None, relu=False):
    """fprop values at flat output indices idx (row-major [N,P,Q,K])."""
    x, w, idx = _f64(x), _f64(w), _idx(idx)
    b = None if bias is None else _f64(bias)
    out = np.empty(idx.shape[0], dtype=np.float64)
    dp = ctypes.c_double
    _check(_load().oracle_fprop_sampled(_dims(prob), _ptr(x, dp), _ptr(w, dp),
                                        None if b is None else _ptr(b, dp), int(bool(relu)),
                                        _ptr(idx, ctypes.c_int64), idx.shape[0], _ptr(out, dp)))
    return out


def dgrad_sampled(prob, dy, w, idx):
    """dgrad values at flat indices idx (row-major [N,H,W,C])."""
    dy, w, idx = _f64(dy), _f64(w), _idx(idx)
    out = np.empty(idx.shape[0], dtype=np.float64)
    dp = ctypes.c_double
    _check(_load().oracle_dgrad_sampled(_dims(prob), _ptr(dy, dp), _ptr(w, dp),
                                        _ptr(idx, ctypes.c_int64), idx.shape[0], _ptr(out, dp)))
    return out


def wgrad_sampled(prob, x, dy, idx):
    """wgrad values at flat indices idx (row-major [K,R,S,C/G])."""
    x, dy, idx = _f64(x), _f64(dy), _idx(idx)
    out = np.empty(idx.shape[0], dtype=np.float64)
    dp = ctypes.c_double
    _check(_load().oracle_wgrad_sampled(_dims(prob), _ptr(x, dp), _ptr(dy, dp),
                                        _ptr(idx, ctypes.c_int64), idx.shape[0], _ptr(out, dp)))
    return out


def linear_combination(r, alpha=1.0, beta=0.0, c=None, bias=None, relu=False):
    """alpha * r + beta * c (+ bias over the last axis) (ReLU), elementwise in
    fp64: the D = alpha*conv + beta*C epilogue of the CUTLASS notebook.  r is a
    pass's fp64 result, c an array of the same shape (or None)."""
    r = _f64(r)
    out = np.empty_like(r)
    K = r.shape[-1]
    cc = None if c is None else _f64(c)
    if cc is not None and cc.shape != r.shape:
        raise ValueError("c must have the result's shape")
    b = None if bias is None else _f64(bias)
    dp = ctypes.c_double
    _load().oracle_linear_combination(_ptr(r, dp), None if cc is None else _ptr(cc, dp), r.size, K,
                                      float(alpha), float(beta), None if b is None else _ptr(b, dp),
                                      int(bool(relu)), _ptr(out, dp))
    return out


def requant_multiplier(act_scale, w_scale, out_scale):
    """act*w/out in double precision, left to right."""
    return _load().oracle_requant_multiplier(float(act_scale), float(w_scale), float(out_scale))


def requant(acc, K, bias=None, relu=False, multiplier=1.0, idx=None):
    """int8 requantisation of exact conv sums acc (flat, output order).

    idx gives the flat output index of each acc entry (for the bias channel);
    None means acc covers the whole output in order.
    """
    acc = _f64(acc).reshape(-1)
    out = np.empty(acc.shape[0], dtype=np.int8)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.int32)
    ix = None if idx is None else _idx(idx)
    _load().oracle_requant(_ptr(acc, ctypes.c_double),
                           None if ix is None else _ptr(ix, ctypes.c_int64),
                           acc.shape[0], int(K),
                           None if b is None else _ptr(b, ctypes.c_int32),
                           int(bool(relu)), float(multiplier), _ptr(out, ctypes.c_int8))
    return out


def round_f16(v):
    """fp64 -> IEEE binary16 bit patterns (uint16), round half to even."""
    v = _f64(v)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_round_f16(_ptr(v, ctypes.c_double), v.size, _ptr(out, ctypes.c_uint16))
    return out


def round_bf16(v):
    """fp64 -> bfloat16 bit patterns (uint16), round half to even."""
    v = _f64(v)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_round_bf16(_ptr(v, ctypes.c_double), v.size, _ptr(out, ctypes.c_uint16))
    return out


def round_to(v, dtype):
    """Round fp64 values once to 'f16' or 'bf16'; returns uint16 bit patterns."""
    if dtype == "f16":
        return round_f16(v)
    if dtype == "bf16":
        return round_bf16(v)
    raise ValueError(dtype)


def bits_to_f64(bits, dtype):
    """Decode uint16 bit patterns of 'f16' / 'bf16' to float64 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


LIB_PATH = _build.LIB
__all__ = ["fprop", "dgrad", "wgrad", "fprop_sampled", "dgrad_sampled", "wgrad_sampled",
           "requant", "requant_multiplier", "round_f16", "round_bf16", "round_to",
           "bits_to_f64", "out_size", "output_hw", "threads"]
