"""Host-side tests of the C ABI: no GPU, no kernel launches.

The library must load on a machine without a GPU, export every function the
public header declares, compute output sizes the way the oracle does (two
independent implementations of the same formula), and reject bad arguments
before anything could be enqueued.
"""
import ctypes
import os
import re

import pytest

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd.workloads import WORKLOADS, problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(\w+)\s*\(", text, flags=re.M):
            if m.group(1) not in ("defined",):
                names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_header_functions_exported(lib):
    names = declared_functions()
    assert {"conv2d_fprop", "conv2d_dgrad", "conv2d_wgrad", "conv2d_output_size",
            "conv2d_workspace_size", "conv2d_plan_info", "conv2d_status_string"} <= names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_status_strings(lib):
    for code in range(0, 6):
        s = B.conv2d_status_string(code)
        assert isinstance(s, str) and s
    assert B.conv2d_status_string(0) == "ok"


def test_output_size_agrees_with_oracle():
    n = 0
    for inp in (1, 2, 5, 8, 13, 28, 57):
        for pad in (0, 1, 2, 3):
            for k in (1, 2, 3, 5):
                for stride in (1, 2, 3):
                    for dil in (1, 2, 3):
                        prob = problem(1, 8, inp, inp + 1, 8, k, k, pad=(pad, pad),
                                       stride=(stride, stride), dil=(dil, dil))
                        exp_h = oracle.out_size(inp, pad, k, stride, dil)
                        exp_w = oracle.out_size(inp + 1, pad, k, stride, dil)
                        if exp_h < 1 or exp_w < 1:
                            with pytest.raises(B.Conv2dError) as e:
                                B.conv2d_output_size(prob)
                            assert e.value.status == B.CONV2D_ERR_INVALID_ARGUMENT
                        else:
                            assert B.conv2d_output_size(prob) == (exp_h, exp_w)
                            n += 1
    assert n > 500


def test_workload_output_sizes():
    exp = {"c1_tiny": (8, 8), "c2_strided": (14, 14), "c3a_resnet3x3": (56, 56),
           "c3b_resnet1x1": (56, 56), "c4_awkward": (27, 27), "c4g_grouped": (27, 27),
           "c5_int8": (56, 56), "n1_stem": (112, 112),
           "d1_depthwise": (56, 56)}
    for name, wl in WORKLOADS.items():
        assert B.conv2d_output_size(wl["prob"]) == exp[name]
        assert oracle.output_hw(wl["prob"]) == exp[name]


@pytest.mark.parametrize("bad", [
    dict(N=0), dict(C=0), dict(K=-1), dict(R=0), dict(pad_h=-1), dict(stride_w=0),
    dict(dil_h=0), dict(groups=0), dict(groups=3), dict(H=1, pad_h=0),
])
def test_invalid_problems(bad):
    prob = dict(problem(2, 8, 8, 8, 16, 3, 3, pad=(1, 1)), **bad)
    for op in (0, 1, 2):
        with pytest.raises(B.Conv2dError) as e:
            B.conv2d_workspace_size(op, prob, "f16")
        assert e.value.status == B.CONV2D_ERR_INVALID_ARGUMENT


def test_padded_channel_plans():
    """C or K not a multiple of 8 (16 for int8) runs on zero-padded copies
    kept in the workspace after the padded problem's own workspace."""
    N, H, W = 2, 8, 8
    p = problem(N, 12, H, W, 16, 3, 3, pad=(1, 1))  # C % 8 != 0
    q = problem(N, 16, H, W, 16, 3, 3, pad=(1, 1))  # the same problem padded
    for op in (0, 1, 2):
        info, inner = B.conv2d_plan_info(op, p, "f16"), B.conv2d_plan_info(op, q, "f16")
        assert info["kernel"] == inner["kernel"] == 1 and info["tile"] == inner["tile"]
        filt = 16 * 3 * 3 * 16 * 2
        act = N * H * W * 16 * 2  # x (fprop, wgrad) or dx (dgrad), padded to 16 channels
        up = lambda v: (v + 255) // 256 * 256
        assert info["workspace_bytes"] == up(inner["workspace_bytes"]) + up(filt) + up(act)
    k = problem(N, 16, H, W, 13, 3, 3, pad=(1, 1))  # K % 8 != 0: y/dy copies (and bias for fprop)
    assert B.conv2d_plan_info(0, k, "f16")["workspace_bytes"] > 0
    assert B.conv2d_plan_info(0, problem(N, 3, H, W, 16, 3, 3), "i8")["kernel"] == 1
    # grouped problems keep the direct kernels for any channel count
    assert B.conv2d_plan_info(0, problem(N, 6, H, W, 9, 3, 3, groups=3), "f16")["workspace_bytes"] == 0


def test_unsupported_cases():
    p = problem(2, 16, 8, 8, 16, 3, 3, pad=(1, 1))  # int8 needs C % 16, fprop only
    assert B.conv2d_plan_info(B.CONV2D_OP_FPROP, p, "i8")["kernel"] == 1
    for op in (B.CONV2D_OP_DGRAD, B.CONV2D_OP_WGRAD):
        with pytest.raises(B.Conv2dError) as e:
            B.conv2d_plan_info(op, p, "i8")
        assert e.value.status == B.CONV2D_ERR_UNSUPPORTED
    with pytest.raises(B.Conv2dError) as e:
        B.conv2d_plan_info(B.CONV2D_OP_FPROP, p, 7)
    assert e.value.status == B.CONV2D_ERR_UNSUPPORTED
    with pytest.raises(B.Conv2dError) as e:  # tile index beyond the table
        B.conv2d_plan_info(B.CONV2D_OP_FPROP, p, "f16", algo=dict(tile=99))
    assert e.value.status == B.CONV2D_ERR_UNSUPPORTED


def test_plan_rules():
    g = problem(2, 12, 9, 9, 12, 3, 3, pad=(1, 1), groups=3)  # grouped -> direct, any channel count
    for op in (0, 1, 2):
        assert B.conv2d_plan_info(op, g, "bf16")["kernel"] == 2
    s = problem(2, 16, 9, 9, 16, 3, 3, pad=(1, 1), stride=(2, 3))
    info = B.conv2d_plan_info(B.CONV2D_OP_DGRAD, s, "f16")
    assert info["kernel"] == 1 and info["phases"] == 6
    assert info["workspace_bytes"] == 0  # the implicit GEMM reads the filter as it is
    w = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, s, "f16", algo=dict(split_k=5))
    assert w["split_k"] == 5 and w["workspace_bytes"] >= 5 * 16 * 3 * 3 * 16 * 4
    assert B.conv2d_plan_info(B.CONV2D_OP_WGRAD, s, "f16", algo=dict(split_k=1))["workspace_bytes"] == 0
    # the plan is a pure function of its arguments
    assert B.conv2d_plan_info(2, s, "f16") == B.conv2d_plan_info(2, s, "f16")
    for t in range(1, B.conv2d_plan_info(0, s, "f16")["num_tiles"] + 1):
        assert B.conv2d_plan_info(0, s, "f16", algo=dict(tile=t))["tile"] == t - 1


def test_pointwise_wgrad_plan():
    """1x1 stride-1 wgrad with K and C in {64, 128, 256}, K*C <= 16384: the
    pointwise wgrad kernel (kernel 5, in the band kernel's tile 2), one fp32
    partial of K*C (+ K with the bias gradient) per pixel slice."""
    prob = problem(64, 64, 56, 56, 256, 1, 1)
    info = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")
    assert info["kernel"] == 5 and info["tile"] == 2 and info["num_tiles"] == 3
    assert info["split_k"] == 256
    assert info["workspace_bytes"] == 256 * 256 * 64 * 4  # slices are whole 256-byte multiples here
    forced = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "bf16", algo=dict(split_k=7))
    assert forced["kernel"] == 5 and forced["split_k"] == 7
    class FakeDb:  # only its address is taken; nothing is enqueued
        def data_ptr(self):
            return 0x10000

    with_db = B.conv2d_workspace_size_ex(B.CONV2D_OP_WGRAD, prob, "f16", epi=dict(db=FakeDb()))
    assert with_db == 256 * (256 * 64 + 256) * 4  # the bias gradient rides in the slices
    small = problem(2, 64, 5, 5, 64, 1, 1)  # 50 pixels: one slice
    assert B.conv2d_plan_info(B.CONV2D_OP_WGRAD, small, "f16")["split_k"] == 1
    # the generic tiles stay selectable
    assert B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16", algo=dict(tile=1))["kernel"] == 1
    for other in (problem(2, 64, 8, 8, 512, 1, 1), problem(2, 32, 8, 8, 64, 1, 1),
                  problem(2, 64, 8, 8, 256, 1, 1, stride=(2, 2)), problem(2, 64, 8, 8, 64, 1, 1, pad=(1, 1)),
                  problem(2, 64, 8, 8, 64, 1, 1, groups=2), problem(2, 192, 8, 8, 64, 1, 1)):
        assert B.conv2d_plan_info(B.CONV2D_OP_WGRAD, other, "f16")["kernel"] != 5, other
    with pytest.raises(B.Conv2dError):  # int8 backward passes are not offered
        B.conv2d_plan_info(B.CONV2D_OP_WGRAD, problem(2, 64, 8, 8, 64, 1, 1), "i8")


def _raw_call(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_errors_return_before_enqueue(lib):
    """Error paths return their code before any HIP call; the fake device
    addresses below are never dereferenced."""
    prob = B.make_problem(problem(2, 8, 8, 8, 16, 3, 3, pad=(1, 1)))
    bad = B.make_problem(problem(2, 8, 8, 8, 16, 3, 3, pad=(1, 1), groups=3))
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    pr = ctypes.byref(prob)
    # invalid problem
    assert lib.conv2d_fprop(ctypes.byref(bad), 0, fake, fake, None, 0, 1.0, 1.0, 1.0, fake, None, 0,
                            None, None) == B.CONV2D_ERR_INVALID_ARGUMENT
    # null required pointer
    assert lib.conv2d_fprop(pr, 0, None, fake, None, 0, 1.0, 1.0, 1.0, fake, None, 0, None,
                            None) == B.CONV2D_ERR_INVALID_ARGUMENT
    # relu must be 0/1
    assert lib.conv2d_fprop(pr, 0, fake, fake, None, 3, 1.0, 1.0, 1.0, fake, None, 0, None,
                            None) == B.CONV2D_ERR_INVALID_ARGUMENT
    # misaligned tensor
    assert lib.conv2d_fprop(pr, 0, odd, fake, None, 0, 1.0, 1.0, 1.0, fake, None, 0, None,
                            None) == B.CONV2D_ERR_UNSUPPORTED
    # int8 scales must be finite and positive
    p16 = B.make_problem(problem(2, 16, 8, 8, 16, 3, 3, pad=(1, 1)))
    assert lib.conv2d_fprop(ctypes.byref(p16), 2, fake, fake, None, 0, 0.0, 1.0, 1.0, fake, None, 0,
                            None, None) == B.CONV2D_ERR_INVALID_ARGUMENT
    # workspace too small (wgrad split four ways needs its fp32 partials)
    assert lib.conv2d_wgrad(pr, 0, fake, fake, fake, None, 0,
                            ctypes.byref(B.Conv2dAlgo(0, 4)), None) == B.CONV2D_ERR_WORKSPACE_TOO_SMALL
    # int8 backward passes are not offered
    assert lib.conv2d_dgrad(ctypes.byref(p16), 2, fake, fake, fake, fake, 1 << 20, None,
                            None) == B.CONV2D_ERR_UNSUPPORTED


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(2, 8, 8, 8, dtype=torch.float16)
    w = torch.zeros(16, 3, 3, 8, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        B.fprop(x, w, padding=1)


def test_epilogue_checks(lib):
    """The linear-combination entry points check their epilogue before any
    device work (the fake addresses below are never dereferenced)."""
    prob = B.make_problem(problem(2, 8, 8, 8, 16, 3, 3, pad=(1, 1)))
    p16 = B.make_problem(problem(2, 16, 8, 8, 16, 3, 3, pad=(1, 1)))
    pr = ctypes.byref(prob)
    fake = ctypes.c_void_p(0x10000)

    def epi(alpha=1.0, beta=0.0, c=None, f32=0):
        return ctypes.byref(B.Conv2dEpilogue(alpha, beta, c, f32))

    inv, uns = B.CONV2D_ERR_INVALID_ARGUMENT, B.CONV2D_ERR_UNSUPPORTED
    assert lib.conv2d_fprop_ex(pr, 0, fake, fake, None, 0, epi(alpha=float("nan")), fake, None, 0,
                               None, None) == inv
    assert lib.conv2d_fprop_ex(pr, 0, fake, fake, None, 0, epi(beta=float("inf"), c=0x10000), fake,
                               None, 0, None, None) == inv
    assert lib.conv2d_dgrad_ex(pr, 0, fake, fake, epi(beta=1.0), fake, fake, 1 << 20, None,
                               None) == inv  # beta != 0 needs C
    assert lib.conv2d_dgrad_ex(pr, 0, fake, fake, epi(beta=1.0, c=0x10008), fake, fake, 1 << 20, None,
                               None) == uns  # C must be 16-byte aligned
    assert lib.conv2d_fprop_ex(pr, 0, fake, fake, None, 0, epi(f32=1), fake, None, 0, None,
                               None) == inv  # fp32 output is for wgrad only
    assert lib.conv2d_fprop_ex(ctypes.byref(p16), 2, fake, fake, None, 0, epi(alpha=2.0), fake, None, 0,
                               None, None) == uns  # no int8 epilogue
    s = problem(2, 16, 9, 9, 16, 3, 3, pad=(1, 1))
    assert B.conv2d_workspace_size(2, s, "f16", algo=dict(split_k=1)) == 0
    # wgrad applies the epilogue in its reduction: partials even for one slice
    n = B.conv2d_workspace_size_ex(2, s, "f16", algo=dict(split_k=1), epi=dict(out_f32=True))
    assert n >= 16 * 3 * 3 * 16 * 4
    assert B.conv2d_workspace_size_ex(2, s, "f16", epi=None) == B.conv2d_workspace_size(2, s, "f16")
    # the bias gradient beside wgrad: its partials follow the pass's workspace
    fake_db = type("T", (), {"data_ptr": lambda self: 0x20000})()
    n0 = B.conv2d_workspace_size_ex(2, s, "f16", epi=dict(alpha=2.0))
    n1 = B.conv2d_workspace_size_ex(2, s, "f16", epi=dict(alpha=2.0, db=fake_db))
    assert n1 >= n0 + 16 * 4 and n1 % 256 == 0
    ep = B.Conv2dEpilogue(1.0, 0.0, None, 0, 0x20000)
    assert lib.conv2d_fprop_ex(pr, 0, fake, fake, None, 0, ctypes.byref(ep), fake, None, 0, None,
                               None) == inv  # db is for wgrad only
    ep = B.Conv2dEpilogue(1.0, 0.0, None, 0, 0x20008)
    assert lib.conv2d_wgrad_ex(pr, 0, fake, fake, ctypes.byref(ep), fake, fake, 1 << 20, None,
                               None) == uns  # db must be 16-byte aligned
    # the band-shaped dgrad needs no workspace plain, nor on the implicit GEMM
    # that runs it with an epilogue (both read the filter as it is)
    band = problem(2, 64, 9, 9, 64, 3, 3, pad=(1, 1))
    assert B.conv2d_workspace_size(1, band, "f16") == 0
    assert B.conv2d_workspace_size_ex(1, band, "f16", epi=dict(alpha=2.0)) == 0


def test_bias_grad_checks(lib):
    """The bias gradient validates and plans before any device work (the fake
    addresses below are never dereferenced)."""
    prob = problem(4, 8, 10, 10, 24, 3, 3, pad=(1, 1))
    pr = ctypes.byref(B.make_problem(prob))
    fake = ctypes.c_void_p(0x10000)
    n = B.conv2d_bias_grad_workspace_size(prob, "f16")
    # one fp32 partial of K (rounded up to 4) per row slice; 400 rows make 6 slices
    assert n >= 6 * 24 * 4 and n % 256 == 0
    inv, uns = B.CONV2D_ERR_INVALID_ARGUMENT, B.CONV2D_ERR_UNSUPPORTED
    assert lib.conv2d_bias_grad(pr, 0, None, fake, 0, fake, n, None) == inv
    assert lib.conv2d_bias_grad(pr, 0, fake, fake, 2, fake, n, None) == inv  # out_f32 is 0 or 1
    assert lib.conv2d_bias_grad(pr, 2, fake, fake, 0, fake, n, None) == uns  # no int8
    assert lib.conv2d_bias_grad(pr, 0, ctypes.c_void_p(0x10008), fake, 0, fake, n, None) == uns
    assert lib.conv2d_bias_grad(pr, 0, fake, fake, 0, fake, n - 256, None) == B.CONV2D_ERR_WORKSPACE_TOO_SMALL
    assert lib.conv2d_bias_grad(pr, 0, fake, fake, 0, None, n, None) == inv
    bad = B.make_problem(problem(4, 8, 10, 10, 24, 3, 3, pad=(1, 1), groups=3))
    bad.c = 7  # C % groups != 0
    assert lib.conv2d_bias_grad(ctypes.byref(bad), 0, fake, fake, 0, fake, n, None) == inv


def test_bench_names_the_band_kernels():
    """bench.py names the kernels of a pass from the plan's tile index; its
    constants must be the band kernels' indices in the library's plans."""
    import bench
    from convolution_nhwc_implicit_amd import workloads as WL

    c3a = WL.WORKLOADS["c3a_resnet3x3"]["prob"]
    assert B.conv2d_plan_info(0, c3a, "f16")["tile"] == bench.BAND_TILE
    assert B.conv2d_plan_info(1, c3a, "f16")["tile"] == bench.BAND_TILE
    assert B.conv2d_plan_info(2, c3a, "f16")["tile"] == bench.WGRAD_BAND_TILE


def test_winograd_tile_offered_only_where_it_applies():
    """The Winograd tile (plan kernel 3) exists for stride-1, dilation-1 3x3
    problems whose source has 64 channels and whose output channels are a
    multiple of 16 (fprop: C = 64, K % 16; dgrad: K = 64, C % 16, pad <= 2),
    fp16 only (bf16 would miss rms_scaled <= 1e-3), without the
    linear-combination epilogue; it is never the default; fprop needs no
    workspace."""
    base = problem(2, 64, 10, 12, 64, 3, 3, pad=(1, 1))
    info = B.conv2d_plan_info(0, base, "f16")
    # fprop table: 5 implicit-GEMM tiles, the band kernel, Winograd, the patch kernel
    assert info["num_tiles"] == 8 and info["tile"] == 5 and info["kernel"] == 1
    w = B.conv2d_plan_info(0, base, "f16", algo=dict(tile=7))
    assert w["kernel"] == 3 and w["tile"] == 6 and w["workspace_bytes"] == 0
    assert B.conv2d_plan_info(0, base, "f16", algo=dict(tile=8))["kernel"] == 6
    # bf16: the band kernel is still the default, and no Winograd tile
    # (fprop: the patch kernel follows the band kernel)
    for op in (0, 1):
        info = B.conv2d_plan_info(op, base, "bf16")
        assert info["num_tiles"] == 7 and info["tile"] == 5 and info["kernel"] == 1
        assert B.conv2d_plan_info(op, base, "bf16", algo=dict(tile=7))["kernel"] == 6
    # dgrad: the forward Winograd kernel on dy with the flipped, transposed
    # filter, whose transform goes to the workspace (16 x C x K elements)
    # (the patch kernel's tile follows it: stride 1 divides any dilation)
    d = B.conv2d_plan_info(1, base, "f16")
    assert d["num_tiles"] == 8 and d["tile"] == 5
    dw = B.conv2d_plan_info(1, base, "f16", algo=dict(tile=7))
    assert dw["kernel"] == 3 and dw["workspace_bytes"] == 16 * 64 * 64 * 2
    assert B.conv2d_plan_info(1, base, "f16", algo=dict(tile=8))["kernel"] == 6

    def has_wino(prob):
        n = B.conv2d_plan_info(1, prob, "f16")["num_tiles"]
        return any(B.conv2d_plan_info(1, prob, "f16", algo=dict(tile=t))["kernel"] == 3 for t in range(1, n + 1))
    assert not has_wino(problem(2, 64, 10, 12, 64, 3, 3, pad=(3, 3)))
    assert has_wino(problem(2, 48, 10, 12, 64, 3, 3, pad=(1, 1)))
    assert not has_wino(problem(2, 40, 10, 12, 64, 3, 3, pad=(1, 1)))
    others = [(base, "i8"), (base, "bf16"),
              (problem(2, 32, 10, 12, 64, 3, 3, pad=(1, 1)), "f16"),
              (problem(2, 64, 10, 12, 40, 3, 3, pad=(1, 1)), "f16"),
              (problem(2, 64, 10, 12, 64, 3, 3, pad=(1, 1), stride=(2, 2)), "f16"),
              (problem(2, 64, 10, 12, 64, 3, 3, pad=(2, 2), dil=(2, 2)), "bf16"),
              (problem(2, 64, 10, 12, 64, 5, 5, pad=(2, 2)), "f16")]
    for prob, dt in others:
        n = B.conv2d_plan_info(0, prob, dt)["num_tiles"]
        assert n <= 7, (prob, dt)
        assert all(B.conv2d_plan_info(0, prob, dt, algo=dict(tile=t))["kernel"] != 3 for t in range(1, n + 1))
        with pytest.raises(B.Conv2dError) as e:
            B.conv2d_plan_info(0, prob, dt, algo=dict(tile=n + 1))
        assert e.value.status == B.CONV2D_ERR_UNSUPPORTED
    with pytest.raises(B.Conv2dError) as e:
        B.conv2d_workspace_size_ex(0, base, "f16", algo=dict(tile=7), epi=dict(alpha=2.0, beta=0.0))
    assert e.value.status == B.CONV2D_ERR_UNSUPPORTED


def test_bench_counters_only_for_their_workload():
    """The committed counter summaries (HBM bytes, clock and MFMA-busy
    fraction) were taken on one workload; bench.py reports them for that
    workload only, and only while the kernel sources hash to the ones they
    were taken on."""
    import json
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    wl = t["workload"]
    other = "c4_awkward" if wl != "c4_awkward" else "c3a_resnet3x3"
    for p in ("fprop", "dgrad", "wgrad"):
        assert bench.measured_traffic(other, p) is None
        assert bench.measured_counters(other, p) is None
        if t["source_hash"] == bench.kernel_source_hash():
            assert bench.measured_traffic(wl, p) == t["passes"][p]["hbm_bytes"]
        else:
            assert bench.measured_traffic(wl, p) is None


@pytest.mark.parametrize("prob,split", [
    (problem(8, 64, 18, 16, 64, 3, 3, pad=(1, 1)), 8 * 9),    # 2-row bands: column halves, 9 per image
    (problem(13, 64, 56, 20, 64, 3, 3, pad=(1, 1)), 85),      # filter rows: 85 bands
    (problem(64, 64, 56, 56, 64, 3, 3, pad=(1, 1)), 85),
    (problem(76, 64, 9, 24, 64, 3, 3, pad=(1, 1)), 85),       # bands of 8-9 rows across 9-row images
    (problem(150, 64, 6, 16, 64, 3, 3, pad=(1, 1)), 85),      # bands of 10-11 rows over 2-3 images
    (problem(128, 64, 56, 56, 64, 3, 3, pad=(1, 1)), 128),    # twice the benchmark's work per CU: halves
], ids=["halves", "rows_small", "rows_c3a", "rows_short_img", "rows_three_imgs", "halves_n128"])
def test_wgrad_band_split(prob, split):
    """The band kernel's partial slices, one per band: the split (column
    halves or filter rows) with the lower estimated time."""
    info = B.conv2d_plan_info(B.CONV2D_OP_WGRAD, prob, "f16")
    assert info["tile"] == 2 and info["split_k"] == split, info
