"""conv2d_wgrad_noalloc (the wgrad entry point whose partials live in the
library's static device scratch) against conv2d_wgrad, through the C ABI.

Same kernels and plan, so the results must be identical bit for bit; on
integer-valued data both must also equal the oracle rounded once.  Two calls
in a row, the second on a smaller problem (the buffer keeps the first call's
contents, which the second must not depend on), then a problem whose plan
needs more than the static buffer, which must be refused with nothing
written."""
import numpy as np
import pytest
import torch

import oracle
from convolution_nhwc_implicit_amd import binding as B
from convolution_nhwc_implicit_amd import workloads as WL
from convolution_nhwc_implicit_amd.workloads import problem

from parity import DEV, check, f64, gpu, run_wgrad

pytestmark = pytest.mark.gpu


def noalloc(prob, dtype, x, dy, algo=None):
    dw = torch.full((prob["K"], prob["R"], prob["S"], prob["C"] // prob["groups"]), float("nan"),
                    dtype=x.dtype, device=DEV)
    B.conv2d_wgrad_noalloc(prob, dtype, gpu(x), gpu(dy), dw, algo)
    torch.cuda.synchronize()
    return dw


CALLS = [
    # the wgrad band kernel, 16 images (85 band slices of partials, one filter row per workgroup)
    ("band", problem(16, 64, 56, 56, 64, 3, 3, pad=(1, 1)), "f16", "int", None),
    # a smaller problem on the generic 64 x 64 wgrad kernel with 7 slices
    ("generic", problem(2, 32, 13, 11, 48, 3, 3, pad=(1, 1), stride=(2, 1)), "bf16", "int", dict(split_k=7)),
    # grouped, the direct kernel with its own slices, Gaussian data
    ("direct", problem(2, 12, 9, 10, 8, 3, 3, pad=(1, 1), groups=2), "f16", "gauss", None),
]


def test_noalloc_matches_wgrad_on_consecutive_calls():
    for i, (cid, prob, dtype, dist, algo) in enumerate(CALLS):
        print(f"call {i}: {cid} {prob} algo {algo}", flush=True)
        P, Q = oracle.output_hw(prob)
        x, _, _, dy = WL.random_case(prob, dtype, dist, 9100 + i, P, Q, bias=False)
        need = B.conv2d_workspace_size(B.CONV2D_OP_WGRAD, prob, B.NAME_CODE[dtype], algo)
        assert need <= B.CONV2D_NOALLOC_SCRATCH_BYTES
        got = noalloc(prob, dtype, x, dy, algo)
        ref = run_wgrad(prob, dtype, x, dy, algo=algo)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{cid}: differs from conv2d_wgrad"
        mode = "exact" if dist == "int" else "tol"
        check(f64(got), oracle.wgrad(prob, f64(x), f64(dy)), dtype, mode, cid)
        # the same call again gives the same bits
        again = noalloc(prob, dtype, x, dy, algo)
        assert torch.equal(again.view(torch.int16), got.view(torch.int16)), f"{cid}: repeat differs"


def test_noalloc_refuses_past_its_scratch():
    prob = problem(2, 64, 12, 12, 64, 3, 3, pad=(1, 1))
    algo = dict(tile=1, split_k=4096)  # 4096 fp32 partials of 36864 outputs: far past the buffer
    assert B.conv2d_workspace_size(B.CONV2D_OP_WGRAD, prob, B.CONV2D_DTYPE_F16, algo) > B.CONV2D_NOALLOC_SCRATCH_BYTES
    P, Q = oracle.output_hw(prob)
    x, _, _, dy = WL.random_case(prob, "f16", "int", 9200, P, Q, bias=False)
    dw = torch.full((64, 3, 3, 64), 5.0, dtype=torch.float16, device=DEV)
    with pytest.raises(B.Conv2dError) as e:
        B.conv2d_wgrad_noalloc(prob, "f16", gpu(x), gpu(dy), dw, algo)
    assert e.value.status == B.CONV2D_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(dw == 5.0)
