"""The three passes captured in a HIP graph (torch.cuda.CUDAGraph around the
C-ABI calls) and replayed: every replay, with eager launches, output fills
and synchronisations between the replays, must give bit-identical results to
the eager calls (the kernels are deterministic), and the first replay on
integer data must equal the oracle.  Covers the band kernels (stride 1,
C = K = 64), the implicit GEMM with the dgrad filter re-layout and the
generic wgrad (stride 2), each with its split-K reduce and a workspace."""
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

CASES = [
    ("band_3x3", problem(2, 64, 20, 24, 64, 3, 3, pad=(1, 1)), "f16"),
    ("strided_3x3", problem(4, 64, 15, 17, 128, 3, 3, pad=(1, 1), stride=(2, 2)), "bf16"),
]


@pytest.mark.parametrize("cid,prob,dtype", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(cid, prob, dtype):
    rng = np.random.Generator(np.random.PCG64(zlib.crc32(cid.encode())))
    P, Q = oracle.output_hw(prob)
    N, H, W, C, K, R, S = (prob[k] for k in ("N", "H", "W", "C", "K", "R", "S"))
    xh = WL.draw((N, H, W, C), dtype, "int", rng)
    wh = WL.draw((K, R, S, C), dtype, "int", rng)
    bh = WL.draw((K,), dtype, "int", rng)
    dyh = WL.draw((N, P, Q, K), dtype, "int", rng)
    x, w, b, dy = (t.to(DEV) for t in (xh, wh, bh, dyh))
    ws = [B.workspace_for(op, prob, dtype, DEV) for op in range(3)]

    def outputs():
        return (torch.empty((N, P, Q, K), dtype=x.dtype, device=DEV), torch.empty_like(x), torch.empty_like(w))

    def passes(out, st):
        y, dx, dw = out
        B.conv2d_fprop(prob, dtype, x, w, b, 1, 1.0, 1.0, 1.0, y, ws[0], stream=st)
        B.conv2d_dgrad(prob, dtype, dy, w, dx, ws[1], stream=st)
        B.conv2d_wgrad(prob, dtype, x, dy, dw, ws[2], stream=st)

    main = torch.cuda.current_stream()
    ref = outputs()
    passes(ref, main)
    torch.cuda.synchronize()

    gout = outputs()
    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        passes(gout, cap)
    main.wait_stream(cap)
    torch.cuda.synchronize()

    names = ("y", "dx", "dw")
    for rep in range(4):
        for t in gout:
            t.fill_(float("nan"))
        side = outputs()
        passes(side, main)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, got, want in zip(names, gout, ref):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{cid} replay {rep}: {n} differs"
        for n, got, want in zip(names, side, ref):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{cid} eager {rep}: {n} differs"
        if rep == 0:
            check(f64(gout[0]), oracle.fprop(prob, f64(xh), f64(wh), bias=f64(bh), relu=True), dtype, "exact",
                  f"{cid} y")
            check(f64(gout[1]), oracle.dgrad(prob, f64(dyh), f64(wh)), dtype, "exact", f"{cid} dx")
            check(f64(gout[2]), oracle.wgrad(prob, f64(xh), f64(dyh)), dtype, "exact", f"{cid} dw")
