"""Benchmark of the conv2d hot path on one MI355X.

One step = fprop (+bias+ReLU) + dgrad + wgrad of one batch of the workload
(default: 64x56x56x64 -> 64, 3x3, stride 1, pad 1, fp16, Gaussian data), all
through the C ABI, inputs resident in HBM before the timed region.  Prints one
JSON line:
  value      = FLOPs of the three passes / wall time per step (TFLOP/s),
               2*N*P*Q*K*(C/G)*R*S FLOPs per pass, over K back-to-back steps
               between two device synchronisations;
  passes     = per-pass time per launch (K back-to-back launches of the pass
               between two HIP events on the launch stream, median of 5
               trials), TFLOP/s, fraction of the dense fp16 MFMA peak (and of
               the peak at the clock the kernel ran at, from the committed
               counter summary), algorithmic GB/s, a cold-cache time (single
               launches after a 512 MiB flush) and the kernels the pass
               launches;
  roofline   = the pass that takes the most time, against its bound, with
               the measured HBM traffic of its kernels;
  cpu_baseline = the fp64 CPU oracle on a bounded sample of the same
               workload (first images of the batch), same FLOP convention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv2d TFLOP/s (fprop/dgrad/wgrad) and % of MFMA peak, 56x56x64 3x3 fp16"
# MI355X published dense peaks: fp16/bf16 MFMA 2.5 PFLOP/s (= 256 CU x 4096
# FLOP/clk x 2.4 GHz = 2516.6 TFLOP/s), int8 5.03 POP/s, HBM3E 8 TB/s.
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "i8": 5033.2}
PEAK_HBM_GBS = 8000.0
SPEC_CLOCK_GHZ = 2.4
TRIALS = 5            # timed trials per pass (median reported)
COLD_LAUNCHES = 7     # single cold-cache launches per pass (median reported)
FLUSH_BYTES = 512 << 20
BAND_TILE, WGRAD_BAND_TILE = 5, 2  # plan tile indices of the band kernels (conv2d_plan_info)
COPY_BYTES = 64 << 20  # reference copy for the HBM byte counters
# Measured HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by
# the same counters on a plain copy) lives in this summary, keyed by a hash of
# the kernel sources it was measured on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c3a_hbm_traffic.json")
KERNEL_SOURCES = ["band.hip", "wgrad_band.hip", "wgrad.hip", "igemm.hip", "api.cpp", "device_common.h", "internal.h", "direct.hip", "repack.hip", "fewchan.hip", "fewchan_wgrad.hip", "fewchan_dgrad.hip", "pointwise.hip", "pointwise_wgrad.hip", "patch.hip"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "convolution_nhwc_implicit_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, pass_name):
    """HBM bytes per launch of a pass from the committed counter summary, or
    None when it is absent, covers another workload or was taken on different
    kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    p = t.get("passes", {}).get(pass_name)
    return None if p is None else p.get("hbm_bytes")


COUNTER_FILE = os.path.join(ROOT, "profiles", "c3a_mfma_counters.json")


def measured_counters(workload, pass_name):
    """(clock GHz, MFMA-busy fraction) of the pass's main kernel under
    rocprofv3, from the committed counter summary, while the kernel sources
    are the ones it was taken on; else None.  The clock is SQ_BUSY_CYCLES per
    shader engine over the kernel's duration (the clock weighted by the time
    the engines were busy, so a lower bound), the fraction the matrix cores'
    busy cycles over all SIMD cycles counted in that clock."""
    try:
        with open(COUNTER_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    p = t.get("passes", {}).get(pass_name)
    return None if p is None else (p.get("clock_ghz"), p.get("mfma_busy_frac"))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3a_resnet3x3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile", type=int, default=0,
                    help="with --only: algorithm tile override (1-based, conv2d_plan_info order; 0 = library choice)")
    ap.add_argument("--split-k", type=int, default=0,
                    help="with --only wgrad: reduction slices override (0 = library choice)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (default: also replay captured HIP graphs)")
    ap.add_argument("--cpu-sample-images", type=int, default=0,
                    help="images of the batch the oracle runs on (0 = auto)")
    ap.add_argument("--only", choices=["fprop", "dgrad", "wgrad", "copy"], default=None,
                    help="profiling aid: run only this pass (prints its timing, no JSON line); "
                         "'copy' runs a plain 64 MiB device copy, the reference for HBM byte counters")
    return ap.parse_args()


def flops(prob, P, Q):
    return 2.0 * prob["N"] * P * Q * prob["K"] * (prob["C"] // prob["groups"]) * prob["R"] * prob["S"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(data-parallel sharding across GPUs is a design, not an implementation)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from convolution_nhwc_implicit_amd import binding as B
    from convolution_nhwc_implicit_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    name = args.workload
    wl = WL.WORKLOADS[name]
    prob, dt = wl["prob"], wl["dtype"]
    if dt == "i8" and args.only != "fprop":
        print("bench.py times the fp16/bf16 three-pass step; int8 is fprop only (use --only fprop)",
              file=sys.stderr)
        sys.exit(2)
    P, Q = B.conv2d_output_size(prob)
    x = WL.make_x(name).to(dev)
    w = WL.make_w(name).to(dev)
    b = WL.make_bias(name).to(dev) if wl["bias"] else None
    relu = wl["relu"]
    sc = wl.get("scales", (1.0, 1.0, 1.0))  # int8 requantisation scales (act, w, out)
    y = torch.empty((prob["N"], P, Q, prob["K"]), dtype=x.dtype, device=dev)
    ops = (0,) if dt == "i8" else (0, 1, 2)
    ws = {op: B.workspace_for(op, prob, dt, dev) for op in ops}
    if dt != "i8":
        dy = WL.make_dy(name, P, Q).to(dev)
        dx = torch.empty_like(x)
        dw = torch.empty_like(w)
    stream = torch.cuda.current_stream()

    def step(st=stream):
        B.conv2d_fprop(prob, dt, x, w, b, relu, sc[0], sc[1], sc[2], y, ws[0], stream=st)
        B.conv2d_dgrad(prob, dt, dy, w, dx, ws[1], stream=st)
        B.conv2d_wgrad(prob, dt, x, dy, dw, ws[2], stream=st)

    if args.only == "copy":
        src_t = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst_t = torch.empty_like(src_t)
        # one elementwise kernel that reads COPY_BYTES and writes COPY_BYTES
        for _ in range(args.warmup):
            torch.neg(src_t, out=dst_t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            torch.neg(src_t, out=dst_t)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        print(f"copy {COPY_BYTES} B: {us:.2f} us/launch, {2 * COPY_BYTES / us / 1e3:.1f} GB/s", flush=True)
        return
    if args.only:
        al = dict(tile=args.tile, split_k=args.split_k) if (args.tile or args.split_k) else None
        op = {"fprop": 0, "dgrad": 1, "wgrad": 2}[args.only]
        wso = B.workspace_for(op, prob, dt, dev, al) if al else ws.get(op)
        run = {"fprop": lambda: B.conv2d_fprop(prob, dt, x, w, b, relu, sc[0], sc[1], sc[2], y, wso, al,
                                               stream=stream),
               "dgrad": lambda: B.conv2d_dgrad(prob, dt, dy, w, dx, wso, al, stream=stream),
               "wgrad": lambda: B.conv2d_wgrad(prob, dt, x, dy, dw, wso, al, stream=stream)}[args.only]
        for _ in range(args.warmup):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        fl = flops(prob, P, Q)
        esz = 1 if dt == "i8" else 2
        nx, ny = prob["N"] * prob["H"] * prob["W"] * prob["C"], prob["N"] * P * Q * prob["K"]
        nw = prob["K"] * prob["R"] * prob["S"] * (prob["C"] // prob["groups"])
        mb = esz * (nx + ny + nw) / 1e6  # algorithmic bytes: each tensor once
        tl = (f" tile {args.tile}" if args.tile else "") + (f" split {args.split_k}" if args.split_k else "")
        print(f"{args.only}{tl} {name}: {us:.2f} us/launch, {fl / us / 1e6:.1f} T{'OP' if dt == 'i8' else 'FLOP'}/s, "
              f"{mb / us * 1e3:.1f} GB/s algorithmic ({mb:.2f} MB)", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region 1: K whole steps back to back (wall clock between two
    # device synchronisations), launched eagerly -> value.  The same step
    # replayed from a captured HIP graph (the library makes no allocation,
    # copy, memset or synchronisation call, so a step captures as its kernel
    # launches) is reported beside it.
    def wall(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    eager_ms = wall(step)
    cap = torch.cuda.Stream()  # default priority
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            step(cap)
        stream.wait_stream(cap)
        for _ in range(args.warmup):
            graph.replay()
        graph_ms = wall(graph.replay)
    ms_per_step = eager_ms

    # Timed region 2: each pass alone, K back-to-back launches between two HIP
    # events recorded on the launch stream -> per-pass time per launch (the
    # figure rocprofv3's kernel trace reports as the kernels' duration); the K
    # launches are replayed from one captured graph unless --eager.
    runs = {"fprop": lambda st: B.conv2d_fprop(prob, dt, x, w, b, relu, sc[0], sc[1], sc[2], y, ws[0], stream=st),
            "dgrad": lambda st: B.conv2d_dgrad(prob, dt, dy, w, dx, ws[1], stream=st),
            "wgrad": lambda st: B.conv2d_wgrad(prob, dt, x, dy, dw, ws[2], stream=st)}

    def events(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    # Each pass is timed in TRIALS trials of K launches; the median is the
    # figure, min and max are reported beside it.
    pass_us, eager_us, pass_trials = {}, {}, {}
    for pname, run in runs.items():
        run(stream)

        def eager_k():
            for _ in range(args.steps):
                run(stream)

        eager_us[pname] = float(np.median([events(eager_k) for _ in range(TRIALS)]))
        if graph is not None:
            g = torch.cuda.CUDAGraph()
            cap.wait_stream(stream)
            with torch.cuda.graph(g, stream=cap):
                for _ in range(args.steps):
                    run(cap)
            stream.wait_stream(cap)
            g.replay()
            trials = [events(g.replay) for _ in range(TRIALS)]
        else:
            trials = [events(eager_k) for _ in range(TRIALS)]
        pass_trials[pname] = trials
        pass_us[pname] = float(np.median(trials))

    # Cold cache: single launches, each after a 512 MiB write that evicts the
    # 256 MB MALL and the L2s, timed by events around the launch alone.
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    cold_us = {}
    for pname, run in runs.items():
        t = []
        for _ in range(COLD_LAUNCHES):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3)
        cold_us[pname] = float(np.median(t))
    del flush

    fl = flops(prob, P, Q)
    esz = 2
    elems_x = prob["N"] * prob["H"] * prob["W"] * prob["C"]
    elems_y = prob["N"] * P * Q * prob["K"]
    elems_w = prob["K"] * prob["R"] * prob["S"] * (prob["C"] // prob["groups"])
    alg_bytes = {
        "fprop": esz * (elems_x + elems_w + elems_y + (prob["K"] if b is not None else 0)),
        "dgrad": esz * (elems_y + elems_w + elems_x),
        "wgrad": esz * (elems_x + elems_y + elems_w),
    }
    plans = {n: B.conv2d_plan_info(op, prob, dt) for op, n in enumerate(("fprop", "dgrad", "wgrad"))}
    direct = plans["fprop"]["kernel"] == 2  # groups > 1
    def main_kernel(pl):
        return ("direct" if direct else "pointwise" if pl["kernel"] == 5 else "few_channel" if pl["kernel"] == 4
                else "patch" if pl["kernel"] == 6 else "band" if pl["tile"] == BAND_TILE else "implicit_gemm")

    kernels = {
        "fprop": [main_kernel(plans["fprop"])],
        "dgrad": ((["filter_relayout"] if plans["dgrad"]["workspace_bytes"] > 0 and plans["dgrad"]["kernel"] == 1
                   else []) + [main_kernel(plans["dgrad"])]),
        "wgrad": (["direct" if direct else "pointwise_wgrad" if plans["wgrad"]["kernel"] == 5
                   else "few_channel_wgrad" if plans["wgrad"]["kernel"] == 4
                   else "wgrad_band" if plans["wgrad"]["tile"] == WGRAD_BAND_TILE else "wgrad_gemm"]
                  + (["splitk_reduce"] if plans["wgrad"]["split_k"] > 1 else [])),
    }
    passes = {}
    for pname in ("fprop", "dgrad", "wgrad"):
        us = pass_us[pname]
        passes[pname] = {
            "us_per_launch": round(us, 3),
            "us_trials": {"n": TRIALS, "median": round(us, 3), "min": round(min(pass_trials[pname]), 3),
                          "max": round(max(pass_trials[pname]), 3)},
            "tflops": round(fl / (us * 1e-6) / 1e12, 2),
            "frac_mfma_peak": round(fl / (us * 1e-6) / 1e12 / PEAK_TFLOPS[dt], 4),
            "alg_gbs": round(alg_bytes[pname] / (us * 1e-6) / 1e9, 1),
            "eager_us_per_launch": round(eager_us[pname], 3),
            "cold_us_per_launch": round(cold_us[pname], 3),
            "cold_tflops": round(fl / (cold_us[pname] * 1e-6) / 1e12, 2),
            "kernels": kernels[pname],
            "plan": plans[pname],
        }
        mc = measured_counters(name, pname)
        if mc is not None and mc[0]:
            # the dense MFMA rate at the (lower-bound) clock the kernel ran at
            # under the profiler, so this fraction is an upper bound
            peak_clk = PEAK_TFLOPS[dt] * mc[0] / SPEC_CLOCK_GHZ
            passes[pname]["clock_ghz_counters"] = mc[0]
            passes[pname]["frac_mfma_peak_at_clock"] = round(fl / (us * 1e-6) / 1e12 / peak_clk, 4)
            passes[pname]["mfma_busy_frac_counters"] = mc[1]
    dom = max(passes, key=lambda k: passes[k]["us_per_launch"])
    d = passes[dom]
    # Compute-bound when the pass's arithmetic intensity exceeds the ridge point.
    ai = fl / alg_bytes[dom]
    ridge = PEAK_TFLOPS[dt] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge * 0.5:
        roof = {"bound": "mfma", "achieved": d["tflops"], "peak": PEAK_TFLOPS[dt], "unit": "TFLOP/s",
                "frac": round(d["tflops"] / PEAK_TFLOPS[dt], 4)}
    else:
        roof = {"bound": "hbm", "achieved": d["alg_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(d["alg_gbs"] / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(name, dom)
    if "frac_mfma_peak_at_clock" in d and roof["bound"] == "mfma":
        roof["clock_ghz_counters"] = d["clock_ghz_counters"]
        roof["frac_at_clock"] = d["frac_mfma_peak_at_clock"]
        roof["mfma_busy_frac_counters"] = d["mfma_busy_frac_counters"]
    roof["kernel"] = dom
    roof["kernels"] = kernels[dom]
    roof["per_launch"] = {"flop": fl, "alg_bytes": alg_bytes[dom], "avg_us": d["us_per_launch"]}

    total_fl = 3 * fl
    result = {
        "metric": METRIC,
        "value": round(total_fl / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "timing": "step: eager launches; passes: " + ("eager launches" if args.eager else
                                                      "HIP graph replay of K launches"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded Gaussian, shapes of the workload)",
        "config": {"workload": name, "N": prob["N"], "H": prob["H"], "W": prob["W"], "C": prob["C"],
                   "K": prob["K"], "R": prob["R"], "S": prob["S"], "stride": prob["stride_h"],
                   "pad": prob["pad_h"], "dilation": prob["dil_h"], "groups": prob["groups"],
                   "passes": "fprop(+bias+relu) + dgrad + wgrad", "gflop_per_pass": round(fl / 1e9, 3)},
        "passes": passes,
        "roofline": roof,
    }
    if graph is not None:
        result["graph_ms_per_step"] = round(graph_ms, 5)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(name, prob, P, Q, args.cpu_sample_images)
    print(json.dumps(result), flush=True)


def cpu_baseline(name, prob, P, Q, n_img):
    """The fp64 oracle (as it stands) on the first n_img images of the batch,
    all three passes, timed on the host's cores."""
    import numpy as np

    import oracle
    from convolution_nhwc_implicit_amd import workloads as WL

    sub = dict(prob)
    if n_img <= 0:
        n_img = prob["N"]
    n_img = min(n_img, prob["N"])
    sub["N"] = n_img
    x = WL.make_x(name)[:n_img].to(dtype=__import__("torch").float64).numpy()
    w = WL.make_w(name).to(dtype=__import__("torch").float64).numpy()
    dy = WL.make_dy(name, P, Q)[:n_img].to(dtype=__import__("torch").float64).numpy()
    bias = WL.make_bias(name).to(dtype=__import__("torch").float64).numpy() if WL.WORKLOADS[name]["bias"] else None
    t0 = time.perf_counter()
    oracle.fprop(sub, x, w, bias=bias, relu=WL.WORKLOADS[name]["relu"])
    oracle.dgrad(sub, dy, w)
    oracle.wgrad(sub, x, dy)
    secs = time.perf_counter() - t0
    fl = 3 * flops(sub, P, Q)
    return {"value": round(fl / secs / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"fprop+dgrad+wgrad on images 0..{n_img - 1} of {prob['N']} "
                      f"({fl / 1e9:.2f} GFLOP, {secs:.1f} s)",
            "seconds": round(secs, 2)}


if __name__ == "__main__":
    main()
