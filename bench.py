"""Benchmark: depthwise conv2d forward + input gradient on one MI355X.

A step is one forward and one input gradient of the 512x512x256 3x3 NHWC
workload (fp32 activations and weights), inputs resident in HBM.  The JSON
line reports whole-step effective HBM bandwidth (algorithmic bytes: x+y+W+b
for the forward, dy+dx+W for the input gradient), the roofline of the
dominant kernel timed with HIP events on its own stream, the CPU oracle timed
on a bounded sample, and a per-workload table (forward and input gradient,
both layouts, back-to-back "warm" and cache-flushed "cold" kernel times).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-table] [--no-cpu]
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
HEADLINE = "large_512x512x256_3x3"
# the sources that decide the headline kernel's code and plan: a change to any
# of them makes the recorded traffic counts stale
KERNEL_SRCS = [os.path.join(ROOT, "depthwise_convolution_amd", "csrc", f)
               for f in ("dwconv_internal.h", "dwconv_device.h", "dwconv_tiled_nhwc.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_large_512x512x256_3x3_nhwc.json")


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest():
    h = hashlib.sha256()
    for src in KERNEL_SRCS:
        with open(src, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(op):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE,
    WRITE_SIZE, scaled by a copy-kernel calibration), or None when the counts
    are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    rec = t.get("ops", {}).get(op)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def to_dev(torch, a):
    return torch.from_numpy(a).to("cuda")


def make_problem(torch, wl, layout, seed=0):
    from depthwise_convolution_amd import workloads
    inp = workloads.make_inputs(wl, layout, seed=seed)
    t = {k: (None if v is None else to_dev(torch, v)) for k, v in inp.items()}
    shape_x = tuple(inp["x"].shape)
    t["y"] = torch.empty(tuple(inp["dy"].shape), dtype=torch.float32, device="cuda")
    t["dx"] = torch.empty(shape_x, dtype=torch.float32, device="cuda")
    import depthwise_convolution_amd as dw
    if wl.general:
        nws = dw.dwconv2d_weight_grad_workspace_size_ex(wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                                        wl.stride, wl.dilation, wl.pads,
                                                        wl.mult, layout)
    else:
        nws = dw.dwconv2d_weight_grad_workspace_size(wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                                     wl.stride, wl.dilation, layout)
    t["ws"] = torch.empty(max(4, (nws + 15) // 16 * 4), dtype=torch.float32, device="cuda")
    t["dW"] = torch.empty((wl.Co, wl.kH, wl.kW), dtype=torch.float32, device="cuda")
    t["db"] = torch.empty((wl.Co,), dtype=torch.float32, device="cuda")
    # inference BatchNorm of the output channels (gamma, beta, mean, var) and
    # float32 weights / bias for the SGD step (updated in place by each call)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    t["bn"] = tuple((torch.rand(wl.Co, generator=g) * s + o).to("cuda")
                    for s, o in ((1.5, 0.5), (2.0, -1.0), (1.0, -0.5), (2.8, 0.2)))
    t["w_sgd"] = torch.from_numpy(inp["w"].astype("float32")).to("cuda")
    t["b_sgd"] = torch.zeros((wl.Co,), dtype=torch.float32, device="cuda")
    return t


def launch_fwd(dw, wl, t, layout, stream):
    if wl.general:
        dw.dwconv2d_launch_ex(dw.OP_FWD, t["x"], t["w"], t["b"], t["y"], wl.H, wl.W, wl.stride,
                              wl.dilation, wl.pads, wl.mult, layout, dw.STRATEGY_AUTO, stream)
    else:
        dw.dwconv2d_fwd(t["x"], t["w"], t["b"], t["y"], wl.stride, wl.dilation, layout, stream)


def launch_ig(dw, wl, t, layout, stream):
    if wl.general:
        dw.dwconv2d_launch_ex(dw.OP_INPUT_GRAD, t["dy"], t["w"], None, t["dx"], wl.H, wl.W,
                              wl.stride, wl.dilation, wl.pads, wl.mult, layout,
                              dw.STRATEGY_AUTO, stream)
    else:
        dw.dwconv2d_input_grad(t["dy"], t["w"], t["dx"], wl.stride, wl.dilation, layout, stream)


def launch_wgrad(dw, wl, t, layout, stream):
    if wl.general:
        dw.dwconv2d_weight_grad_ex(t["x"], t["dy"], t["dW"], t["db"], t["ws"], wl.stride,
                                   wl.dilation, wl.pads, wl.mult, layout, dw.STRATEGY_AUTO,
                                   stream)
    else:
        dw.dwconv2d_weight_grad(t["x"], t["dy"], t["dW"], t["db"], t["ws"], wl.stride,
                                wl.dilation, layout, dw.STRATEGY_AUTO, stream)


def launch_fwd_bn_act(dw, wl, t, layout, stream):
    """Forward with the fused BatchNorm + ReLU6 epilogue (MobileNetV2 block)."""
    dw.dwconv2d_fwd_bn_act_ex(t["x"], t["w"], t["b"], t["y"], t["bn"], 1e-3, dw.ACT_RELU6,
                              wl.stride, wl.dilation, wl.pads, wl.mult, layout,
                              dw.STRATEGY_AUTO, stream)


def launch_wgrad_sgd(dw, wl, t, layout, stream):
    """Weight + bias gradient with the fused SGD step (w, b updated in place)."""
    dw.dwconv2d_weight_grad_sgd_ex(t["x"], t["dy"], t["w_sgd"], t["b_sgd"], 1e-4, t["ws"],
                                   None, None, wl.stride, wl.dilation, wl.pads, wl.mult, layout,
                                   dw.STRATEGY_AUTO, stream)


def fwd_bn_act_bytes(wl):
    """x + y + W + b + the four BatchNorm arrays."""
    return wl.fwd_bytes() + 16 * wl.Co


def wgrad_sgd_bytes(wl):
    """x + dy + W and b read and written (the gradients are not written)."""
    return (4 * wl.N * wl.H * wl.W * wl.C + 4 * wl.N * wl.Ho * wl.Wo * wl.Co
            + 8 * wl.Co * wl.kH * wl.kW + 8 * wl.Co)


def wgrad_bytes(wl):
    """Algorithmic bytes of the weight + bias gradient: x + dy + dW + db."""
    return wl.wgrad_bytes()


def describe(dw, wl, op, layout):
    """Kernel name of an op of a workload under the AUTO strategy."""
    wt = 0 if op == dw.OP_WEIGHT_GRAD else int(wl.fp16_weights)
    if wl.general:
        return dw.dwconv2d_describe_ex(op, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride,
                                       wl.dilation, wl.pads, wl.mult, layout, wt,
                                       op == dw.OP_FWD)[0]
    return dw.dwconv2d_describe(op, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride,
                                wl.dilation, layout, wt, op == dw.OP_FWD)[0]


_SPIN_CYCLES_PER_US = None


def queue_ahead(torch, stream, us):
    """Enqueue a spin kernel of about `us` microseconds on `stream`.  It
    touches no memory; launches enqueued behind it then run back to back on
    the device, instead of each one waiting for the host to submit it (for
    launches of a few microseconds the binding's host time is longer than
    the kernel)."""
    global _SPIN_CYCLES_PER_US
    if _SPIN_CYCLES_PER_US is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda._sleep(10000)
            a.record(stream)
            torch.cuda._sleep(1000000)
            b.record(stream)
        stream.synchronize()
        _SPIN_CYCLES_PER_US = 1e6 / max(1.0, a.elapsed_time(b) * 1e3)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(us * _SPIN_CYCLES_PER_US))


def time_kernel(torch, fn, stream, iters, flush=None):
    """Per-launch kernel time (us) from HIP events recorded on `stream`.
    Without `flush` the launches are queued behind a spin kernel, so the
    events bracket device time only; with it, the 1 GiB pass before each
    launch keeps the device busy while the host submits."""
    times = []
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    if flush is None:
        queue_ahead(torch, stream, 200 + 150 * iters)
    with torch.cuda.stream(stream):
        for i in range(iters):
            if flush is not None:
                flush.add_(1.0)          # 1 GiB read+write: evicts L2 and the 256 MB MALL
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
    stream.synchronize()
    for s, e in zip(starts, ends):
        times.append(s.elapsed_time(e) * 1000.0)
    return times


def cpu_baseline(wl, rows=None, min_seconds=10.0):
    """The oracle (as it stands) on the first `rows` rows of the workload's
    image, forward and input gradient, repeated until about `min_seconds` of
    CPU work; the mean pass is scaled to the whole step."""
    import oracle
    from depthwise_convolution_amd import workloads
    rows = wl.H if rows is None else rows
    sub = workloads.Workload(name=wl.name + "_rows", N=wl.N, H=rows, W=wl.W, C=wl.C, kH=wl.kH,
                             kW=wl.kW, stride=wl.stride, dilation=wl.dilation)
    inp = workloads.make_inputs(sub, workloads.NHWC, seed=0)
    threads = max(1, min(16, os.cpu_count() or 1))
    reps, total = 0, 0.0
    while reps == 0 or total < min_seconds:
        t0 = time.perf_counter()
        oracle.fwd(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, workloads.NHWC,
                   nthreads=threads)
        oracle.input_grad(inp["dy"], inp["w"], rows, wl.W, wl.stride, wl.dilation,
                          workloads.NHWC, nthreads=threads)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    scale = wl.H / rows
    step_s = dt * scale
    gbs = (wl.fwd_bytes() + wl.ig_bytes()) / step_s / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"the whole {wl.H}x{wl.W}x{wl.C} image" if rows == wl.H else
                       f"rows 0..{rows - 1} of the {wl.H}x{wl.W}x{wl.C} image "
                       f"({rows / wl.H:.3g} of the outputs, time scaled x{scale:g})") +
                      f", forward + input gradient, fp64 oracle, mean of {reps} passes",
            "sample_seconds": round(total, 3), "passes": reps,
            "ms_per_step_est": round(step_s * 1e3, 1)}


def per_config_table(torch, dw, iters=20):
    from depthwise_convolution_amd import workloads
    rows = []
    flush = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device="cuda")   # 1 GiB
    stream = torch.cuda.Stream()
    for name, wl in workloads.WORKLOADS.items():
        if "parity_only" in wl.tags:
            continue
        for layout in (workloads.NHWC, workloads.NCHW):
            t = make_problem(torch, wl, layout, seed=0)
            for op, fn, nbytes in (("fwd", launch_fwd, wl.fwd_bytes()),
                                   ("ig", launch_ig, wl.ig_bytes()),
                                   ("wgrad", launch_wgrad, wgrad_bytes(wl)),
                                   ("fwd_bn_relu6", launch_fwd_bn_act, fwd_bn_act_bytes(wl)),
                                   ("wgrad_sgd", launch_wgrad_sgd, wgrad_sgd_bytes(wl))):
                if op.startswith("wgrad") and wl.fp16_weights:
                    continue              # the weight gradient does not read the weights
                call = (lambda f=fn: f(dw, wl, t, layout, stream))
                opc = {"fwd": dw.OP_FWD, "ig": dw.OP_INPUT_GRAD, "wgrad": dw.OP_WEIGHT_GRAD,
                       "fwd_bn_relu6": dw.OP_FWD, "wgrad_sgd": dw.OP_WEIGHT_GRAD}[op]
                kname = describe(dw, wl, opc, layout)
                time_kernel(torch, call, stream, 3)
                warm = statistics.median(time_kernel(torch, call, stream, iters))
                cold = statistics.median(time_kernel(torch, call, stream, max(5, iters // 4),
                                                     flush))
                rows.append({"workload": name, "layout": workloads.LAYOUT_NAMES[layout],
                             "op": op, "kernel": kname, "bytes": nbytes,
                             "warm_us": round(warm, 2), "cold_us": round(cold, 2),
                             "warm_GBs": round(nbytes / warm / 1e3, 1),
                             "cold_GBs": round(nbytes / cold / 1e3, 1),
                             "cold_pct_peak": round(100 * nbytes / cold / 1e3 / PEAK_HBM_GBS, 1)})
            del t
        _log(f"[table] {name} done")
    del flush
    return rows


def graph_leg(torch, dw, reps=20):
    """Launch-bound small problems: one training step (forward, input
    gradient, weight + bias gradient: 4 kernels) of the 112x112x32 3x3 NHWC
    workload, enqueued eagerly through the binding vs replayed from a HIP
    graph that holds `reps` steps.  Per-step time from the wall clock between
    device synchronisations."""
    from depthwise_convolution_amd import workloads
    wl = workloads.WORKLOADS["mobilenet_112x112x32_3x3"]
    layout = workloads.NHWC
    t = make_problem(torch, wl, layout, seed=0)
    stream = torch.cuda.Stream()

    def step():
        launch_fwd(dw, wl, t, layout, stream)
        launch_ig(dw, wl, t, layout, stream)
        launch_wgrad(dw, wl, t, layout, stream)

    def wall(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for _ in range(n):
                fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6

    with torch.cuda.stream(stream):
        for _ in range(20):
            step()
    eager_us = min(wall(step, reps) for _ in range(3)) / reps
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                step()
    torch.cuda.synchronize()
    g.replay()
    graph_us = min(wall(g.replay, 1) for _ in range(5)) / reps
    nbytes = wl.fwd_bytes() + wl.ig_bytes() + wgrad_bytes(wl)
    del g, t
    return {"workload": wl.name + " nhwc", "step": "fwd + ig + wgrad (4 kernels)",
            "eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
            "graph_GBs": round(nbytes / graph_us / 1e3, 1),
            "timing": f"best of 3 (eager) / 5 (graph) runs of {reps} steps, wall clock"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 50 untimed steps (~10 ms): the first ~100 steps of a process run ~6%
    # slower while the device settles, measured on MI355X
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-table", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path (the operator "
              "shards over images and channels with no exchange between GPUs, so each GPU "
              "would run this same kernel on its own share)", file=sys.stderr)
        sys.exit(2)

    import torch
    import depthwise_convolution_amd as dw
    from depthwise_convolution_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dw.lib()
    wl = workloads.WORKLOADS[HEADLINE]
    layout = workloads.NHWC
    _log(f"[bench] generating {HEADLINE} inputs")
    t = make_problem(torch, wl, layout, seed=0)
    stream = torch.cuda.Stream()

    def step():
        launch_fwd(dw, wl, t, layout, stream)
        launch_ig(dw, wl, t, layout, stream)

    _log("[bench] warmup")
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    # timed region: K steps, wall clock between device-wide synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    _log(f"[bench] timed {args.steps} steps in {wall * 1e3:.2f} ms")
    # per-kernel durations: the same steps again, untimed by the wall clock,
    # with HIP events on the launch stream around every kernel
    n_ev = min(args.steps, 50)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    with torch.cuda.stream(stream):
        for i in range(n_ev):
            ev[i][0].record(stream)
            launch_fwd(dw, wl, t, layout, stream)
            ev[i][1].record(stream)
            launch_ig(dw, wl, t, layout, stream)
            ev[i][2].record(stream)
    torch.cuda.synchronize()
    fwd_us = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
    ig_us = [e[1].elapsed_time(e[2]) * 1e3 for e in ev]

    step_bytes = wl.fwd_bytes() + wl.ig_bytes()
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    fwd_avg, ig_avg = statistics.mean(fwd_us), statistics.mean(ig_us)
    dom, dom_bytes = ("fwd", wl.fwd_bytes()) if fwd_avg >= ig_avg else ("ig", wl.ig_bytes())
    dom_kernel = dw.dwconv2d_describe(dw.OP_FWD if dom == "fwd" else dw.OP_INPUT_GRAD, wl.N,
                                      wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride, wl.dilation,
                                      layout, 0, dom == "fwd")[0]
    # Dominant kernel's launch duration with the event overhead amortised: two
    # events around 40 back-to-back launches that alternate between two
    # disjoint buffer sets (256 MiB in / out each), so no launch finds its
    # input in the 256 MB Infinity Cache.
    alt = {"x": t["dy"] if dom == "fwd" else t["x"], "y": t["dx"] if dom == "fwd" else t["y"]}
    assert t["x"].shape == t["dy"].shape, "the alternating-buffer timing needs stride 1"
    k_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n_rep = 40
    with torch.cuda.stream(stream):
        for i in range(n_rep + 4):
            if i == 4:
                k_ev[0].record(stream)
            if dom == "fwd":
                src, dst = (t["x"], t["y"]) if i % 2 == 0 else (alt["x"], alt["y"])
                dw.dwconv2d_fwd(src, t["w"], t["b"], dst, wl.stride, wl.dilation, layout, stream)
            else:
                src, dst = (t["dy"], t["dx"]) if i % 2 == 0 else (alt["y"], alt["x"])
                dw.dwconv2d_input_grad(src, t["w"], dst, wl.stride, wl.dilation, layout, stream)
        k_ev[1].record(stream)
    torch.cuda.synchronize()
    dom_us = k_ev[0].elapsed_time(k_ev[1]) * 1e3 / n_rep
    achieved = dom_bytes / dom_us / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(dom), "kernel": dom_kernel,
                "avg_launch_us": round(dom_us, 2),
                "avg_launch_us_events_each_launch": round(fwd_avg if dom == "fwd" else ig_avg, 2),
                "algorithmic_bytes_per_launch": dom_bytes}

    result = {
        "metric": "effective HBM bandwidth of depthwise conv2d forward + input-gradient "
                  "(x+y+W+b and dy+dx+W bytes)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic, seeded numpy: x, dy ~ N(0,1); W ~ N(0,1/9); b ~ U(-0.1,0.1)",
        "config": {"workload": HEADLINE, "N": wl.N, "H": wl.H, "W": wl.W, "C": wl.C,
                   "kernel": f"{wl.kH}x{wl.kW}", "stride": wl.stride, "dilation": wl.dilation,
                   "layout": "nhwc", "weights": "f32"},
        "fwd_us": round(fwd_avg, 2), "ig_us": round(ig_avg, 2),
        "fwd_pct_peak": round(100 * wl.fwd_bytes() / fwd_avg / 1e3 / PEAK_HBM_GBS, 1),
        "ig_pct_peak": round(100 * wl.ig_bytes() / ig_avg / 1e3 / PEAK_HBM_GBS, 1),
        "roofline": roofline,
    }
    # Weight gradient, fused epilogues: timed like the roofline launch (two
    # events around back-to-back launches alternating between two disjoint
    # buffer sets, so no launch reads what the previous one left in the
    # 256 MB Infinity Cache).  The second set for the weight gradient is a
    # copy of x and dy.
    x2, dy2 = t["x"].clone(), t["dy"].clone()
    ws, dW, db, bn = t["ws"], t["dW"], t["db"], t["bn"]

    def amortised(calls, n=40, what=""):
        """Median per-call time (us) of n back-to-back calls with an event
        between consecutive calls; a stall of the whole device (seen now and
        then on this machine, tens of milliseconds, outside any kernel's
        control) would otherwise dominate a mean, so it is reported apart."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        with torch.cuda.stream(stream):
            for c in calls:
                c()
            ev[0].record(stream)
            for i in range(n):
                calls[i % len(calls)]()
                ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)]
        med = statistics.median(us)
        if max(us) > 3 * med:
            _log(f"[bench] {what}: one call took {max(us):.0f} us (median {med:.1f} us)")
        return med

    def wgrad_call(xx, gg):
        return lambda: dw.dwconv2d_weight_grad(xx, gg, dW, db, ws, wl.stride, wl.dilation,
                                               layout, dw.STRATEGY_AUTO, stream)

    def sgd_call(xx, gg):
        return lambda: dw.dwconv2d_weight_grad_sgd_ex(xx, gg, t["w_sgd"], t["b_sgd"], 1e-4, ws,
                                                      None, None, wl.stride, wl.dilation, None,
                                                      1, layout, dw.STRATEGY_AUTO, stream)

    def fused_call(src, dst):
        return lambda: dw.dwconv2d_fwd_bn_act_ex(src, t["w"], t["b"], dst, bn, 1e-3,
                                                 dw.ACT_RELU6, wl.stride, wl.dilation, None, 1,
                                                 layout, dw.STRATEGY_AUTO, stream)

    def fwd_call(src, dst):
        return lambda: dw.dwconv2d_fwd(src, t["w"], t["b"], dst, wl.stride, wl.dilation, layout,
                                       stream)

    wg_us = amortised([wgrad_call(t["x"], t["dy"]), wgrad_call(x2, dy2)], what="wgrad")
    sgd_us = amortised([sgd_call(t["x"], t["dy"]), sgd_call(x2, dy2)], what="wgrad_sgd")
    fwd_ref_us = amortised([fwd_call(t["x"], t["y"]), fwd_call(t["dy"], t["dx"])], what="fwd")
    epi_us = amortised([fused_call(t["x"], t["y"]), fused_call(t["dy"], t["dx"])],
                       what="fwd_bn_relu6")
    # practical ceilings in the same run: a device copy of the headline
    # forward's bytes (256 MiB read + 256 MiB written, alternating two buffer
    # pairs like the roofline leg) and the smallest launch of this library
    c_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(stream):
        for src, dst in ((t["x"], t["y"]), (t["dy"], t["dx"])):
            dst.copy_(src)
        c_ev[0].record(stream)
        for i in range(n_rep):
            if i % 2 == 0:
                t["y"].copy_(t["x"])
            else:
                t["dx"].copy_(t["dy"])
        c_ev[1].record(stream)
    torch.cuda.synchronize()
    copy_us = c_ev[0].elapsed_time(c_ev[1]) * 1e3 / n_rep
    # the same bytes through torch's elementwise kernel (out = in * 1)
    with torch.cuda.stream(stream):
        torch.mul(t["x"], 1.0, out=t["y"])
        c_ev[0].record(stream)
        for i in range(n_rep):
            if i % 2 == 0:
                torch.mul(t["x"], 1.0, out=t["y"])
            else:
                torch.mul(t["dy"], 1.0, out=t["dx"])
        c_ev[1].record(stream)
    torch.cuda.synchronize()
    ew_us = c_ev[0].elapsed_time(c_ev[1]) * 1e3 / n_rep
    copy_bytes = 2 * t["x"].numel() * 4
    from depthwise_convolution_amd import workloads as _wls
    tiny = _wls.WORKLOADS["tiny_16x16x8_3x3"]
    tt = make_problem(torch, tiny, layout, seed=0)
    # GPU-side time of the smallest launch: 20 forwards of 16x16x8 captured in
    # a graph, replayed (the host cost of the Python binding is not in it)
    g_tiny = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        launch_fwd(dw, tiny, tt, layout, stream)
    stream.synchronize()
    with torch.cuda.graph(g_tiny, stream=stream):
        for _ in range(20):
            launch_fwd(dw, tiny, tt, layout, stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g_tiny.replay()
        c_ev[0].record(stream)
        for _ in range(5):
            g_tiny.replay()
        c_ev[1].record(stream)
    torch.cuda.synchronize()
    tiny_us = c_ev[0].elapsed_time(c_ev[1]) * 1e3 / 100
    del g_tiny, tt
    best_copy_gbs = copy_bytes / min(copy_us, ew_us) / 1e3
    result["ceilings"] = {
        "copy_bytes": copy_bytes,
        "runtime_copy_us": round(copy_us, 2),
        "runtime_copy_GBs": round(copy_bytes / copy_us / 1e3, 1),
        "elementwise_copy_us": round(ew_us, 2),
        "elementwise_copy_GBs": round(copy_bytes / ew_us / 1e3, 1),
        "headline_frac_of_best_copy": round(result["roofline"]["achieved"] / best_copy_gbs, 3),
        "tiny_fwd_launch_us_in_graph": round(tiny_us, 2),
        "timing": "copies: two events around 40 back-to-back copies alternating x->y and "
                  "dy->dx (256 MiB each way), as the roofline leg times its kernel; the "
                  "runtime copy is Tensor.copy_ (device-to-device memcpy), the elementwise "
                  "copy torch.mul(src, 1, out=dst); tiny launch: 20 forwards of 16x16x8 3x3 "
                  "captured in a HIP graph, replayed 5 times, per launch"}
    del x2, dy2
    result["wgrad"] = {
        "kernel": dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                       wl.stride, wl.dilation, layout)[0],
        "us": round(wg_us, 2), "algorithmic_bytes": wgrad_bytes(wl),
        "GBs": round(wgrad_bytes(wl) / wg_us / 1e3, 1),
        "pct_peak": round(100 * wgrad_bytes(wl) / wg_us / 1e3 / PEAK_HBM_GBS, 1),
        "timing": "median over 40 back-to-back calls (partial sums + reduction each) with an "
                  "event between calls, alternating between two copies of x and dy"}
    result["fused"] = {
        "timing": "median over 40 back-to-back calls with an event between calls, "
                  "alternating between two disjoint buffer sets",
        "fwd_bn_relu6_us": round(epi_us, 2), "fwd_us_same_timing": round(fwd_ref_us, 2),
        "fwd_bn_relu6_pct_peak": round(100 * fwd_bn_act_bytes(wl) / epi_us / 1e3 /
                                       PEAK_HBM_GBS, 1),
        "wgrad_sgd_us": round(sgd_us, 2),
        "wgrad_sgd_pct_peak": round(100 * wgrad_sgd_bytes(wl) / sgd_us / 1e3 / PEAK_HBM_GBS, 1),
        "note": "one pass each: the BatchNorm + ReLU6 epilogue is applied in the forward's "
                "store, the SGD step in the weight-gradient reduction"}
    del t
    torch.cuda.empty_cache()
    result["graph"] = graph_leg(torch, dw)
    if args.calib_copy:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter
        # readings calibrate the counters of the kernels above
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = src.numel() * 4
        del src, dst
    if not args.no_cpu:
        _log("[bench] cpu baseline (oracle sample)")
        result["cpu_baseline"] = cpu_baseline(wl)
    else:
        result["cpu_baseline"] = None
    if not args.no_table:
        _log("[bench] per-workload table")
        result["per_config"] = per_config_table(torch, dw)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
