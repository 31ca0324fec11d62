"""Benchmark: depthwise conv2d forward + input gradient on one MI355X.

A step is one forward and one input gradient of the 512x512x256 3x3 NHWC
workload (fp32 activations and weights), inputs resident in HBM.  The last
stdout line is one short JSON object: whole-step effective HBM bandwidth
(algorithmic bytes: x+y+W+b for the forward, dy+dx+W for the input
gradient), the roofline of the dominant kernel timed with HIP events on its
own stream, and the CPU oracle (single-precision timing build) on the host's
cores.  Everything else -- the per-workload table (forward, input gradient,
weight gradient and the fused ops in both layouts, each against its HBM or
VALU floor, an empty-launch floor and a same-bytes copy, and the oracle's
time on all cores and on one), the practical ceilings, the weight-gradient,
fused and graph legs -- goes to a JSON detail file (--detail, default
dwconv_bench_detail.json in the system's temporary directory) and, one line
per row, to stderr.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-table] [--no-cpu]
                       [--detail PATH] [--table-only] [--calib-copy]
       python bench.py --trace-table KERNEL_TRACE_CSV [--out MD]   (no GPU: summarise a
                       rocprofv3 kernel trace of a --table-only run per workload)
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
# fp32 FMA without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz
PEAK_VALU_TFLOPS = 78.6
HEADLINE = "large_512x512x256_3x3"
# the sources that decide the headline kernel's code and plan: a change to any
# of them makes the recorded traffic counts stale
KERNEL_SRCS = [os.path.join(ROOT, "depthwise_convolution_amd", "csrc", f)
               for f in ("dwconv_internal.h", "dwconv_device.h", "dwconv_tiled_nhwc.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_large_512x512x256_3x3_nhwc.json")
OPS = ("fwd", "ig", "wgrad", "fwd_bn_relu6", "wgrad_sgd")


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


# ------------------------------------------------------------------ problems
def to_dev(torch, a):
    return torch.from_numpy(a).to("cuda")


def workspace_bytes(dw, wl, layout):
    if wl.general:
        return dw.dwconv2d_weight_grad_workspace_size_ex(wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                                         wl.stride, wl.dilation, wl.pads,
                                                         wl.mult, layout)
    return dw.dwconv2d_weight_grad_workspace_size(wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                                  wl.stride, wl.dilation, layout)


def make_problem(torch, wl, layout, seed=0, inputs=None):
    """Device tensors of a workload: x, w, b, dy (seeded draws), outputs y, dx,
    dW, db, the weight-gradient workspace, BatchNorm arrays and the SGD step's
    float32 weights / bias."""
    from depthwise_convolution_amd import workloads
    import depthwise_convolution_amd as dw
    inp = inputs if inputs is not None else workloads.make_inputs(wl, layout, seed=seed)
    t = {k: (None if v is None else to_dev(torch, v)) for k, v in inp.items()}
    t["y"] = torch.empty(tuple(inp["dy"].shape), dtype=torch.float32, device="cuda")
    t["dx"] = torch.empty(tuple(inp["x"].shape), dtype=torch.float32, device="cuda")
    nws = workspace_bytes(dw, wl, layout)
    t["ws"] = torch.empty(max(4, (nws + 15) // 16 * 4), dtype=torch.float32, device="cuda")
    t["dW"] = torch.empty((wl.Co, wl.kH, wl.kW), dtype=torch.float32, device="cuda")
    t["db"] = torch.empty((wl.Co,), dtype=torch.float32, device="cuda")
    # inference BatchNorm of the output channels (gamma, beta, mean, var)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    t["bn"] = tuple((torch.rand(wl.Co, generator=g) * s + o).to("cuda")
                    for s, o in ((1.5, 0.5), (2.0, -1.0), (1.0, -0.5), (2.8, 0.2)))
    t["w_sgd"] = torch.from_numpy(inp["w"].astype("float32")).to("cuda")
    t["b_sgd"] = torch.zeros((wl.Co,), dtype=torch.float32, device="cuda")
    return t


def second_set(torch, t):
    """Another copy of the tensors a launch reads and writes, so back-to-back
    launches can alternate between two disjoint buffer sets."""
    u = dict(t)
    for k in ("x", "dy", "y", "dx", "ws", "dW", "db"):
        u[k] = t[k].clone()
    return u


# ------------------------------------------------------------------ launches
def launch(dw, wl, t, layout, op, stream):
    """Enqueue one op of a workload through the C ABI (the AUTO strategy)."""
    g = wl.general
    if op == "fwd":
        if g:
            dw.dwconv2d_launch_ex(dw.OP_FWD, t["x"], t["w"], t["b"], t["y"], wl.H, wl.W,
                                  wl.stride, wl.dilation, wl.pads, wl.mult, layout,
                                  dw.STRATEGY_AUTO, stream)
        else:
            dw.dwconv2d_fwd(t["x"], t["w"], t["b"], t["y"], wl.stride, wl.dilation, layout,
                            stream)
    elif op == "ig":
        if g:
            dw.dwconv2d_launch_ex(dw.OP_INPUT_GRAD, t["dy"], t["w"], None, t["dx"], wl.H, wl.W,
                                  wl.stride, wl.dilation, wl.pads, wl.mult, layout,
                                  dw.STRATEGY_AUTO, stream)
        else:
            dw.dwconv2d_input_grad(t["dy"], t["w"], t["dx"], wl.stride, wl.dilation, layout,
                                   stream)
    elif op == "wgrad":
        if g:
            dw.dwconv2d_weight_grad_ex(t["x"], t["dy"], t["dW"], t["db"], t["ws"], wl.stride,
                                       wl.dilation, wl.pads, wl.mult, layout, dw.STRATEGY_AUTO,
                                       stream)
        else:
            dw.dwconv2d_weight_grad(t["x"], t["dy"], t["dW"], t["db"], t["ws"], wl.stride,
                                    wl.dilation, layout, dw.STRATEGY_AUTO, stream)
    elif op == "fwd_bn_relu6":
        # forward with the fused BatchNorm + ReLU6 epilogue (MobileNetV2 block)
        dw.dwconv2d_fwd_bn_act_ex(t["x"], t["w"], t["b"], t["y"], t["bn"], 1e-3, dw.ACT_RELU6,
                                  wl.stride, wl.dilation, wl.pads, wl.mult, layout,
                                  dw.STRATEGY_AUTO, stream)
    elif op == "wgrad_sgd":
        # weight + bias gradient with the fused SGD step (w, b updated in place)
        dw.dwconv2d_weight_grad_sgd_ex(t["x"], t["dy"], t["w_sgd"], t["b_sgd"], 1e-4, t["ws"],
                                       None, None, wl.stride, wl.dilation, wl.pads, wl.mult,
                                       layout, dw.STRATEGY_AUTO, stream)
    else:
        raise ValueError(op)


def op_bytes(wl, op):
    """Algorithmic HBM bytes of one call."""
    if op == "fwd":
        return wl.fwd_bytes()
    if op == "ig":
        return wl.ig_bytes()
    if op == "wgrad":
        return wl.wgrad_bytes()                       # x + dy + dW + db
    if op == "fwd_bn_relu6":
        return wl.fwd_bytes() + 16 * wl.Co            # + the four BatchNorm arrays
    # x + dy read, W and b read and written (the gradients are not written)
    return (4 * wl.N * wl.H * wl.W * wl.C + 4 * wl.N * wl.Ho * wl.Wo * wl.Co
            + 8 * wl.Co * wl.kH * wl.kW + 8 * wl.Co)


def op_flops(wl, op):
    """Algorithmic fp32 flops: every dy / y element meets every tap once (one
    FMA = 2 flops) in all three ops."""
    return 2 * wl.kH * wl.kW * wl.N * wl.Ho * wl.Wo * wl.Co


def floors(wl, op):
    """(bound, floor us): the larger of the HBM time of the algorithmic bytes
    at 8 TB/s and the VALU time of the algorithmic flops at 78.6 TFLOP/s."""
    t_hbm = op_bytes(wl, op) / PEAK_HBM_GBS / 1e3
    t_alu = op_flops(wl, op) / PEAK_VALU_TFLOPS / 1e6
    return ("hbm", t_hbm) if t_hbm >= t_alu else ("alu", t_alu)


def describe(dw, wl, op, layout):
    """Kernel name of an op of a workload under the AUTO strategy."""
    opc = {"fwd": dw.OP_FWD, "ig": dw.OP_INPUT_GRAD, "wgrad": dw.OP_WEIGHT_GRAD,
           "fwd_bn_relu6": dw.OP_FWD, "wgrad_sgd": dw.OP_WEIGHT_GRAD}[op]
    wt = 0 if opc == dw.OP_WEIGHT_GRAD else int(wl.fp16_weights)
    return dw.dwconv2d_describe_ex(opc, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride,
                                   wl.dilation, wl.pads, wl.mult, layout, wt,
                                   opc == dw.OP_FWD)[0]


# ------------------------------------------------------------------ timing
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


def amortised(torch, stream, calls, n=40, host_us=60.0, reps=3):
    """Per-call device time (us) of n back-to-back calls that cycle through
    `calls` (e.g. the same op on two disjoint buffer sets), between two events,
    all queued behind a spin kernel so the device never waits for the host;
    the median of `reps` such runs."""
    return statistics.median(_amortised_once(torch, stream, calls, n, host_us)
                             for _ in range(reps))


def _amortised_once(torch, stream, calls, n, host_us):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    queue_ahead(torch, stream, 300 + host_us * (n + 2))
    with torch.cuda.stream(stream):
        calls[0]()
        calls[-1]()
        a.record(stream)
        for i in range(n):
            calls[i % len(calls)]()
        b.record(stream)
    stream.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def cold_median(torch, stream, call, flush, sink, reps=5):
    """Median of `reps` single-call times, each after a read-only pass over a
    1 GiB buffer (evicts L2 and the 256 MB Infinity Cache without leaving
    dirty lines for the timed call to write back); two events around the
    call, so an event pair's own overhead is in it (`event_pair_us`)."""
    times = []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        with torch.cuda.stream(stream):
            torch.sum(flush, 0, out=sink)
            ev[0].record(stream)
            call()
            ev[1].record(stream)
        stream.synchronize()
        times.append(ev[0].elapsed_time(ev[1]) * 1e3)
    return statistics.median(times)


# ------------------------------------------------------------------ CPU oracle
def cpu_threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n or 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class CpuOracle:
    """The oracle's timing build (same source, single-precision accumulation,
    -O3 -march=native, OpenMP), compiled on this host; the parity build is
    restored on close."""

    def __init__(self):
        import oracle
        from oracle import build as obuild
        self.oracle = oracle
        self.dir = tempfile.mkdtemp(prefix="dwconv_cpu_")
        self.prev = oracle.swap_library(obuild.build_timing(self.dir))

    def close(self):
        import shutil
        self.oracle.restore_library(self.prev)
        shutil.rmtree(self.dir, ignore_errors=True)

    def run(self, wl, inp, layout, op, threads):
        o = self.oracle
        if op == "fwd":
            if wl.general:
                o.fwd_general(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, wl.pads,
                              wl.mult, layout, nthreads=threads, with_sum=False)
            else:
                o.fwd(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, layout,
                      nthreads=threads, with_sum=False)
        else:
            if wl.general:
                o.input_grad_general(inp["dy"], inp["w"], wl.H, wl.W, wl.stride, wl.dilation,
                                     wl.pads, wl.mult, layout, nthreads=threads, with_sum=False)
            else:
                o.input_grad(inp["dy"], inp["w"], wl.H, wl.W, wl.stride, wl.dilation, layout,
                             nthreads=threads, with_sum=False)

    def time(self, wl, inp, layout, op, threads, reps=3):
        """Median of `reps` timed runs (us) after one untimed run."""
        self.run(wl, inp, layout, op, threads)
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            self.run(wl, inp, layout, op, threads)
            ts.append((time.perf_counter() - t0) * 1e6)
        return statistics.median(ts)


def cpu_baseline(cpu, wl, inp, threads):
    """The oracle on the host's cores: the headline step (forward + input
    gradient of the whole image), median of 3 each, and on one thread."""
    fwd = cpu.time(wl, inp, 0, "fwd", threads)
    ig = cpu.time(wl, inp, 0, "ig", threads)
    fwd1 = cpu.time(wl, inp, 0, "fwd", 1, reps=1)
    ig1 = cpu.time(wl, inp, 0, "ig", 1, reps=1)
    step_bytes = wl.fwd_bytes() + wl.ig_bytes()
    return {
        "value": round(step_bytes / (fwd + ig) / 1e3, 2), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"whole {wl.H}x{wl.W}x{wl.C} {wl.kH}x{wl.kW} NHWC image, fwd + ig, oracle "
                   f"timing build (fp32 accumulation, -O3 -march=native), median of 3"),
        "detail": {"fwd_us": round(fwd, 1), "ig_us": round(ig, 1),
                   "fwd_us_1thread": round(fwd1, 1), "ig_us_1thread": round(ig1, 1),
                   "GBs_1thread": round(step_bytes / (fwd1 + ig1) / 1e3, 2),
                   "cpu_model": cpu_model()}}


# ------------------------------------------------------------------ legs
def per_config_table(torch, dw, cpu, threads, only=None):
    """Every workload (not parity-only), both layouts, all ops: amortised
    back-to-back device time, cold single-call time, the op's HBM / VALU
    floor, a same-bytes copy for problems up to 8 MB, and the oracle's forward
    and input-gradient times on all cores (median of 3) and on one thread."""
    from depthwise_convolution_amd import workloads
    rows = []
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")   # 1 GiB
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    for name, wl in workloads.WORKLOADS.items():
        if "parity_only" in wl.tags or (only and name not in only):
            continue
        for layout in (workloads.NHWC, workloads.NCHW):
            inp = workloads.make_inputs(wl, layout, seed=0)
            t = make_problem(torch, wl, layout, inputs=inp)
            t2 = second_set(torch, t)
            for op in OPS:
                if op.startswith("wgrad") and wl.fp16_weights:
                    continue              # the weight gradient does not read the weights
                nbytes = op_bytes(wl, op)
                calls = [(lambda tt=tt: launch(dw, wl, tt, layout, op, stream)) for tt in (t, t2)]
                am = amortised(torch, stream, calls)
                cold = cold_median(torch, stream, calls[0], flush, sink)
                bound, floor_us = floors(wl, op)
                row = {"workload": name, "layout": workloads.LAYOUT_NAMES[layout], "op": op,
                       "kernel": describe(dw, wl, op, layout), "bytes": nbytes,
                       "flops": op_flops(wl, op),
                       "us": round(am, 2), "cold_us": round(cold, 2),
                       "GBs": round(nbytes / am / 1e3, 1),
                       "pct_hbm_peak": round(100 * nbytes / am / 1e3 / PEAK_HBM_GBS, 1),
                       "TFLOPs": round(op_flops(wl, op) / am / 1e6, 2),
                       "bound": bound, "floor_us": round(floor_us, 3),
                       "frac_of_bound": round(floor_us / am, 3)}
                if nbytes <= 8 * 1000 * 1000 and op in ("fwd", "ig"):
                    half = max(1, nbytes // 8)           # floats each way
                    src = [torch.ones(half, device="cuda") for _ in range(2)]
                    dst = [torch.empty(half, device="cuda") for _ in range(2)]
                    cp = [(lambda i=i: dst[i].copy_(src[i])) for i in range(2)]
                    row["copy_same_bytes_us"] = round(amortised(torch, stream, cp), 2)
                    del src, dst
                if cpu is not None and op in ("fwd", "ig"):
                    row["cpu_us"] = round(cpu.time(wl, inp, layout, op, threads), 1)
                    row["cpu_us_1thread"] = round(cpu.time(wl, inp, layout, op, 1, reps=1), 1)
                    row["cpu_threads"] = threads
                rows.append(row)
                _log("[row] " + json.dumps(row))
            del t, t2
        torch.cuda.empty_cache()
    del flush
    return rows


def calibration_kernels(torch, dw, workloads, detail, layout, stream):
    """Kernels of known HBM traffic, whose FETCH_SIZE / WRITE_SIZE counter
    readings calibrate the counters of the kernels above: a plain 256 MiB
    device copy, and the 1x1 tiled forward of 512x512x256 (its input read
    once through the same 16-byte loads into LDS as the 3x3 kernels, its
    output written once), alternating two buffer sets so neither finds its
    input in the Infinity Cache."""
    src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    detail["calib_copy_bytes"] = src.numel() * 4
    sets = [(torch.randn(1, 512, 512, 256, device="cuda"),
             torch.empty(1, 512, 512, 256, device="cuda")) for _ in range(2)]
    w1 = torch.randn(256, 1, 1, device="cuda")
    b1 = torch.randn(256, device="cuda")
    detail["calib_1x1_kernel"] = describe(dw, workloads.Workload(
        name="calib", N=1, H=512, W=512, C=256, kH=1, kW=1), "fwd", layout)
    for i in range(6):
        xx, yy = sets[i % 2]
        dw.dwconv2d_fwd(xx, w1, b1, yy, 1, 1, layout, stream)
    torch.cuda.synchronize()
    detail["calib_1x1_bytes"] = {"read": 512 * 512 * 256 * 4 + 256 * 8,
                                 "written": 512 * 512 * 256 * 4}
    del src, dst, sets


def launch_floor(torch, stream, flush, sink):
    """The smallest launch: an empty kernel (a zero-cycle spin), back to back
    (amortised, queued ahead) and as one call between two events after the
    read-only flush (the overhead in every `cold_us`)."""
    k = (lambda: torch.cuda._sleep(0))
    with torch.cuda.stream(stream):
        am = amortised(torch, stream, [k], n=200, host_us=10.0)
    ev = cold_median(torch, stream, k, flush, sink, reps=9)
    return {"empty_launch_us": round(am, 3), "event_pair_us": round(ev, 3),
            "note": "empty kernel (torch.cuda._sleep(0)): 200 back-to-back launches between "
                    "two events, queued behind a spin kernel; and one launch between two "
                    "events after the 1 GiB read-only flush, median of 9"}


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
        for op in ("fwd", "ig", "wgrad"):
            launch(dw, wl, t, layout, op, stream)

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
    nbytes = wl.fwd_bytes() + wl.ig_bytes() + wl.wgrad_bytes()
    del g, t
    return {"workload": wl.name + " nhwc", "step": "fwd + ig + wgrad (4 kernels)",
            "eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
            "graph_GBs": round(nbytes / graph_us / 1e3, 1),
            "timing": f"best of 3 (eager) / 5 (graph) runs of {reps} steps, wall clock"}


def headline_extras(torch, dw, wl, t, layout, stream, n_rep=40):
    """Weight gradient and fused ops of the headline workload, and the plain
    copies of its forward's bytes, each timed like the roofline leg
    (back-to-back calls alternating between two disjoint buffer sets)."""
    t2 = second_set(torch, t)
    out = {}
    for op in ("wgrad", "wgrad_sgd", "fwd", "fwd_bn_relu6"):
        calls = [(lambda tt=tt: launch(dw, wl, tt, layout, op, stream)) for tt in (t, t2)]
        us = amortised(torch, stream, calls, n=n_rep)
        out[op] = {"kernel": describe(dw, wl, op, layout), "us": round(us, 2),
                   "pct_hbm_peak": round(100 * op_bytes(wl, op) / us / 1e3 / PEAK_HBM_GBS, 1)}
    # practical ceilings: the forward's bytes (256 MiB read + 256 MiB written)
    # through the runtime's device copy and through torch's elementwise kernel
    cp = [(lambda: t["y"].copy_(t["x"])), (lambda: t2["y"].copy_(t2["x"]))]
    ew = [(lambda: torch.mul(t["x"], 1.0, out=t["y"])),
          (lambda: torch.mul(t2["x"], 1.0, out=t2["y"]))]
    copy_bytes = 2 * t["x"].numel() * 4
    copy_us = amortised(torch, stream, cp, n=n_rep)
    ew_us = amortised(torch, stream, ew, n=n_rep)
    out["ceilings"] = {"copy_bytes": copy_bytes,
                       "runtime_copy_us": round(copy_us, 2),
                       "runtime_copy_GBs": round(copy_bytes / copy_us / 1e3, 1),
                       "elementwise_copy_us": round(ew_us, 2),
                       "elementwise_copy_GBs": round(copy_bytes / ew_us / 1e3, 1)}
    del t2
    return out


# ------------------------------------------------------------------ trace table
# plan-name prefix -> the HIP kernel (family) that runs it
PLAN_KERNEL_FAMILIES = {
    "tiled_nhwc": "k_tiled_nhwc", "tiled_nchw": "k_tiled_nchw",
    "stream_nhwc": "k_stream_nhwc", "stream_nchw": "k_stream_nchw",
    "stream_nchw_planes": "k_stream_nchw_planes",
    "direct_nhwc": "k_direct_nhwc", "direct_nchw": "k_direct_nchw",
    "wgrad_tiled_nhwc": "k_wgrad_tiled_nhwc", "wgrad_tiled_nchw": "k_wgrad_tiled_nchw",
    "wgrad_stream_nchw": "k_wgrad_stream_nchw", "wgrad_stream_nhwc": "k_wgrad_stream_nhwc",
    "wgrad_direct": "k_wgrad_gen"}


def kernel_family(plan_name):
    """The kernel family of a plan name (longest matching prefix), or None."""
    return next((v for k, v in sorted(PLAN_KERNEL_FAMILIES.items(), key=lambda kv: -len(kv[0]))
                 if plan_name.startswith(k)), None)


def _row_matcher(dw, wl, layout, op):
    """The kernel name the plan of (workload, layout, op) reports and a
    predicate on a trace's (kernel name, grid size in threads) that accepts
    that plan's main kernel: the family and grid from the describe call, the
    weight type and the op from the template arguments where the kernel is a
    template (the weight-gradient and direct kernels take their shape at run
    time, so several workloads share one name; `_assign_rows` tells them
    apart by dispatch order)."""
    import re
    opc = {"fwd": dw.OP_FWD, "ig": dw.OP_INPUT_GRAD, "wgrad": dw.OP_WEIGHT_GRAD,
           "fwd_bn_relu6": dw.OP_FWD, "wgrad_sgd": dw.OP_WEIGHT_GRAD}[op]
    kname, grid, block = dw.dwconv2d_describe_ex(
        opc, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride, wl.dilation, wl.pads,
        wl.mult, layout, 0 if opc == dw.OP_WEIGHT_GRAD else int(wl.fp16_weights),
        opc == dw.OP_FWD)
    kfam = kernel_family(kname)
    # the tiled and streaming kernels' mode: 0 forward, 1 input gradient,
    # 2 forward with the BatchNorm + activation epilogue
    want = {"fwd": "0", "ig": "1", "fwd_bn_relu6": "2"}.get(op)

    def match(kn, g):
        m = re.search(r"(k_\w+)(?:<(.*?)>)?\(", kn)
        if not m or m.group(1) != kfam or g != grid * block:
            return False
        parts = (m.group(2) or "").replace(" ", "").split(",")
        if want is None:
            return True
        if parts[0] in ("float", "_Float16", "half") and \
                (parts[0] != "float") != bool(wl.fp16_weights):
            return False
        # the mode in the template arguments: the tiled kernels' third from
        # last, the streaming kernels' last; the direct kernels' input-gradient
        # flag (their epilogue is a run-time argument)
        if kfam.startswith("k_tiled") and parts[-3] != want:
            return False
        if kfam.startswith("k_stream") and parts[-1] != want:
            return False
        if kfam.startswith("k_direct"):
            flags = [q for q in parts if q in ("true", "false")]
            if flags and flags[0] != ("true" if want == "1" else "false"):
                return False
        return True
    return kname, match


def _assign_rows(dw, order, seq):
    """Split `seq`, the trace's dispatches in issue order as (kernel name,
    grid threads, value), over `order`, the (workload, layout, op) rows in
    the order the table ran them: a row takes the run of dispatches that
    match its kernel, skipping other programs' kernels (flush, copies, spin)
    and the fixed-order weight-gradient reduction, up to the first dwconv
    kernel it does not launch.  A row that meets the next row's kernel
    before its own ran nothing (it takes no later row's dispatches of a
    kernel the two share); dispatches no row claims (legs before the table,
    a trace of an older plan) are skipped.  Adjacent rows always differ in
    layout or op, hence in kernel.  Returns one (reported name, trace name,
    values) per row."""
    def own_kernel(n):
        return "dwconv::" in n and "k_wgrad_reduce" not in n

    matchers = [_row_matcher(dw, wl, layout, op) for wl, layout, op in order]
    out, cursor = [], 0
    for r in range(len(order)):
        kname, match = matchers[r]
        nxt = matchers[r + 1][1] if r > 0 and r + 1 < len(order) else None
        i = cursor
        while i < len(seq) and not match(seq[i][0], seq[i][1]):
            if nxt is not None and nxt(seq[i][0], seq[i][1]):
                i = len(seq)              # the next row's kernel: this row ran nothing
                break
            i += 1
        if i == len(seq):
            out.append((kname, None, []))
            continue
        vals, tname, j = [], seq[i][0], i
        while j < len(seq):
            n, g, v = seq[j]
            if match(n, g):
                vals.append(v)
            elif own_kernel(n):
                break
            j += 1
        out.append((kname, tname, vals))
        cursor = j
    return out


def _table_order(detail_path):
    """The (workload, layout, op) rows of a `bench.py` detail file, in the
    order its per-workload table ran them."""
    from depthwise_convolution_amd import workloads
    with open(detail_path) as f:
        rows = json.load(f)["per_config"]
    lay = {v: k for k, v in workloads.LAYOUT_NAMES.items()}
    return [(workloads.WORKLOADS[r["workload"]], lay[r["layout"]], r["op"]) for r in rows]


def _dispatch_seq(csv_path, counter=None):
    """(kernel name, grid threads, value) per dispatch in dispatch order: the
    counter's reading for a --pmc CSV, the duration in us for a kernel trace."""
    import csv
    seq = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if counter is not None:
                if r.get("Counter_Name") != counter:
                    continue
                v = float(r["Counter_Value"])
            else:
                v = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            g = int(r.get("Grid_Size_X", r.get("Grid_Size", "0")) or 0)
            seq.append((int(r.get("Dispatch_Id", 0) or 0), int(r["Start_Timestamp"]),
                        r["Kernel_Name"], g, v))
    seq.sort(key=lambda s: (s[1], s[0]) if counter is None else (s[0], s[1]))
    return [s[2:] for s in seq]


def counter_table(fetch_csv, write_csv, detail_path, out_path=None):
    """HBM traffic per workload from two rocprofv3 --pmc runs of `bench.py
    --table-only --calib-copy` (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch) and that run's detail file (the row order): the counters of
    the runtime's 256 MiB device copies calibrate them (bytes moved /
    counter reading), and the 1x1 tiled forward of 512x512x256, which reads
    its input and writes its output exactly once through the same 16-byte
    loads into LDS as the tiled kernels, checks the calibration.  Per
    (workload, layout, op): median counter per dispatch, scaled, against
    the algorithmic bytes.  No GPU needed."""
    import depthwise_convolution_amd as dw
    from depthwise_convolution_amd import workloads

    fseq, wseq = _dispatch_seq(fetch_csv, "FETCH_SIZE"), _dispatch_seq(write_csv, "WRITE_SIZE")
    kib = 1024.0
    copy_bytes = 256 * 1024 * 1024

    def calib(seq):
        # the 256 MiB copies: the runtime copy dispatches within 10 % of the
        # largest reading (the smaller same-bytes copies share their grid)
        vals = [v for n, g, v in seq if "copyBuffer" in n]
        if not vals:
            return None, 0
        big = [v for v in vals if v >= 0.9 * max(vals)]
        return copy_bytes / (statistics.median(big) * kib), len(big)

    (sf, nf), (sw, nw) = calib(fseq), calib(wseq)
    one = workloads.Workload(name="calib_1x1", N=1, H=512, W=512, C=256, kH=1, kW=1)
    lines = [f"Calibration: {nf} / {nw} runtime copies of 256 MiB read FETCH_SIZE = "
             f"{copy_bytes / sf / kib:.1f} KiB and write WRITE_SIZE = {copy_bytes / sw / kib:.1f} "
             f"KiB per dispatch (medians): FETCH_SIZE x {sf:.4f}, WRITE_SIZE x {sw:.4f} "
             f"give bytes." if sf and sw else "Calibration: no copy dispatch found."]
    (_, _, v1f), = _assign_rows(dw, [(one, workloads.NHWC, "fwd")], fseq)
    (_, _, v1w), = _assign_rows(dw, [(one, workloads.NHWC, "fwd")], wseq)
    if v1f and v1w and sf and sw:
        r1 = statistics.median(v1f) * kib * sf
        w1 = statistics.median(v1w) * kib * sw
        lines.append(f"Check: the 1x1 tiled forward of 512x512x256 (reads 268,437,504 B, writes "
                     f"268,435,456 B; {len(v1f)} dispatches) measures {r1:,.0f} B read "
                     f"({r1 / 268437504:.3f}x) and {w1:,.0f} B written ({w1 / 268435456:.3f}x) "
                     f"with this calibration.")
    lines += ["", "Per dispatch, median over the row's dispatches (warm-up, back-to-back and "
              "cold calls; weight gradient: its partial-sum kernel, the reduction excluded).",
              "", "| workload | layout | op | kernel | dispatches | read MiB | written MiB | "
              "HBM bytes | algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|---|---|---|"]
    order = _table_order(detail_path)
    rows = {}
    for (wl, layout, op), (kname, _, vf), (_, _, vw) in zip(
            order, _assign_rows(dw, order, fseq), _assign_rows(dw, order, wseq)):
        if not vf or not vw or not sf:
            continue
        rb = statistics.median(vf) * kib * sf
        wb = statistics.median(vw) * kib * sw
        alg = op_bytes(wl, op)
        lname = workloads.LAYOUT_NAMES[layout]
        rows[(wl.name, lname, op)] = {
            "kernel": kname, "hbm_bytes_per_launch": round(rb + wb),
            "read_bytes": round(rb), "written_bytes": round(wb),
            "algorithmic_bytes": alg, "ratio": round((rb + wb) / alg, 3)}
        lines.append(f"| {wl.name} | {lname} | {op} | `{kname}` | {len(vf)} | "
                     f"{rb / 2**20:.2f} | {wb / 2**20:.2f} | {rb + wb:,.0f} | {alg:,} | "
                     f"{(rb + wb) / alg:.3f} |")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text, rows, (sf, sw)


def trace_table(csv_path, detail_path, out_path=None):
    """Summarise a rocprofv3 kernel-trace CSV of a `bench.py` run per
    workload, with that run's detail file giving the table's row order: each
    row's dispatches (`_assign_rows`) give median / mean / min device time
    (for the weight gradient: its first, partial-sum kernel; the fixed-order
    reduction that follows is a dispatch of its own, 3-5 us).  No GPU
    needed."""
    import depthwise_convolution_amd as dw
    from depthwise_convolution_amd import workloads
    seq = _dispatch_seq(csv_path)
    order = _table_order(detail_path)
    lines = ["| workload | layout | op | kernel | calls | median us | mean us | min us | "
             "floor us (bound) | median frac of floor |", "|---|---|---|---|---|---|---|---|---|---|"]
    for (wl, layout, op), (kname, _, ds) in zip(order, _assign_rows(dw, order, seq)):
        if not ds:
            continue
        bound, floor_us = floors(wl, op)
        med = statistics.median(ds)
        lines.append(f"| {wl.name} | {workloads.LAYOUT_NAMES[layout]} | {op} | "
                     f"`{kname}` | {len(ds)} | {med:.2f} | {statistics.mean(ds):.2f} | "
                     f"{min(ds):.2f} | {floor_us:.2f} ({bound}) | "
                     f"{floor_us / med:.3f} |")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text


def detail_table(detail_path, out_path=None):
    """The per-workload table of a `bench.py` detail file as markdown, with
    the run's floors, ceilings, CPU baseline and graph leg.  No GPU needed."""
    with open(detail_path) as f:
        d = json.load(f)
    res = d.get("result", {})
    lines = []
    if res:
        roof = res.get("roofline", {})
        lines += [f"Headline: {res.get('config', {}).get('workload')} {res.get('config', {}).get('layout')}"
                  f" fwd + ig, {res.get('value')} {res.get('unit')} ({res.get('ms_per_step')} ms per "
                  f"step); dominant kernel `{roof.get('kernel')}` {roof.get('avg_launch_us')} us per "
                  f"launch = {roof.get('achieved')} GB/s = {roof.get('frac')} of 8 TB/s.", ""]
    lf = d.get("launch_floor")
    if lf:
        lines += [f"Launch floor: empty kernel back to back {lf['empty_launch_us']} us; one launch "
                  f"between two events after the flush {lf['event_pair_us']} us.", ""]
    ce = d.get("headline_extras", {}).get("ceilings")
    if ce:
        lines += [f"Ceilings (headline forward's bytes, {ce['copy_bytes']:,} B): runtime copy "
                  f"{ce['runtime_copy_us']} us ({ce['runtime_copy_GBs']} GB/s), elementwise copy "
                  f"{ce['elementwise_copy_us']} us ({ce['elementwise_copy_GBs']} GB/s); headline "
                  f"kernel at {ce['headline_frac_of_best_copy']} of the better copy.", ""]
    cb = d.get("cpu_baseline") or res.get("cpu_baseline")
    if cb:
        det = cb.get("detail", {})
        lines += [f"CPU baseline: {cb.get('value')} {cb.get('unit')} on {cb.get('cores')} threads "
                  f"({det.get('cpu_model', '?')}); {cb.get('sample')}.", ""]
    g = d.get("graph")
    if g:
        lines += [f"Graph leg ({g['workload']}, {g['step']}): eager {g['eager_us_per_step']} us "
                  f"per step, replayed graph {g['graph_us_per_step']} us per step.", ""]
    lines += ["Per workload: `us` = amortised device time per call (40 calls alternating two "
              "buffer sets, median of 3 runs); `cold` = one call after a read-only 1 GiB pass "
              "(median of 5, an event pair's overhead included); floor = the larger of the HBM "
              "(8 TB/s) and VALU (78.6 TFLOP/s) floors; copy = a device copy of the same bytes, "
              "amortised the same way (problems up to 8 MB); CPU = the oracle's timing build on "
              "all cores (median of 3) and on one thread.", "",
              "| workload | layout | op | kernel | us | cold us | floor us (bound) | "
              "floor / us | GB/s | % of 8 TB/s | copy us | CPU us (threads) | CPU 1-thread us |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in d.get("per_config", []):
        cpu = (f"{r['cpu_us']:,.1f} ({r.get('cpu_threads')})" if "cpu_us" in r else "")
        lines.append(f"| {r['workload']} | {r['layout']} | {r['op']} | `{r['kernel']}` | "
                     f"{r['us']} | {r['cold_us']} | {r['floor_us']} ({r['bound']}) | "
                     f"{r['frac_of_bound']} | {r['GBs']} | {r['pct_hbm_peak']} | "
                     f"{r.get('copy_same_bytes_us', '')} | {cpu} | "
                     f"{r.get('cpu_us_1thread', '')} |")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text


SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVE_CYCLES",
               "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU")


def sq_table(csv_path, detail_path, out_path=None):
    """Instruction counters per workload row from a rocprofv3 --pmc run of
    `bench.py --table-only` (the SQ_COUNTERS) and that run's detail file.
    Per row, medians over the row's dispatches (the weight gradient: its
    partial-sum kernel): VALU, LDS and SALU instructions per wave, the FMA
    wave-instructions the op needs per wave (flops / 2 / 64) against the
    VALU ones, the VALU issue time of the whole launch at one wave64 FMA per
    4 cycles on each of 1024 SIMDs at 2.4 GHz, and the share of wave cycles
    spent waiting to issue (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, both in
    quad-cycles).  No GPU needed."""
    import csv
    import depthwise_convolution_amd as dw
    from depthwise_convolution_amd import workloads
    by_id = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            did = int(r["Dispatch_Id"])
            e = by_id.setdefault(did, [r["Kernel_Name"], int(r.get("Grid_Size", "0") or 0), {}])
            e[2][r["Counter_Name"]] = float(r["Counter_Value"])
    seq = [tuple(by_id[k]) for k in sorted(by_id)]
    order = _table_order(detail_path)
    lines = ["| workload | layout | op | kernel | waves | VALU / wave | FMA / wave | FMA share | "
             "VALU issue us | LDS / wave | SALU / wave | waiting to issue |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for (wl, layout, op), (kname, _, vals) in zip(order, _assign_rows(dw, order, seq)):
        if not vals or any(c not in vals[0] for c in SQ_COUNTERS):
            continue
        med = {c: statistics.median(v[c] for v in vals) for c in SQ_COUNTERS}
        waves = med["SQ_WAVES"]
        valu = med["SQ_INSTS_VALU"] / waves
        fma = op_flops(wl, op) / 2 / 64 / waves
        issue_us = med["SQ_INSTS_VALU"] * 4 / 1024 / 2.4e3
        lines.append(f"| {wl.name} | {workloads.LAYOUT_NAMES[layout]} | {op} | `{kname}` | "
                     f"{waves:.0f} | {valu:.0f} | {fma:.0f} | {fma / valu:.2f} | {issue_us:.2f} | "
                     f"{med['SQ_INSTS_LDS'] / waves:.0f} | {med['SQ_INSTS_SALU'] / waves:.0f} | "
                     f"{med['SQ_WAIT_INST_ANY'] / med['SQ_WAVE_CYCLES']:.2f} |")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text


def headline_trace(csv_path, detail_path, out_path=None):
    """The headline kernels in a rocprofv3 kernel trace of the default
    `bench.py` run: per-dispatch statistics of the forward and input-gradient
    kernels against the bench's amortised figure from the same run, and the
    kernels with the most device time.  No GPU needed."""
    import depthwise_convolution_amd as dw
    from depthwise_convolution_amd import workloads
    with open(detail_path) as f:
        d = json.load(f)
    roof = d.get("headline", {}).get("roofline", {})
    seq = _dispatch_seq(csv_path)
    wl = workloads.WORKLOADS[HEADLINE]
    lines = [f"Bench (same run): dominant kernel `{roof.get('kernel')}`, {roof.get('avg_launch_us')} "
             f"us per launch amortised (40 back-to-back launches over two buffer sets) = "
             f"{roof.get('achieved')} GB/s, frac {roof.get('frac')} of 8 TB/s.", "",
             "| op | kernel | dispatches | mean us | median us | min us | GB/s at the median | "
             "frac of 8 TB/s at the median |", "|---|---|---|---|---|---|---|---|"]
    for op in ("fwd", "ig"):
        kname, match = _row_matcher(dw, wl, workloads.NHWC, op)
        ds = [v for n, g, v in seq if match(n, g)]
        if not ds:
            continue
        med = statistics.median(ds)
        gbs = op_bytes(wl, op) / med / 1e3
        lines.append(f"| {op} | `{kname}` | {len(ds)} | {statistics.mean(ds):.2f} | {med:.2f} | "
                     f"{min(ds):.2f} | {gbs:.1f} | {gbs / PEAK_HBM_GBS:.4f} |")
    tot = {}
    for n, g, v in seq:
        k = (n.replace("(anonymous namespace)::", "").split("(")[0][:90], g)
        t = tot.setdefault(k, [0.0, 0])
        t[0] += v
        t[1] += 1
    lines += ["", "Kernels by total device time in the trace (name, grid in threads):", "",
              "| kernel | grid | calls | total ms | mean us |", "|---|---|---|---|---|"]
    for (n, g), (t, c) in sorted(tot.items(), key=lambda kv: -kv[1][0])[:15]:
        lines.append(f"| `{n}` | {g} | {c} | {t / 1e3:.2f} | {t / c:.2f} |")
    text = "\n".join(lines) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-table", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--table-only", action="store_true",
                    help="only the per-workload table (for a profiler run)")
    ap.add_argument("--workloads", default="",
                    help="comma-separated workload names for the table (default: all)")
    ap.add_argument("--detail",
                    default=os.path.join(tempfile.gettempdir(), "dwconv_bench_detail.json"))
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times (counter calibration)")
    ap.add_argument("--trace-table", default="", help="summarise a kernel-trace CSV and exit")
    ap.add_argument("--counter-table", nargs=2, default=None, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--traffic-json", default="",
                    help="with --counter-table: also write the headline kernel's traffic file")
    ap.add_argument("--detail-table", action="store_true",
                    help="write the detail file's per-workload table as markdown and exit")
    ap.add_argument("--sq-table", default="", help="summarise an SQ counter CSV and exit")
    ap.add_argument("--headline-trace", default="",
                    help="summarise the headline kernels of a kernel-trace CSV and exit")
    ap.add_argument("--out", default="")
    args = ap.parse_args()
    if args.detail_table:
        print(detail_table(args.detail, args.out or None))
        return
    if args.sq_table:
        print(sq_table(args.sq_table, args.detail, args.out or None))
        return
    if args.headline_trace:
        print(headline_trace(args.headline_trace, args.detail, args.out or None))
        return
    if args.trace_table:
        print(trace_table(args.trace_table, args.detail, args.out or None))
        return
    if args.counter_table:
        text, rows, (sf, sw) = counter_table(*args.counter_table, args.detail,
                                             args.out or None)
        print(text)
        if args.traffic_json:
            ops = {op: rows[(HEADLINE, "nhwc", op)] for op in ("fwd", "ig", "wgrad")
                   if (HEADLINE, "nhwc", op) in rows}
            with open(args.traffic_json, "w") as f:
                json.dump({"workload": HEADLINE + " nhwc",
                           "kernel_source_sha256": kernel_source_digest(),
                           "fetch_scale": sf, "write_scale": sw, "ops": ops}, f, indent=1)
        return
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
    detail = {"bench_detail_of": "bench.py", "argv": sys.argv[1:]}
    threads = cpu_threads()
    cpu = None if args.no_cpu else CpuOracle()
    only = [s for s in args.workloads.split(",") if s]
    if args.table_only:
        detail["per_config"] = per_config_table(torch, dw, cpu, threads, only)
        if args.calib_copy:
            calibration_kernels(torch, dw, workloads, detail, workloads.NHWC, torch.cuda.Stream())
        _write_detail(args.detail, detail)
        if cpu:
            cpu.close()
        return

    wl = workloads.WORKLOADS[HEADLINE]
    layout = workloads.NHWC
    _log(f"[bench] generating {HEADLINE} inputs")
    inp = workloads.make_inputs(wl, layout, seed=0)
    t = make_problem(torch, wl, layout, inputs=inp)
    stream = torch.cuda.Stream()

    def step():
        launch(dw, wl, t, layout, "fwd", stream)
        launch(dw, wl, t, layout, "ig", stream)

    # warmup: the requested steps, and at least 100 steps and 50 ms of them
    # (the device takes ~10 ms of steady work before its step time settles)
    _log("[bench] warmup")
    n_warm, t_warm = 0, time.perf_counter()
    while n_warm < args.warmup or n_warm < 100 or time.perf_counter() - t_warm < 0.05:
        with torch.cuda.stream(stream):
            for _ in range(10):
                step()
        n_warm += 10
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
    # per-kernel durations: HIP events on the launch stream around every
    # kernel of 50 more steps (each pair of events adds its own overhead)
    n_ev = min(args.steps, 50)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    with torch.cuda.stream(stream):
        for i in range(n_ev):
            ev[i][0].record(stream)
            launch(dw, wl, t, layout, "fwd", stream)
            ev[i][1].record(stream)
            launch(dw, wl, t, layout, "ig", stream)
            ev[i][2].record(stream)
    torch.cuda.synchronize()
    fwd_avg = statistics.mean(e[0].elapsed_time(e[1]) * 1e3 for e in ev)
    ig_avg = statistics.mean(e[1].elapsed_time(e[2]) * 1e3 for e in ev)

    step_bytes = wl.fwd_bytes() + wl.ig_bytes()
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom = "fwd" if fwd_avg >= ig_avg else "ig"
    dom_bytes = op_bytes(wl, dom)
    # Dominant kernel's launch duration with the event overhead amortised: two
    # events around 40 back-to-back launches that alternate between two
    # disjoint buffer sets (256 MiB in / out each), so no launch finds its
    # input in the 256 MB Infinity Cache.
    alt = {"x": t["dy"], "y": t["dx"], "dy": t["x"], "dx": t["y"]}
    k_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n_rep = 40
    with torch.cuda.stream(stream):
        for i in range(n_rep + 4):
            if i == 4:
                k_ev[0].record(stream)
            launch(dw, wl, t if i % 2 == 0 else dict(t, **alt), layout, dom, stream)
        k_ev[1].record(stream)
    torch.cuda.synchronize()
    dom_us = k_ev[0].elapsed_time(k_ev[1]) * 1e3 / n_rep
    achieved = dom_bytes / dom_us / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(dom), "kernel": describe(dw, wl, dom, layout),
                "avg_launch_us": round(dom_us, 2)}
    result = {
        "metric": "effective HBM bandwidth of depthwise conv2d forward + input-gradient "
                  "(x+y+W+b and dy+dx+W bytes)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic, seeded: x, dy ~ N(0,1); W ~ N(0,1/9); b ~ U(-0.1,0.1)",
        "config": {"workload": HEADLINE, "N": wl.N, "H": wl.H, "W": wl.W, "C": wl.C,
                   "kernel": f"{wl.kH}x{wl.kW}", "layout": "nhwc", "weights": "f32"},
        "fwd_us": round(fwd_avg, 2), "ig_us": round(ig_avg, 2),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    detail["headline"] = {"warmup_steps_run": n_warm, "fwd_us_events_each_launch":
                          round(fwd_avg, 2), "ig_us_events_each_launch": round(ig_avg, 2),
                          "dominant": dom, "algorithmic_bytes_per_launch": dom_bytes,
                          "roofline": roofline}
    _log(f"[bench] headline {json.dumps(result)}")
    detail["headline_extras"] = headline_extras(torch, dw, wl, t, layout, stream, n_rep)
    best = max(detail["headline_extras"]["ceilings"]["runtime_copy_GBs"],
               detail["headline_extras"]["ceilings"]["elementwise_copy_GBs"])
    detail["headline_extras"]["ceilings"]["headline_frac_of_best_copy"] = round(achieved / best, 3)
    del t
    torch.cuda.empty_cache()
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    detail["launch_floor"] = launch_floor(torch, stream, flush, sink)
    del flush
    detail["graph"] = graph_leg(torch, dw)
    _log(f"[bench] floor {json.dumps(detail['launch_floor'])} graph {json.dumps(detail['graph'])}")
    if args.calib_copy:
        calibration_kernels(torch, dw, workloads, detail, layout, stream)
    if cpu is not None:
        _log("[bench] cpu baseline (oracle timing build)")
        cb = cpu_baseline(cpu, wl, inp, threads)
        detail["cpu_baseline"] = cb
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    del inp
    if not args.no_table:
        _log("[bench] per-workload table")
        detail["per_config"] = per_config_table(torch, dw, cpu, threads, only)
    if cpu is not None:
        cpu.close()
    detail["result"] = result
    _write_detail(args.detail, detail)
    print(json.dumps(result), flush=True)


def _write_detail(path, detail):
    if not path:
        return
    d = os.path.dirname(os.path.abspath(path))
    os.makedirs(d, exist_ok=True)
    with open(path, "w") as f:
        json.dump(detail, f, indent=1)
    _log(f"[bench] detail written to {path}")


if __name__ == "__main__":
    main()
