"""HIP graph capture of a training step through the C ABI.

A forward, input gradient, weight gradient and the fused-SGD weight gradient
are captured once into a graph (the library enqueues kernels only: no
allocation, no memset, no host synchronisation) and replayed several times,
with eager library calls and device synchronisations between the replays.
Every replay must reproduce the eager results bit for bit (same kernels,
same fixed-order reductions).
"""
import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, NCHW, WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _dev(t, a):
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("wl_name", ["mobilenet_112x112x32_3x3", "mobilenet_s2_xla_224x224x32_3x3",
                                     "asr_n64_30x19x128_7x7", "mobilenet_m2_112x112x32_3x3"])
@pytest.mark.parametrize("layout", [NHWC, NCHW])
def test_graph_replays_match_eager(torch, wl_name, layout):
    wl = WORKLOADS[wl_name]
    print(f"\n[case] graph {wl_name} layout={layout}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=41)
    x, w, b, dy = (_dev(torch, inp[k]) for k in ("x", "w", "b", "dy"))
    stream = torch.cuda.Stream()
    pads = wl.pads if wl.pads is not None else dw.dwconv2d_same_pads(
        dw.PAD_SAME, wl.H, wl.W, wl.kH, wl.kW, wl.stride, wl.dilation)
    y = torch.empty_like(dy)
    dx = torch.empty_like(x)
    dW = torch.empty((wl.Co, wl.kH, wl.kW), device="cuda")
    db = torch.empty((wl.Co,), device="cuda")
    nws = dw.dwconv2d_weight_grad_workspace_size_ex(wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                                    wl.stride, wl.dilation, pads, wl.mult, layout)
    ws = torch.empty((nws + 15) // 16 * 4 + 4, device="cuda")
    w_sgd = w.clone()

    def step(s):
        dw.dwconv2d_launch_ex(dw.OP_FWD, x, w, b, y, wl.H, wl.W, wl.stride, wl.dilation, pads,
                              wl.mult, layout, dw.STRATEGY_AUTO, s)
        dw.dwconv2d_launch_ex(dw.OP_INPUT_GRAD, dy, w, None, dx, wl.H, wl.W, wl.stride,
                              wl.dilation, pads, wl.mult, layout, dw.STRATEGY_AUTO, s)
        dw.dwconv2d_weight_grad_ex(x, dy, dW, db, ws, wl.stride, wl.dilation, pads, wl.mult,
                                   layout, dw.STRATEGY_AUTO, s)

    # eager reference
    with torch.cuda.stream(stream):
        step(stream)
    stream.synchronize()
    ref = [t.clone() for t in (y, dx, dW, db)]

    # capture, then replay with eager work and synchronisations in between
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            step(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        for t_ in (y, dx, dW, db):
            t_.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((y, dx, dW, db), ref, ("y", "dx", "dW", "db")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from eager"
        # eager library work between replays (the SGD step on a copy of W)
        with torch.cuda.stream(stream):
            dw.dwconv2d_weight_grad_sgd_ex(x, dy, w_sgd, None, 1e-3, ws, None, None, wl.stride,
                                           wl.dilation, pads, wl.mult, layout,
                                           dw.STRATEGY_AUTO, stream)
        stream.synchronize()


def test_graph_of_many_small_launches(torch):
    """Launch-bound case: 20 forward launches of a 16x16x8 problem captured
    once; each replay equals the eager result."""
    wl = WORKLOADS["tiny_16x16x8_3x3"]
    inp = wlmod.make_inputs(wl, NHWC, seed=42)
    x, w, b = (_dev(torch, inp[k]) for k in ("x", "w", "b"))
    outs = [torch.empty_like(x) for _ in range(20)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for o in outs:
            dw.dwconv2d_fwd(x, w, b, o, 1, 1, NHWC, stream)
    stream.synchronize()
    ref = outs[0].clone()
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for o in outs:
                dw.dwconv2d_fwd(x, w, b, o, 1, 1, NHWC, stream)
    torch.cuda.synchronize()
    for _ in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o, ref)
