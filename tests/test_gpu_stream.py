"""GPU parity of the row-streaming kernels (strategy STREAM, both layouts).

Shapes with ragged channel tiles (a prime channel count; NHWC tail tiles of
16 and 32 channels per lane group, alone and after full tiles), images narrower
and shorter than a wave's columns and rows, a single row or column, planes
wider than 64 lane groups, SAME / asymmetric / cropping pads, dilation 1 and
2 (the phase split), forward, input gradient and the fused BatchNorm + ReLU6
forward, f32 and f16 weights.  Integer inputs must equal the oracle bit for
bit (every partial sum is exact); random inputs must lie within
1e-5*S + 1e-6 of it (S: the element's sum of |products|).
"""
import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, NCHW

pytestmark = pytest.mark.gpu
LNAME = {NHWC: "nhwc", NCHW: "nchw"}
SHAPES = [(2, 13, 19, 131), (1, 30, 19, 128), (3, 7, 5, 64), (1, 1, 24, 40), (2, 9, 1, 70),
          (1, 9, 150, 3), (1, 70, 9, 2), (2, 11, 23, 91), (1, 5, 47, 24)]
PADS = ["same", (0, 3, 2, 1), (-1, 2, 0, 0)]


def _stream_shapes(layout):
    out = []
    for k, d in ((7, 1), (7, 2), (5, 1), (3, 1)):
        try:
            dw.dwconv2d_describe(dw.OP_FWD, 1, 30, 19, 64, k, k, 1, d, layout,
                                 strategy=dw.STRATEGY_STREAM)
            out.append((k, d))
        except dw.DwconvError:
            pass
    return out


CASES = [(l, k, d, shp, pads, op) for l in (NHWC, NCHW) for (k, d) in _stream_shapes(l)
         for shp in SHAPES for pads in PADS for op in ("fwd", "ig")]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _cid(c):
    l, k, d, shp, pads, op = c
    return f"{LNAME[l]}-{k}x{k}d{d}-{'x'.join(map(str, shp))}-{pads}-{op}"


def _pads(pads, H, W, k, d):
    return tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, H, W, k, k, 1, d)) if pads == "same" else pads


@pytest.mark.parametrize("layout,k,d,shape,pads,op", CASES, ids=[_cid(c) for c in CASES])
def test_stream_matches_oracle(torch, oracle_mod, layout, k, d, shape, pads, op):
    N, H, W, C = shape
    pads = _pads(pads, H, W, k, d)
    try:
        dw.dwconv2d_out_extents(H, W, k, k, 1, d, pads)
    except dw.DwconvError:
        pytest.skip("no output position with these pads")
    wl = wlmod.Workload(name="stream", N=N, H=H, W=W, C=C, kH=k, kW=k, dilation=d, pads=pads,
                        x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    name = dw.dwconv2d_describe_ex(dw.OP_FWD if op == "fwd" else dw.OP_INPUT_GRAD, N, H, W, C,
                                   k, k, 1, d, pads, 1, layout, 0, op == "fwd",
                                   dw.STRATEGY_STREAM)[0]
    print(f"\n[case] {_cid((layout, k, d, shape, pads, op))} kernel={name}", flush=True)
    assert name.startswith("stream_")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    for integer in (True, False):
        inp = wlmod.make_inputs(wl, layout, seed=k + d, integer=integer)
        if op == "fwd":
            ref, S = oracle_mod.fwd_general(inp["x"], inp["w"], inp["b"], 1, d, pads, 1, layout)
            got = dw.fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), 1, d, layout,
                         dw.STRATEGY_STREAM, pads=pads)
        else:
            ref, S = oracle_mod.input_grad_general(inp["dy"], inp["w"], H, W, 1, d, pads, 1,
                                                   layout)
            got = dw.input_grad(dev(inp["dy"]), dev(inp["w"]), H, W, 1, d, layout,
                                dw.STRATEGY_STREAM, pads=pads)
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        if integer:
            np.testing.assert_array_equal(g, ref.astype(np.float32))
        else:
            err = np.abs(g.astype(np.float64) - ref)
            assert np.all(err <= 1e-5 * S + 1e-6), f"max err/bound {np.max(err / (1e-5 * S + 1e-6))}"


WG_CASES = [(l, k, d, shp, pads) for l in (NHWC, NCHW) for (k, d) in ((7, 1), (7, 2))
            for shp in SHAPES + [(2, 40, 33, 5)] for pads in PADS]


@pytest.mark.parametrize("layout,k,d,shape,pads", WG_CASES,
                         ids=[_cid((l, k, d, shp, pads, "wgrad")) for l, k, d, shp, pads in WG_CASES])
def test_stream_weight_grad_matches_oracle(torch, oracle_mod, layout, k, d, shape, pads):
    """The row-streaming weight and bias gradients: integer inputs bit for
    bit, random inputs within the bound (NCHW: the lane sums of each plane
    added in a fixed tree order; NHWC: the four waves of a workgroup added
    in wave order; the chunks by the fixed-order reduction)."""
    N, H, W, C = shape
    pads = _pads(pads, H, W, k, d)
    try:
        dw.dwconv2d_out_extents(H, W, k, k, 1, d, pads)
    except dw.DwconvError:
        pytest.skip("no output position with these pads")
    name = dw.dwconv2d_describe_ex(dw.OP_WEIGHT_GRAD, N, H, W, C, k, k, 1, d, pads, 1, layout, 0,
                                   False, dw.STRATEGY_STREAM)[0]
    print(f"\n[case] wgrad {LNAME[layout]} {k}x{k} d{d} {shape} {pads} kernel={name}", flush=True)
    assert name.startswith("wgrad_stream_" + LNAME[layout])
    wl = wlmod.Workload(name="streamwg", N=N, H=H, W=W, C=C, kH=k, kW=k, dilation=d, pads=pads,
                        x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    for integer in (True, False):
        inp = wlmod.make_inputs(wl, layout, seed=k + d, integer=integer)
        rW, SW = oracle_mod.weight_grad_general(inp["x"], inp["dy"], k, k, 1, d, pads, 1, layout)
        rb, Sb = oracle_mod.bias_grad(inp["dy"], layout)
        gW, gb = dw.weight_grad(dev(inp["x"]), dev(inp["dy"]), k, k, 1, d, layout,
                                strategy=dw.STRATEGY_STREAM, pads=pads)
        torch.cuda.synchronize()
        gW, gb = gW.cpu().numpy(), gb.cpu().numpy()
        if integer:
            np.testing.assert_array_equal(gW, rW.astype(np.float32))
            np.testing.assert_array_equal(gb, rb.astype(np.float32))
        else:
            assert np.all(np.abs(gW.astype(np.float64) - rW) <= 1e-5 * SW + 1e-6)
            assert np.all(np.abs(gb.astype(np.float64) - rb) <= 1e-5 * Sb + 1e-6)


@pytest.mark.parametrize("layout", [NHWC, NCHW])
@pytest.mark.parametrize("kd", [(7, 1), (7, 2)])
def test_stream_f16_weights_and_epilogue(torch, oracle_mod, layout, kd):
    """f16 weights equal f32 weights holding the same values bit for bit;
    the fused BatchNorm + ReLU6 forward equals the oracle's convolution
    followed by the textbook layer (bit-exact on integer inputs with
    gamma = 1, var + eps = 1, integer mean and beta)."""
    k, d = kd
    N, H, W, C = 2, 13, 19, 131
    wl = wlmod.Workload(name="stream16", N=N, H=H, W=W, C=C, kH=k, kW=k, dilation=d,
                        x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    if not _stream_shapes(layout) or (k, d) not in _stream_shapes(layout):
        pytest.skip("no streaming kernel for this shape")
    print(f"\n[case] stream f16/epilogue {LNAME[layout]} {k}x{k} d{d}", flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    inp = wlmod.make_inputs(wl, layout, seed=3)
    w16 = inp["w"].astype(np.float16)
    w16.flat[0] = np.float16(2.0 ** -24)
    st = dw.STRATEGY_STREAM
    for op in ("fwd", "ig"):
        if op == "fwd":
            a = dw.fwd(dev(inp["x"]), dev(w16), dev(inp["b"]), 1, d, layout, st)
            b = dw.fwd(dev(inp["x"]), dev(w16.astype(np.float32)), dev(inp["b"]), 1, d, layout, st)
        else:
            a = dw.input_grad(dev(inp["dy"]), dev(w16), H, W, 1, d, layout, st)
            b = dw.input_grad(dev(inp["dy"]), dev(w16.astype(np.float32)), H, W, 1, d, layout, st)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    ii = wlmod.make_inputs(wl, layout, seed=4, integer=True)
    rng = np.random.default_rng(9)
    gamma = np.ones(C, np.float32)
    beta = rng.integers(-2, 3, C).astype(np.float32)
    mean = rng.integers(-2, 3, C).astype(np.float32)
    var = np.full(C, 0.75, np.float32)              # var + eps = 1 exactly
    bn = (gamma, beta, mean, var)
    y = dw.fwd_bn_act(dev(ii["x"]), dev(ii["w"]), dev(ii["b"]), tuple(dev(v) for v in bn), 0.25,
                      dw.ACT_RELU6, 1, d, layout, st)
    z, _ = oracle_mod.fwd(ii["x"], ii["w"], ii["b"], 1, d, layout)
    ref, _ = oracle_mod.batchnorm_act(z, bn, 0.25, oracle_mod.ACT_RELU6, layout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("C", [67, 144, 150])
def test_stream_tail_tiles_full_size(torch, oracle_mod, C):
    """The NHWC walks' tail tile at 64 images (thousands of workgroups, the
    tail's interleaved among the full tiles' under per-XCD ranges): C = 67
    (16 lanes after one full tile), 144 (16 lanes after two, C % 4 == 0) and
    150 (32 lanes).  Forward, input gradient and weight gradient on integer
    inputs, bit for bit against the oracle."""
    N, H, W, k = 64, 30, 19, 7
    wl = wlmod.Workload(name="tailfull", N=N, H=H, W=W, C=C, kH=k, kW=k)
    pads = _pads("same", H, W, k, 1)
    want = "_t16" if C in (67, 144) else "_t32"
    names = [dw.dwconv2d_describe_ex(op, N, H, W, C, k, k, 1, 1, pads, 1, NHWC, 0,
                                     op == dw.OP_FWD, dw.STRATEGY_AUTO)[0]
             for op in (dw.OP_FWD, dw.OP_INPUT_GRAD, dw.OP_WEIGHT_GRAD)]
    print(f"\n[case] tail full size C={C} kernels={names}", flush=True)
    assert all(want in nm for nm in names), names
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    inp = wlmod.make_inputs(wl, NHWC, seed=C, integer=True)
    y = dw.fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), 1, 1, NHWC)
    dx = dw.input_grad(dev(inp["dy"]), dev(inp["w"]), H, W, 1, 1, NHWC)
    gW, gb = dw.weight_grad(dev(inp["x"]), dev(inp["dy"]), k, k, 1, 1, NHWC)
    torch.cuda.synchronize()
    ry, _ = oracle_mod.fwd(inp["x"], inp["w"], inp["b"], 1, 1, NHWC)
    rdx, _ = oracle_mod.input_grad_general(inp["dy"], inp["w"], H, W, 1, 1, pads, 1, NHWC)
    rW, _ = oracle_mod.weight_grad_general(inp["x"], inp["dy"], k, k, 1, 1, pads, 1, NHWC)
    rb, _ = oracle_mod.bias_grad(inp["dy"], NHWC)
    np.testing.assert_array_equal(y.cpu().numpy(), ry.astype(np.float32))
    np.testing.assert_array_equal(dx.cpu().numpy(), rdx.astype(np.float32))
    np.testing.assert_array_equal(gW.cpu().numpy(), rW.astype(np.float32))
    np.testing.assert_array_equal(gb.cpu().numpy(), rb.astype(np.float32))
