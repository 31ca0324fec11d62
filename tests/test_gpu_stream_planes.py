"""GPU parity of the plane-per-lane NCHW kernel (strategy STREAM_PLANES).

One plane per lane, 64 planes per workgroup, input rows and output rows
transposed through LDS.  Shapes: a plane count that is not a multiple of 64
(and fewer than 64 planes), planes wider than one 20-column block (several
column blocks, a ragged last one), images shorter than a row tile, a single
row or column, SAME / asymmetric / cropping pads, dilation 1 and 2 (the
phase split), forward and input gradient, the fused BatchNorm + ReLU6
forward, f32 and f16 weights, and the 64-image workloads at full size.
Integer inputs must equal the oracle bit for bit (every partial sum is
exact); random inputs must lie within 1e-5*S + 1e-6 of it (S: the
element's sum of |products|).
"""
import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NCHW

pytestmark = pytest.mark.gpu
SHAPES = [(2, 13, 19, 131), (1, 30, 19, 128), (3, 7, 5, 64), (1, 1, 24, 40), (2, 9, 1, 70),
          (1, 9, 150, 3), (1, 70, 9, 2), (2, 11, 23, 91), (1, 5, 47, 24), (1, 4, 41, 65)]
PADS = ["same", (0, 3, 2, 1), (-1, 2, 0, 0)]
CASES = [(k, d, shp, pads, op) for (k, d) in ((7, 1), (7, 2)) for shp in SHAPES
         for pads in PADS for op in ("fwd", "ig")]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _cid(c):
    k, d, shp, pads, op = c
    return f"{k}x{k}d{d}-{'x'.join(map(str, shp))}-{pads}-{op}"


def _pads(pads, H, W, k, d):
    return tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, H, W, k, k, 1, d)) if pads == "same" else pads


def _run(torch, oracle_mod, k, d, shape, pads, op, integer_only=False):
    N, H, W, C = shape
    wl = wlmod.Workload(name="planes", N=N, H=H, W=W, C=C, kH=k, kW=k, dilation=d, pads=pads,
                        x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    name = dw.dwconv2d_describe_ex(dw.OP_FWD if op == "fwd" else dw.OP_INPUT_GRAD, N, H, W, C,
                                   k, k, 1, d, pads, 1, NCHW, 0, op == "fwd",
                                   dw.STRATEGY_STREAM_PLANES)[0]
    print(f"\n[case] {_cid((k, d, shape, pads, op))} kernel={name}", flush=True)
    assert name.startswith("stream_nchw_planes_")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    for integer in ((True,) if integer_only else (True, False)):
        inp = wlmod.make_inputs(wl, NCHW, seed=k + d, integer=integer)
        if op == "fwd":
            ref, S = oracle_mod.fwd_general(inp["x"], inp["w"], inp["b"], 1, d, pads, 1, NCHW)
            got = dw.fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), 1, d, NCHW,
                         dw.STRATEGY_STREAM_PLANES, pads=pads)
        else:
            ref, S = oracle_mod.input_grad_general(inp["dy"], inp["w"], H, W, 1, d, pads, 1,
                                                   NCHW)
            got = dw.input_grad(dev(inp["dy"]), dev(inp["w"]), H, W, 1, d, NCHW,
                                dw.STRATEGY_STREAM_PLANES, pads=pads)
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        if integer:
            np.testing.assert_array_equal(g, ref.astype(np.float32))
        else:
            err = np.abs(g.astype(np.float64) - ref)
            assert np.all(err <= 1e-5 * S + 1e-6), f"max err/bound {np.max(err / (1e-5 * S + 1e-6))}"


@pytest.mark.parametrize("k,d,shape,pads,op", CASES, ids=[_cid(c) for c in CASES])
def test_planes_matches_oracle(torch, oracle_mod, k, d, shape, pads, op):
    N, H, W, C = shape
    pads = _pads(pads, H, W, k, d)
    try:
        dw.dwconv2d_out_extents(H, W, k, k, 1, d, pads)
    except dw.DwconvError:
        pytest.skip("no output position with these pads")
    _run(torch, oracle_mod, k, d, shape, pads, op)


FULL = [(k, d, shp, op) for (k, d) in ((7, 1), (7, 2)) for shp in ((64, 30, 19, 128),
                                                                  (64, 30, 19, 131))
        for op in ("fwd", "ig")]


@pytest.mark.parametrize("k,d,shape,op", FULL, ids=[_cid((k, d, s, "same", o)) for k, d, s, o in FULL])
def test_planes_full_size(torch, oracle_mod, k, d, shape, op):
    """The 64-image workloads (thousands of waves under per-XCD ranges),
    integer inputs, every element bit for bit; AUTO takes this kernel there
    at dilation 2 (at dilation 1 it keeps the lane-along-columns kernel)."""
    N, H, W, C = shape
    pads = _pads("same", H, W, k, d)
    auto = dw.dwconv2d_describe_ex(dw.OP_FWD if op == "fwd" else dw.OP_INPUT_GRAD, N, H, W, C,
                                   k, k, 1, d, pads, 1, NCHW, 0, op == "fwd",
                                   dw.STRATEGY_AUTO)[0]
    assert auto.startswith("stream_nchw_planes_" if d == 2 else "stream_nchw_s1_"), auto
    _run(torch, oracle_mod, k, d, shape, pads, op, integer_only=True)


@pytest.mark.parametrize("kd", [(7, 1), (7, 2)])
def test_planes_f16_weights_and_epilogue(torch, oracle_mod, kd):
    """f16 weights equal f32 weights holding the same values bit for bit;
    the fused BatchNorm + ReLU6 forward equals the oracle's convolution
    followed by the textbook layer (bit-exact on integer inputs with
    gamma = 1, var + eps = 1, integer mean and beta)."""
    k, d = kd
    N, H, W, C = 2, 13, 19, 131
    wl = wlmod.Workload(name="planes16", N=N, H=H, W=W, C=C, kH=k, kW=k, dilation=d,
                        x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    print(f"\n[case] planes f16/epilogue {k}x{k} d{d}", flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    inp = wlmod.make_inputs(wl, NCHW, seed=3)
    w16 = inp["w"].astype(np.float16)
    w16.flat[0] = np.float16(2.0 ** -24)
    st = dw.STRATEGY_STREAM_PLANES
    for op in ("fwd", "ig"):
        if op == "fwd":
            a = dw.fwd(dev(inp["x"]), dev(w16), dev(inp["b"]), 1, d, NCHW, st)
            b = dw.fwd(dev(inp["x"]), dev(w16.astype(np.float32)), dev(inp["b"]), 1, d, NCHW, st)
        else:
            a = dw.input_grad(dev(inp["dy"]), dev(w16), H, W, 1, d, NCHW, st)
            b = dw.input_grad(dev(inp["dy"]), dev(w16.astype(np.float32)), H, W, 1, d, NCHW, st)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    ii = wlmod.make_inputs(wl, NCHW, seed=4, integer=True)
    rng = np.random.default_rng(9)
    gamma = np.ones(C, np.float32)
    beta = rng.integers(-2, 3, C).astype(np.float32)
    mean = rng.integers(-2, 3, C).astype(np.float32)
    var = np.full(C, 0.75, np.float32)              # var + eps = 1 exactly
    bn = (gamma, beta, mean, var)
    y = dw.fwd_bn_act(dev(ii["x"]), dev(ii["w"]), dev(ii["b"]), tuple(dev(v) for v in bn), 0.25,
                      dw.ACT_RELU6, 1, d, NCHW, st)
    z, _ = oracle_mod.fwd(ii["x"], ii["w"], ii["b"], 1, d, NCHW)
    ref, _ = oracle_mod.batchnorm_act(z, bn, 0.25, oracle_mod.ACT_RELU6, NCHW)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), ref.astype(np.float32))
