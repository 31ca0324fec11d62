"""Channel multipliers on the tiled kernels against the oracle: multiplier 2
on the NHWC forward, input gradient and weight gradient, any multiplier on
the NCHW forward.

With a multiplier m, output channel o reads input channel o/m (Reactant.jl
issue 331: a grouped convolution with groups = input channels; the MLX
conv-transpose weight page for the [C_out][kH][kW] weight layout).  The
tiled kernels walk the output channels: the forward stages each input
channel once and uses it for its m outputs, the input gradient sums the m
output channels of each input channel, the weight gradient pairs every dy
channel with its input channel.  Shapes span several tiles with ragged
tails, partial channel tiles and cropped or asymmetric pads.  Integer inputs
give exact sums, so the results must match the oracle bit for bit; random
inputs are held to |err| <= 1e-5*S + 1e-6.
"""
import os

import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, Workload

pytestmark = pytest.mark.gpu
NTHREADS = max(1, min(16, os.cpu_count() or 1))

# (N, H, W, C, k, pads or None for SAME); the multiplier is 2
SHAPES = [
    (2, 37, 75, 12, 3, None),           # 24 output channels: a partial channel tile
    (1, 56, 56, 64, 5, None),
    (3, 29, 41, 20, 5, (0, 0, 0, 0)),   # VALID
    (1, 130, 18, 32, 3, (-1, 2, 1, 0)), # a cropped top, asymmetric pads
    (1, 23, 300, 8, 3, None),           # wide rows: several column tiles
    (1, 112, 112, 32, 3, None),         # the MobileNet shape with two filters per channel
]
OPS = [dw.OP_FWD, dw.OP_INPUT_GRAD, dw.OP_WEIGHT_GRAD]
OPNAME = {dw.OP_FWD: "fwd", dw.OP_INPUT_GRAD: "ig", dw.OP_WEIGHT_GRAD: "wgrad"}


def _wl(shape):
    N, H, W, C, k, pads = shape
    if pads is None:
        pads = tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, H, W, k, k, 1, 1))
    return Workload(name=f"m2_{N}x{H}x{W}x{C}_k{k}_{pads}", N=N, H=H, W=W, C=C, kH=k, kW=k,
                    pads=pads, mult=2, x_dist="uniform1", w_dist="uniform1",
                    dy_dist="uniform1")


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _dev(t, a):
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _name(wl, op):
    return dw.dwconv2d_describe_ex(op, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, 1, 1, wl.pads, 2,
                                   NHWC, 0, op == dw.OP_FWD, dw.STRATEGY_TILED)[0]


def _oracle(wl, inp, op):
    import oracle
    if op == dw.OP_FWD:
        return oracle.fwd_general(inp["x"], inp["w"], inp["b"], 1, 1, wl.pads, 2, NHWC,
                                  nthreads=NTHREADS)
    if op == dw.OP_INPUT_GRAD:
        return oracle.input_grad_general(inp["dy"], inp["w"], wl.H, wl.W, 1, 1, wl.pads, 2,
                                         NHWC, nthreads=NTHREADS)
    dW, SW = oracle.weight_grad_general(inp["x"], inp["dy"], wl.kH, wl.kW, 1, 1, wl.pads, 2,
                                        NHWC, nthreads=NTHREADS)
    db, Sb = oracle.bias_grad(inp["dy"], NHWC)
    return (dW, db), (SW, Sb)


def _gpu(torch, wl, inp, op, w=None):
    st = dw.STRATEGY_TILED
    w = _dev(torch, inp["w"]) if w is None else w
    if op == dw.OP_FWD:
        out = dw.fwd(_dev(torch, inp["x"]), w, _dev(torch, inp["b"]), 1, 1, NHWC, st,
                     pads=wl.pads, mult=2)
        res = out.cpu().numpy()
    elif op == dw.OP_INPUT_GRAD:
        out = dw.input_grad(_dev(torch, inp["dy"]), w, wl.H, wl.W, 1, 1, NHWC, st,
                            pads=wl.pads, mult=2)
        res = out.cpu().numpy()
    else:
        dW, db = dw.weight_grad(_dev(torch, inp["x"]), _dev(torch, inp["dy"]), wl.kH, wl.kW, 1,
                                1, NHWC, strategy=st, pads=wl.pads, mult=2)
        res = (dW.cpu().numpy(), db.cpu().numpy())
    torch.cuda.synchronize()
    return res


CASES = [(i, o) for i in range(len(SHAPES)) for o in OPS]
IDS = [f"{_wl(SHAPES[i]).name}-{OPNAME[o]}" for i, o in CASES]


def test_plans_are_tiled_m2():
    for shape in SHAPES:
        wl = _wl(shape)
        for op in OPS:
            name = _name(wl, op)
            assert "tiled_nhwc" in name and "_m2_" in name, (wl.name, op, name)


@pytest.mark.parametrize("idx,op", CASES, ids=IDS)
def test_m2_tiled_integer_bit_exact(torch, idx, op):
    wl = _wl(SHAPES[idx])
    print(f"\n[case] m2 int {wl.name} {OPNAME[op]} {_name(wl, op)}", flush=True)
    inp = wlmod.make_inputs(wl, NHWC, seed=90 + idx, integer=True)
    ref, _ = _oracle(wl, inp, op)
    got = _gpu(torch, wl, inp, op)
    if op == dw.OP_WEIGHT_GRAD:
        np.testing.assert_array_equal(got[0], ref[0].astype(np.float32))
        np.testing.assert_array_equal(got[1], ref[1].astype(np.float32))
    else:
        np.testing.assert_array_equal(got, ref.astype(np.float32))
        # fp16 weights carrying the same (integer) values give the same bits
        w16 = _dev(torch, inp["w"].astype(np.float16))
        np.testing.assert_array_equal(_gpu(torch, wl, inp, op, w=w16), got)


def _within(got, ref, S, what):
    err = np.abs(got.astype(np.float64) - ref)
    bound = 1e-5 * S + 1e-6
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), f"{what}: worst err/bound {np.max(err / bound):.3g}"


@pytest.mark.parametrize("idx,op", CASES, ids=IDS)
def test_m2_tiled_random_within_bound(torch, idx, op):
    wl = _wl(SHAPES[idx])
    print(f"\n[case] m2 rand {wl.name} {OPNAME[op]}", flush=True)
    inp = wlmod.make_inputs(wl, NHWC, seed=110 + idx)
    ref, S = _oracle(wl, inp, op)
    got = _gpu(torch, wl, inp, op)
    if op == dw.OP_WEIGHT_GRAD:
        _within(got[0], ref[0], S[0], f"{wl.name} dW")
        _within(got[1], ref[1], S[1], f"{wl.name} db")
    else:
        _within(got, ref, S, wl.name)


# NCHW: the tiled forward takes any multiplier (output plane n*mC + o reads
# input plane n*C + o/m); the tiled input gradient takes a multiplier of 2
# (dx plane n*C + c sums dy planes (n*C + c)*2 + j), others run direct.
NCHW_SHAPES = [
    (2, 37, 75, 6, 3, 2, None),
    (1, 56, 56, 16, 5, 3, (0, 0, 0, 0)),
    (3, 30, 19, 5, 7, 2, None),
    (1, 23, 300, 4, 3, 4, (-1, 2, 1, 0)),
    (2, 20, 64, 8, 3, 2, None),            # 16-byte staging
    (1, 40, 64, 8, 5, 2, (1, 2, 2, 1)),
    (1, 30, 19, 4, 7, 2, (0, 0, 0, 0)),
]


def _wl_nchw(shape):
    N, H, W, C, k, m, pads = shape
    if pads is None:
        pads = tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, H, W, k, k, 1, 1))
    return Workload(name=f"nchw_m{m}_{N}x{H}x{W}x{C}_k{k}_{pads}", N=N, H=H, W=W, C=C, kH=k,
                    kW=k, pads=pads, mult=m, x_dist="uniform1", w_dist="uniform1",
                    dy_dist="uniform1")


@pytest.mark.parametrize("idx", range(len(NCHW_SHAPES)),
                         ids=[_wl_nchw(s).name for s in NCHW_SHAPES])
def test_nchw_multiplier_forward_tiled(torch, idx):
    import oracle
    from depthwise_convolution_amd.workloads import NCHW
    wl = _wl_nchw(NCHW_SHAPES[idx])
    name = dw.dwconv2d_describe_ex(dw.OP_FWD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, 1, 1,
                                   wl.pads, wl.mult, NCHW, 0, True, dw.STRATEGY_TILED)[0]
    print(f"\n[case] nchw fwd {wl.name} {name}", flush=True)
    assert name.startswith("tiled_nchw") and f"_m{wl.mult}_" in name
    for integer, seed in ((True, 130 + idx), (False, 140 + idx)):
        inp = wlmod.make_inputs(wl, NCHW, seed=seed, integer=integer)
        ref, S = oracle.fwd_general(inp["x"], inp["w"], inp["b"], 1, 1, wl.pads, wl.mult, NCHW,
                                    nthreads=NTHREADS)
        got = dw.fwd(_dev(torch, inp["x"]), _dev(torch, inp["w"]), _dev(torch, inp["b"]), 1, 1,
                     NCHW, dw.STRATEGY_TILED, pads=wl.pads, mult=wl.mult).cpu().numpy()
        torch.cuda.synchronize()
        if integer:
            np.testing.assert_array_equal(got, ref.astype(np.float32))
        else:
            _within(got, ref, S, wl.name)


@pytest.mark.parametrize("idx", [i for i, s in enumerate(NCHW_SHAPES) if s[5] == 2],
                         ids=[_wl_nchw(s).name for s in NCHW_SHAPES if s[5] == 2])
def test_nchw_multiplier2_input_grad_tiled(torch, idx):
    import oracle
    from depthwise_convolution_amd.workloads import NCHW
    wl = _wl_nchw(NCHW_SHAPES[idx])
    name = dw.dwconv2d_describe_ex(dw.OP_INPUT_GRAD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, 1, 1,
                                   wl.pads, 2, NCHW, 0, False, dw.STRATEGY_TILED)[0]
    print(f"\n[case] nchw ig {wl.name} {name}", flush=True)
    assert name.startswith("tiled_nchw") and "_m2_" in name
    for integer, seed in ((True, 150 + idx), (False, 160 + idx)):
        inp = wlmod.make_inputs(wl, NCHW, seed=seed, integer=integer)
        ref, S = oracle.input_grad_general(inp["dy"], inp["w"], wl.H, wl.W, 1, 1, wl.pads, 2,
                                           NCHW, nthreads=NTHREADS)
        got = dw.input_grad(_dev(torch, inp["dy"]), _dev(torch, inp["w"]), wl.H, wl.W, 1, 1,
                            NCHW, dw.STRATEGY_TILED, pads=wl.pads, mult=2).cpu().numpy()
        torch.cuda.synchronize()
        if integer:
            np.testing.assert_array_equal(got, ref.astype(np.float32))
        else:
            _within(got, ref, S, wl.name)
