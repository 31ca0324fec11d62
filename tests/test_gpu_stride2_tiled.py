"""Stride-2 tiled kernels (forward, input gradient, weight gradient) against
the oracle, on shapes that span several tiles with ragged tails in every
direction, odd extents, channel counts with and without whole 16-byte
vectors, SAME, XLA-SAME and other explicit pads.

The forward keeps the even positions of a stride-1 tile grid, the input
gradient stages dy zero-upsampled (the LeanMlir "Depthwise" page: stride 2
as the even decimation of the stride-1 result; the backward through the
upsampled dy), and the weight gradient meets dy position (m, j) with x at
(2m + kh*d - pt, 2j + kw*d - pl).  Integer inputs give exact sums, so the
tiled kernels must match the oracle bit for bit; random inputs are held to
|err| <= 1e-5*S + 1e-6.
"""
import os

import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, NCHW, Workload

pytestmark = pytest.mark.gpu
NTHREADS = max(1, min(16, os.cpu_count() or 1))
LNAME = {NHWC: "nhwc", NCHW: "nchw"}

# (N, H, W, C, k, pads or None for SAME)
SHAPES = [
    (2, 37, 75, 36, 3, None),           # C = 36: partial channel tiles
    (1, 50, 66, 13, 3, (0, 1, 0, 1)),   # XLA-SAME, prime C (4-byte staging)
    (3, 29, 41, 20, 5, None),
    (1, 64, 64, 8, 5, (1, 2, 2, 1)),
    (1, 23, 1100, 4, 3, None),          # wide rows: several NCHW column tiles
    (2, 9, 9, 5, 3, (0, 0, 0, 0)),      # VALID, a single tile
    (1, 130, 18, 32, 3, (-1, 2, 1, 0)), # a cropped top, odd pads
]


def _wl(shape):
    N, H, W, C, k, pads = shape
    return Workload(name=f"s2_{N}x{H}x{W}x{C}_k{k}_{pads}", N=N, H=H, W=W, C=C, kH=k, kW=k,
                    stride=2, pads=pads if pads is not None else
                    tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, H, W, k, k, 2, 1)),
                    x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _dev(t, a):
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _name(wl, layout, op):
    return dw.dwconv2d_describe_ex(op, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, 2, 1, wl.pads, 1,
                                   layout, 0, op == dw.OP_FWD, dw.STRATEGY_TILED)[0]


def _oracle(wl, inp, layout, op):
    import oracle
    if op == dw.OP_FWD:
        return oracle.fwd_general(inp["x"], inp["w"], inp["b"], 2, 1, wl.pads, 1, layout,
                                  nthreads=NTHREADS)
    if op == dw.OP_INPUT_GRAD:
        return oracle.input_grad_general(inp["dy"], inp["w"], wl.H, wl.W, 2, 1, wl.pads, 1,
                                         layout, nthreads=NTHREADS)
    dW, SW = oracle.weight_grad_general(inp["x"], inp["dy"], wl.kH, wl.kW, 2, 1, wl.pads, 1,
                                        layout, nthreads=NTHREADS)
    db, Sb = oracle.bias_grad(inp["dy"], layout)
    return (dW, db), (SW, Sb)


def _gpu(torch, wl, inp, layout, op):
    st = dw.STRATEGY_TILED
    if op == dw.OP_FWD:
        out = dw.fwd(_dev(torch, inp["x"]), _dev(torch, inp["w"]), _dev(torch, inp["b"]), 2, 1,
                     layout, st, pads=wl.pads)
        res = out.cpu().numpy()
    elif op == dw.OP_INPUT_GRAD:
        out = dw.input_grad(_dev(torch, inp["dy"]), _dev(torch, inp["w"]), wl.H, wl.W, 2, 1,
                            layout, st, pads=wl.pads)
        res = out.cpu().numpy()
    else:
        dW, db = dw.weight_grad(_dev(torch, inp["x"]), _dev(torch, inp["dy"]), wl.kH, wl.kW, 2,
                                1, layout, strategy=st, pads=wl.pads)
        res = (dW.cpu().numpy(), db.cpu().numpy())
    torch.cuda.synchronize()
    return res


OPS = [dw.OP_FWD, dw.OP_INPUT_GRAD, dw.OP_WEIGHT_GRAD]
OPNAME = {dw.OP_FWD: "fwd", dw.OP_INPUT_GRAD: "ig", dw.OP_WEIGHT_GRAD: "wgrad"}
CASES = [(i, l, o) for i in range(len(SHAPES)) for l in (NHWC, NCHW) for o in OPS]
IDS = [f"{_wl(SHAPES[i]).name}-{LNAME[l]}-{OPNAME[o]}" for i, l, o in CASES]


def test_plans_are_tiled_stride2():
    for shape in SHAPES:
        wl = _wl(shape)
        for layout in (NHWC, NCHW):
            for op in OPS:
                name = _name(wl, layout, op)
                assert "tiled" in name and "_s2_" in name, (wl.name, layout, op, name)


@pytest.mark.parametrize("idx,layout,op", CASES, ids=IDS)
def test_stride2_tiled_integer_bit_exact(torch, idx, layout, op):
    wl = _wl(SHAPES[idx])
    print(f"\n[case] s2 int {wl.name} {LNAME[layout]} {OPNAME[op]} "
          f"{_name(wl, layout, op)}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=60 + idx, integer=True)
    ref, _ = _oracle(wl, inp, layout, op)
    got = _gpu(torch, wl, inp, layout, op)
    if op == dw.OP_WEIGHT_GRAD:
        np.testing.assert_array_equal(got[0], ref[0].astype(np.float32))
        np.testing.assert_array_equal(got[1], ref[1].astype(np.float32))
    else:
        np.testing.assert_array_equal(got, ref.astype(np.float32))


def _within(got, ref, S, what):
    err = np.abs(got.astype(np.float64) - ref)
    bound = 1e-5 * S + 1e-6
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), f"{what}: worst err/bound {np.max(err / bound):.3g}"


@pytest.mark.parametrize("idx,layout,op", CASES, ids=IDS)
def test_stride2_tiled_random_within_bound(torch, idx, layout, op):
    wl = _wl(SHAPES[idx])
    print(f"\n[case] s2 rand {wl.name} {LNAME[layout]} {OPNAME[op]}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=80 + idx)
    ref, S = _oracle(wl, inp, layout, op)
    got = _gpu(torch, wl, inp, layout, op)
    if op == dw.OP_WEIGHT_GRAD:
        _within(got[0], ref[0], S[0], f"{wl.name} dW")
        _within(got[1], ref[1], S[1], f"{wl.name} db")
    else:
        _within(got, ref, S, wl.name)
