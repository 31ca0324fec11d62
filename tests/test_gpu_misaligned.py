"""GPU parity for tensors that are not 16-byte aligned.

The C ABI asks for 4-byte aligned float arrays only; the planner takes the
kernels with 16-byte loads and stores (and the 8-byte stores of the NCHW
tiles) only when the addresses allow them.  Every tensor here is a
contiguous view at a storage offset of 1, 2 or 3 floats, so the launches
run the 4-byte staging variants, the 1-channel direct kernels and the
scalar or 8-byte NCHW stores; each result is compared with the oracle
element by element at 1e-5*S + 1e-6 (S: the element's sum of |products|).
"""
import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, NCHW

pytestmark = pytest.mark.gpu
LNAME = {NHWC: "nhwc", NCHW: "nchw"}
STRATS = {"auto": dw.STRATEGY_AUTO, "direct": dw.STRATEGY_DIRECT, "tiled": dw.STRATEGY_TILED,
          "stream": dw.STRATEGY_STREAM, "planes": dw.STRATEGY_STREAM_PLANES}
# (kH, kW, dilation); N=2, H=19, W=20 spans several tiles with a ragged tail,
# C=36 fills a 16-byte-staged NHWC channel tile when aligned, W % 4 == 0 gives
# the NCHW 16-byte rows when aligned
KERNELS = [(3, 3, 1), (5, 5, 1), (7, 7, 1), (7, 7, 2)]
N, H, W, C = 2, 19, 20, 36


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _at_offset(torch, a, off):
    """A contiguous GPU tensor holding `a`, starting `off` floats past a
    16-byte boundary."""
    a = np.ascontiguousarray(a)
    buf = torch.zeros(a.size + 8, dtype=torch.float32, device="cuda")
    assert buf.data_ptr() % 16 == 0
    t = buf[off:off + a.size].view(a.shape)
    t.copy_(torch.from_numpy(a))
    assert t.data_ptr() % 16 == 4 * off and t.is_contiguous()
    return t


def _empty_at_offset(torch, shape, off):
    return _at_offset(torch, np.full(shape, np.nan, np.float32), off)


def _check(got, ref, S, what):
    got = got.cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, what
    err = np.abs(got - ref)
    bound = 1e-5 * S + 1e-6
    assert np.all(np.isfinite(got)) and np.all(err <= bound), \
        f"{what}: max err/bound {np.max(err / bound):.3g}"


CASES = [(l, k, op, s, off) for l in (NHWC, NCHW) for k in KERNELS
         for op in ("fwd", "ig", "wgrad") for s in STRATS for off in (1, 2, 3)]


def _cid(c):
    l, k, op, s, off = c
    return f"{LNAME[l]}-{k[0]}x{k[1]}d{k[2]}-{op}-{s}-off{off}"


@pytest.mark.parametrize("layout,k,op,strat,off", CASES, ids=[_cid(c) for c in CASES])
def test_misaligned_views_match_oracle(torch, oracle_mod, layout, k, op, strat, off):
    kH, kW, d = k
    wl = wlmod.Workload(name="misaligned", N=N, H=H, W=W, C=C, kH=kH, kW=kW, dilation=d,
                        x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    inp = wlmod.make_inputs(wl, layout, seed=off)
    what = _cid((layout, k, op, strat, off))
    st = STRATS[strat]
    # every float array at the same offset; the weights too
    w = _at_offset(torch, inp["w"], off)
    try:
        name = dw.dwconv2d_describe_addr_ex(
            {"fwd": dw.OP_FWD, "ig": dw.OP_INPUT_GRAD, "wgrad": dw.OP_WEIGHT_GRAD}[op],
            N, H, W, C, kH, kW, dilation=d, layout=layout, has_bias=op == "fwd", strategy=st,
            addr_bits=4 * off)[0]
    except dw.DwconvError as e:
        if e.status == -12 and strat in ("stream", "planes"):
            pytest.skip("no streaming kernel for this problem")
        raise
    print(f"\n[case] {what} kernel={name}", flush=True)
    # 4-byte loads and stores only (the streaming kernels use no other)
    assert "_v4" not in name and ("_l1" in name or "_v1" in name or "direct" in name or
                                  "stream_" in name), name
    if op == "fwd":
        x = _at_offset(torch, inp["x"], off)
        b = _at_offset(torch, inp["b"], off)
        y = _empty_at_offset(torch, inp["dy"].shape, off)
        dw.dwconv2d_launch(dw.OP_FWD, x, w, b, y, H, W, 1, d, layout, st)
        ref, S = oracle_mod.fwd(inp["x"], inp["w"], inp["b"], 1, d, layout)
        torch.cuda.synchronize()
        _check(y, ref, S, what)
    elif op == "ig":
        dy = _at_offset(torch, inp["dy"], off)
        dx = _empty_at_offset(torch, inp["x"].shape, off)
        dw.dwconv2d_launch(dw.OP_INPUT_GRAD, dy, w, None, dx, H, W, 1, d, layout, st)
        ref, S = oracle_mod.input_grad(inp["dy"], inp["w"], H, W, 1, d, layout)
        torch.cuda.synchronize()
        _check(dx, ref, S, what)
    else:
        x = _at_offset(torch, inp["x"], off)
        dy = _at_offset(torch, inp["dy"], off)
        dW = _empty_at_offset(torch, (C, kH, kW), off)
        db = _empty_at_offset(torch, (C,), off)
        nws = dw.dwconv2d_weight_grad_workspace_size(N, H, W, C, kH, kW, 1, d, layout, st)
        ws = torch.empty((nws + 15) // 16 * 4 + 4, dtype=torch.float32, device="cuda")
        dw.dwconv2d_weight_grad(x, dy, dW, db, ws, 1, d, layout, st)
        rW, SW = oracle_mod.weight_grad(inp["x"], inp["dy"], kH, kW, 1, d, layout)
        rb, Sb = oracle_mod.bias_grad(inp["dy"], layout)
        torch.cuda.synchronize()
        _check(dW, rW, SW, what + " dW")
        _check(db, rb, Sb, what + " db")


@pytest.mark.parametrize("layout", [NHWC, NCHW])
@pytest.mark.parametrize("which", ["in", "out", "bias", "bn"])
def test_one_misaligned_array(torch, oracle_mod, layout, which):
    """Only one array off a 16-byte boundary (the input, the output, the bias
    or the BatchNorm arrays): the plan still avoids 16-byte accesses, and the
    fused forward matches the oracle's convolution + BatchNorm + ReLU6."""
    wl = wlmod.Workload(name="misaligned1", N=N, H=H, W=W, C=C, kH=3, kW=3,
                        x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    inp = wlmod.make_inputs(wl, layout, seed=11)
    rng = np.random.default_rng(5)
    bn = [rng.uniform(0.5, 2, C), rng.uniform(-1, 1, C), rng.uniform(-0.5, 0.5, C),
          rng.uniform(0.2, 3, C)]
    bn = [a.astype(np.float32) for a in bn]
    off = {k: (1 if k == which else 0) for k in ("in", "out", "bias", "bn")}
    x = _at_offset(torch, inp["x"], off["in"])
    y = _empty_at_offset(torch, inp["dy"].shape, off["out"])
    b = _at_offset(torch, inp["b"], off["bias"])
    bnt = tuple(_at_offset(torch, a, off["bn"]) for a in bn)
    w = _at_offset(torch, inp["w"], 0)
    print(f"\n[case] {LNAME[layout]} misaligned {which}", flush=True)
    dw.dwconv2d_fwd_bn_act_ex(x, w, b, y, bnt, 1e-3, dw.ACT_RELU6, 1, 1, None, 1, layout)
    z, S = oracle_mod.fwd(inp["x"], inp["w"], inp["b"], 1, 1, layout)
    ref, inv = oracle_mod.batchnorm_act(z, bn, 1e-3, oracle_mod.ACT_RELU6, layout)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    # the convolution's bound scaled by |inv| = |gamma|/sqrt(var+eps), plus a
    # relative 2e-6 of |inv*(z - mean)| and of |t| for the roundings of the
    # affine step (ReLU6 only clamps, which shrinks any error)
    inv_c = np.abs(oracle_mod._chan(inv, layout))
    mean_c = oracle_mod._chan(bn[2], layout)
    t = (z - mean_c) * oracle_mod._chan(inv, layout) + oracle_mod._chan(bn[1], layout)
    bound = inv_c * (1e-5 * S + 1e-6) + 2e-6 * (inv_c * np.abs(z - mean_c) + np.abs(t)) + 1e-7
    assert np.all(np.abs(got - ref) <= bound), f"max err/bound {np.max(np.abs(got - ref) / bound):.3g}"
