"""GPU parity of the fused epilogues against the CPU oracle.

Forward + inference BatchNorm + activation (one pass): the GPU value is
compared with the oracle's act((z - mean) * gamma / sqrt(var + eps) + beta)
computed in float64 from the oracle's convolution z.  Bound, from the fp32
arithmetic of the kernel: the convolution's own bound e_z = 1e-5*S + 1e-6
(S = sum of |products|) scaled by |inv| = |gamma| / sqrt(var + eps), plus a
relative 2e-6 of |inv*(z - mean)| and of |t| for the roundings of z - mean,
inv (sqrt, divide) and the fused multiply-add; ReLU and ReLU6 are
1-Lipschitz, SiLU's slope is below 1.1 and its exp / divide add a relative
2e-6 of |y|.

SGD step fused into the weight-gradient reduction: w - lr*dW, b - lr*db with
dW, db from the oracle; bound |lr| * (1e-5*S + 1e-6) + 2^-23 * |result| (one
rounding of the fused multiply-add); bit-exact on integer inputs with a
power-of-two learning rate.
"""
import os

import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, NCHW, WORKLOADS

pytestmark = pytest.mark.gpu
LAYOUTS = [NHWC, NCHW]
NTHREADS = max(1, min(16, os.cpu_count() or 1))
ACTS = [dw.ACT_NONE, dw.ACT_RELU, dw.ACT_RELU6, dw.ACT_SILU]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _dev(t, a):
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _bn_params(Co, seed):
    rng = np.random.default_rng(seed)
    gamma = (rng.uniform(0.5, 2.0, Co) * rng.choice([-1, 1], Co)).astype(np.float32)
    beta = rng.uniform(-1, 1, Co).astype(np.float32)
    mean = rng.uniform(-0.5, 0.5, Co).astype(np.float32)
    var = rng.uniform(0.2, 3.0, Co).astype(np.float32)
    return gamma, beta, mean, var


def _conv_ref(wl, inp, layout):
    import oracle
    if wl.general:
        return oracle.fwd_general(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, wl.pads,
                                  wl.mult, layout, nthreads=NTHREADS)
    return oracle.fwd(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, layout,
                      nthreads=NTHREADS)


def _check_epilogue(got, z, S, bn, eps, act, layout, what):
    import oracle
    y, inv = oracle.batchnorm_act(z, bn, eps, act, layout)
    e_z = 1e-5 * S + 1e-6
    if bn is not None:
        inv_c = np.abs(oracle._chan(inv, layout))
        mean_c = oracle._chan(bn[2], layout)
        t, _ = oracle.batchnorm_act(z, bn, eps, dw.ACT_NONE, layout)
        bound = inv_c * e_z + 2e-6 * (inv_c * np.abs(z - mean_c) + np.abs(t)) + 1e-7
    else:
        bound = e_z + 2e-6 * np.abs(z) + 1e-7
    if act == dw.ACT_SILU:
        bound = 1.1 * bound + 2e-6 * np.abs(y)
    assert got.shape == y.shape and np.all(np.isfinite(got)), what
    err = np.abs(got.astype(np.float64) - y)
    if np.any(err > bound):
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        pytest.fail(f"{what}: {int((err > bound).sum())} of {err.size} out of bound; worst {i}: "
                    f"got {got[i]!r} want {y[i]!r} bound {bound[i]:.3g}")


EPI_WL = ["mobilenet_112x112x32_3x3", "mobilenet_s2_224x224x32_3x3", "effnet_n1_56x56x128_5x5",
          "effnet_n1_56x56x128_5x5_f16w", "asr_n1_30x19x128_7x7_d2", "prime_n1_30x19x131_7x7",
          "asr_n1_1x24x256_1x31", "mobilenet_s2_xla_224x224x32_3x3",
          "effnet_n32_56x56x128_5x5_valid", "mobilenet_m2_112x112x32_3x3",
          "reactant_4x4x4_3x3_m2_valid", "large_512x512x256_3x3"]


@pytest.mark.parametrize("wl_name", EPI_WL)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_fwd_bn_act_parity(torch, wl_name, layout):
    """Every activation, with and without BatchNorm, under AUTO and each
    applicable strategy."""
    wl = WORKLOADS[wl_name]
    print(f"\n[case] fwd_bn_act {wl_name} layout={layout}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=31)
    z, S = _conv_ref(wl, inp, layout)
    bn = _bn_params(wl.Co, 7)
    x, w = _dev(torch, inp["x"]), _dev(torch, inp["w"])
    b = None if inp["b"] is None else _dev(torch, inp["b"])
    tbn = tuple(_dev(torch, v) for v in bn)
    strategies = [dw.STRATEGY_AUTO]
    if "large" not in wl.tags:
        strategies += [dw.STRATEGY_DIRECT, dw.STRATEGY_TILED]
    for strategy in strategies:
        for act in ACTS:
            for use_bn in (True, False):
                try:
                    y = dw.fwd_bn_act(x, w, b, tbn if use_bn else None, 1e-3, act, wl.stride,
                                      wl.dilation, layout, strategy, pads=wl.pads, mult=wl.mult)
                except dw.DwconvError as e:
                    assert e.status == -12 and strategy == dw.STRATEGY_TILED
                    continue
                torch.cuda.synchronize()
                _check_epilogue(y.cpu().numpy(), z, S, bn if use_bn else None, 1e-3, act, layout,
                                f"{wl_name} strategy={strategy} act={act} bn={use_bn}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fwd_act_integer_bit_exact(torch, layout):
    """Without BatchNorm, ReLU and ReLU6 of integer convolutions are exact."""
    for name in ("mobilenet_112x112x32_3x3", "effnet_n1_56x56x128_5x5", "prime_n1_30x19x131_7x7"):
        wl = WORKLOADS[name]
        inp = wlmod.make_inputs(wl, layout, seed=32, integer=True)
        z, _ = _conv_ref(wl, inp, layout)
        x, w, b = _dev(torch, inp["x"]), _dev(torch, inp["w"]), _dev(torch, inp["b"])
        for act, want in ((dw.ACT_RELU, np.maximum(z, 0)),
                          (dw.ACT_RELU6, np.minimum(np.maximum(z, 0), 6))):
            y = dw.fwd_bn_act(x, w, b, None, 0.0, act, wl.stride, wl.dilation, layout)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y.cpu().numpy(), want.astype(np.float32))


def test_plain_forward_unchanged_by_epilogue_build(torch):
    """ACT_NONE without BatchNorm gives the plain forward's bits."""
    wl = WORKLOADS["effnet_n32_56x56x128_5x5"]
    for layout in LAYOUTS:
        inp = wlmod.make_inputs(wl, layout, seed=33)
        x, w, b = _dev(torch, inp["x"]), _dev(torch, inp["w"]), _dev(torch, inp["b"])
        y0 = dw.fwd(x, w, b, 1, 1, layout)
        y1 = dw.fwd_bn_act(x, w, b, None, 0.0, dw.ACT_NONE, 1, 1, layout)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


# ------------------------------------------------------------------ fused SGD
SGD_WL = ["mobilenet_112x112x32_3x3", "mobilenet_s2_224x224x32_3x3", "effnet_n32_56x56x128_5x5",
          "prime_n1_30x19x131_7x7", "asr_n64_30x19x128_7x7_d2", "mobilenet_s2_xla_224x224x32_3x3",
          "mobilenet_m2_112x112x32_3x3", "reactant_4x4x4_3x3_m2_valid", "large_512x512x256_3x3"]


def _wgrad_ref(wl, inp, layout):
    import oracle
    if wl.general:
        dW, SW = oracle.weight_grad_general(inp["x"], inp["dy"], wl.kH, wl.kW, wl.stride,
                                            wl.dilation, wl.pads, wl.mult, layout,
                                            nthreads=NTHREADS)
    else:
        dW, SW = oracle.weight_grad(inp["x"], inp["dy"], wl.kH, wl.kW, wl.stride, wl.dilation,
                                    layout, nthreads=NTHREADS)
    db, Sb = oracle.bias_grad(inp["dy"], layout)
    return dW, SW, db, Sb


@pytest.mark.parametrize("wl_name", SGD_WL)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_weight_grad_sgd_parity(torch, wl_name, layout):
    import oracle
    wl = WORKLOADS[wl_name]
    print(f"\n[case] sgd {wl_name} layout={layout}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=34)
    dW, SW, db, Sb = _wgrad_ref(wl, inp, layout)
    lr = 0.01
    w0 = inp["w"].astype(np.float32)
    b0 = inp["b"]
    w_new, b_new = oracle.sgd_step(w0, b0, dW, db, lr)
    x, g = _dev(torch, inp["x"]), _dev(torch, inp["dy"])
    for strategy in (dw.STRATEGY_AUTO, dw.STRATEGY_DIRECT):
        w, b = _dev(torch, w0), _dev(torch, b0)
        gW = torch.full(w.shape, float("nan"), device="cuda")
        gb = torch.full(b.shape, float("nan"), device="cuda")
        n = dw.dwconv2d_weight_grad_workspace_size_ex(wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                                      wl.stride, wl.dilation, wl.pads, wl.mult,
                                                      layout, strategy)
        ws = torch.empty((n + 15) // 16 * 4 + 4, device="cuda")
        dw.dwconv2d_weight_grad_sgd_ex(x, g, w, b, lr, ws, gW, gb, wl.stride, wl.dilation,
                                       wl.pads, wl.mult, layout, strategy)
        torch.cuda.synchronize()
        for got, ref, bound, what in (
                (w, w_new, lr * (1e-5 * SW + 1e-6) + 2.0 ** -23 * np.abs(w_new), "w"),
                (b, b_new, lr * (1e-5 * Sb + 1e-6) + 2.0 ** -23 * np.abs(b_new), "b"),
                (gW, dW, 1e-5 * SW + 1e-6, "dW"), (gb, db, 1e-5 * Sb + 1e-6, "db")):
            err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
            assert np.all(err <= bound), f"{wl_name} {what} strategy={strategy}: max err " \
                                         f"{err.max():.3g}"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_weight_grad_sgd_integer_bit_exact_and_optional_outputs(torch, layout):
    """Integer inputs and lr = 1/4: the step is exact.  Without b only w moves;
    without dw / db no gradient is written."""
    import oracle
    wl = WORKLOADS["effnet_n1_56x56x128_5x5"]
    inp = wlmod.make_inputs(wl, layout, seed=35, integer=True)
    dW, _, db, _ = _wgrad_ref(wl, inp, layout)
    w_new, b_new = oracle.sgd_step(inp["w"], inp["b"], dW, db, 0.25)
    x, g = _dev(torch, inp["x"]), _dev(torch, inp["dy"])
    w, b = _dev(torch, inp["w"]), _dev(torch, inp["b"])
    dw.weight_grad_sgd(x, g, w, b, 0.25, 1, 1, layout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.cpu().numpy(), w_new.astype(np.float32))
    np.testing.assert_array_equal(b.cpu().numpy(), b_new.astype(np.float32))
    w2 = _dev(torch, inp["w"])
    dw.weight_grad_sgd(x, g, w2, None, 0.25, 1, 1, layout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w2.cpu().numpy(), w_new.astype(np.float32))
