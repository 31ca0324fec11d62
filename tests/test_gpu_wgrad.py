"""GPU parity of the weight and bias gradients against the CPU oracle.

dW[c,kh,kw] = sum over batch and output positions of x * dy (LeanMlir
"Depthwise" weight-VJP); db[c] = sum of dy (bias-gradient closed form).
Acceptance: |gpu - oracle| <= 1e-5*S + 1e-6 per element, S = sum of |terms|;
bit-exact on integer inputs; bitwise repeatable.
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


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _dev(t, a):
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _ref(wl, inp, layout):
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


def _gpu(torch, wl, inp, layout, strategy=dw.STRATEGY_AUTO):
    x, g = _dev(torch, inp["x"]), _dev(torch, inp["dy"])
    dW, db = dw.weight_grad(x, g, wl.kH, wl.kW, wl.stride, wl.dilation, layout,
                            strategy=strategy, pads=wl.pads, mult=wl.mult)
    torch.cuda.synchronize()
    return dW.cpu().numpy(), db.cpu().numpy()


def _has_strategy(wl, layout, strategy):
    try:
        if wl.general:
            dw.dwconv2d_describe_ex(dw.OP_WEIGHT_GRAD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                    wl.stride, wl.dilation, wl.pads, wl.mult, layout, 0, False,
                                    strategy)
        else:
            dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                 wl.stride, wl.dilation, layout, 0, False, strategy)
    except dw.DwconvError as e:
        assert e.status == -12
        return False
    return True


def _check(got, ref, S, what):
    err = np.abs(got.astype(np.float64) - ref)
    bound = 1e-5 * S + 1e-6
    assert np.all(np.isfinite(got)), what
    if np.any(err > bound):
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        pytest.fail(f"{what}: {int((err > bound).sum())} out of bound; worst {i}: "
                    f"got {got[i]!r} want {ref[i]!r} bound {bound[i]:.3g}")


WG_CASES = [(n, l) for n, w in WORKLOADS.items() for l in LAYOUTS if not w.fp16_weights]


@pytest.mark.parametrize("wl_name,layout", WG_CASES,
                         ids=[f"{n}-{'nhwc' if l == NHWC else 'nchw'}" for n, l in WG_CASES])
def test_weight_grad_full_size(torch, wl_name, layout):
    wl = WORKLOADS[wl_name]
    print(f"\n[case] wgrad {wl_name} layout={layout}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=3)
    dW, SW, db, Sb = _ref(wl, inp, layout)
    gW, gb = _gpu(torch, wl, inp, layout)
    _check(gW, dW, SW, f"{wl_name} dW")
    _check(gb, db, Sb, f"{wl_name} db")


@pytest.mark.parametrize("wl_name", ["tiny_16x16x8_3x3", "mobilenet_112x112x32_3x3",
                                     "mobilenet_s2_224x224x32_3x3", "effnet_n1_56x56x128_5x5",
                                     "asr_n1_30x19x128_7x7_d2", "asr_n1_1x24x256_1x31",
                                     "prime_n1_30x19x131_7x7", "mobilenet_s2_xla_224x224x32_3x3",
                                     "effnet_n32_56x56x128_5x5_valid",
                                     "mobilenet_m2_112x112x32_3x3", "reactant_4x4x4_3x3_m2_valid",
                                     "asr_n64_30x19x128_7x7", "prime_n64_30x19x131_7x7",
                                     "asr_n64_30x19x128_7x7_d2"])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("strategy", [dw.STRATEGY_DIRECT, dw.STRATEGY_TILED,
                                      dw.STRATEGY_STREAM])
def test_weight_grad_integer_bit_exact(torch, wl_name, layout, strategy):
    wl = WORKLOADS[wl_name]
    if not _has_strategy(wl, layout, strategy):
        pytest.skip("no kernel of this strategy for the problem")
    print(f"\n[case] wgrad int {wl_name} layout={layout} strategy={strategy}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=4, integer=True)
    dW, _, db, _ = _ref(wl, inp, layout)
    gW, gb = _gpu(torch, wl, inp, layout, strategy)
    np.testing.assert_array_equal(gW, dW.astype(np.float32))
    np.testing.assert_array_equal(gb, db.astype(np.float32))


def test_weight_grad_deterministic_and_workspace_contents_irrelevant(torch):
    wl = WORKLOADS["effnet_n32_56x56x128_5x5"]
    inp = wlmod.make_inputs(wl, NHWC, seed=5)
    x, g = _dev(torch, inp["x"]), _dev(torch, inp["dy"])
    n = dw.dwconv2d_weight_grad_workspace_size(wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW)
    outs = []
    for fill in (0.0, float("nan"), 1e30):
        ws = torch.full(((n + 15) // 16 * 4 + 64,), fill, device="cuda")
        dW = torch.full((wl.C, wl.kH, wl.kW), 7.0, device="cuda")
        db = torch.full((wl.C,), 7.0, device="cuda")
        dw.dwconv2d_weight_grad(x, g, dW, db, ws[:(n + 15) // 16 * 4])
        torch.cuda.synchronize()
        assert torch.all(ws[(n + 15) // 16 * 4:] == fill) or (fill != fill)
        outs.append((dW.cpu().numpy(), db.cpu().numpy()))
    for o in outs[1:]:
        np.testing.assert_array_equal(o[0], outs[0][0])
        np.testing.assert_array_equal(o[1], outs[0][1])


def test_weight_grad_without_bias_and_small_workspace(torch):
    wl = WORKLOADS["mobilenet_112x112x32_3x3"]
    inp = wlmod.make_inputs(wl, NHWC, seed=6)
    x, g = _dev(torch, inp["x"]), _dev(torch, inp["dy"])
    dW, db = dw.weight_grad(x, g, 3, 3, with_bias=False)
    assert db is None
    ref, S, _, _ = _ref(wl, inp, NHWC)
    _check(dW.cpu().numpy(), ref, S, "no-bias dW")
    ws = torch.empty(4, device="cuda")
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_weight_grad(x, g, dW, None, ws)
    assert e.value.status == -13


RANDOM = [wlmod.random_problem(np.random.default_rng(100 + i), max_hw=20, max_c=40)
          for i in range(20)]


@pytest.mark.parametrize("idx", range(len(RANDOM)))
@pytest.mark.parametrize("layout", LAYOUTS)
def test_weight_grad_random_shapes(torch, idx, layout):
    wl = RANDOM[idx]
    print(f"\n[case] wgrad {wl}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=idx)
    dW, SW, db, Sb = _ref(wl, inp, layout)
    for strategy in (dw.STRATEGY_AUTO, dw.STRATEGY_DIRECT):
        gW, gb = _gpu(torch, wl, inp, layout, strategy)
        _check(gW, dW, SW, f"dW {wl}")
        _check(gb, db, Sb, f"db {wl}")


def _general_cases():
    from tests.test_gpu_parity import _random_general_cases
    return _random_general_cases(count=24, seed=777)


GENERAL = _general_cases()


@pytest.mark.parametrize("idx", range(len(GENERAL)))
@pytest.mark.parametrize("layout", LAYOUTS)
def test_weight_grad_padded_and_multiplier_shapes(torch, idx, layout):
    wl = GENERAL[idx]
    print(f"\n[case] wgrad {wl}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=200 + idx)
    dW, SW, db, Sb = _ref(wl, inp, layout)
    for strategy in (dw.STRATEGY_AUTO, dw.STRATEGY_DIRECT, dw.STRATEGY_TILED,
                     dw.STRATEGY_STREAM):
        if not _has_strategy(wl, layout, strategy):
            continue
        gW, gb = _gpu(torch, wl, inp, layout, strategy)
        _check(gW, dW, SW, f"dW {wl} strategy={strategy}")
        _check(gb, db, Sb, f"db {wl} strategy={strategy}")
