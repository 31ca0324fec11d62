"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Acceptance: every element within |gpu - oracle| <= 1e-5*S + 1e-6, S being the
element's sum of |products| (the bound of the fp32 accumulation); bit-exact on
integer-valued inputs, where every partial sum is exact in fp32.  Workloads run
at their full sizes in the launch configuration the bench times (strategy
AUTO), compared element by element.
"""
import functools
import os

import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, NCHW, WORKLOADS, to_layout, from_layout

pytestmark = pytest.mark.gpu
LAYOUTS = [NHWC, NCHW]
LNAME = {NHWC: "nhwc", NCHW: "nchw"}
NTHREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _dev(t, a):
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


@functools.lru_cache(maxsize=4)
def _oracle_case(wl_name, layout, op, integer=False, seed=0):
    import oracle
    wl = WORKLOADS[wl_name]
    inp = wlmod.make_inputs(wl, layout, seed=seed, integer=integer)
    return (inp,) + _oracle(wl, inp, layout, op)


def _oracle(wl, inp, layout, op):
    """Oracle result and magnitude sums (SAME routines, or the general ones
    for explicit pads / a channel multiplier)."""
    import oracle
    if wl.general:
        if op == dw.OP_FWD:
            return oracle.fwd_general(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation,
                                      wl.pads, wl.mult, layout, nthreads=NTHREADS)
        return oracle.input_grad_general(inp["dy"], inp["w"], wl.H, wl.W, wl.stride,
                                         wl.dilation, wl.pads, wl.mult, layout,
                                         nthreads=NTHREADS)
    if op == dw.OP_FWD:
        return oracle.fwd(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, layout,
                          nthreads=NTHREADS)
    return oracle.input_grad(inp["dy"], inp["w"], wl.H, wl.W, wl.stride, wl.dilation, layout,
                             nthreads=NTHREADS)


def _run_gpu(torch, wl, inp, layout, op, strategy=dw.STRATEGY_AUTO):
    w = _dev(torch, inp["w"])
    if op == dw.OP_FWD:
        x = _dev(torch, inp["x"])
        b = None if inp["b"] is None else _dev(torch, inp["b"])
        out = dw.fwd(x, w, b, wl.stride, wl.dilation, layout, strategy, pads=wl.pads,
                     mult=wl.mult)
    else:
        dy = _dev(torch, inp["dy"])
        out = dw.input_grad(dy, w, wl.H, wl.W, wl.stride, wl.dilation, layout, strategy,
                            pads=wl.pads, mult=wl.mult)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _assert_within_bound(got, ref, S, what):
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref)
    bound = 1e-5 * S + 1e-6
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        pytest.fail(f"{what}: {int(bad.sum())} of {err.size} elements out of bound; worst at "
                    f"{i}: got {got[i]!r} want {ref[i]!r} bound {bound[i]:.3g}")


def _case_id(wl_name, layout, op):
    return f"{wl_name}-{LNAME[layout]}-{'fwd' if op == dw.OP_FWD else 'ig'}"


FULL_CASES = [(n, l, o) for n in WORKLOADS for l in LAYOUTS for o in (dw.OP_FWD, dw.OP_INPUT_GRAD)]


@pytest.mark.parametrize("wl_name,layout,op", FULL_CASES,
                         ids=[_case_id(*c) for c in FULL_CASES])
def test_workload_parity_full_size(torch, wl_name, layout, op):
    """Every workload at full size, AUTO strategy, element by element."""
    wl = WORKLOADS[wl_name]
    print(f"\n[case] {_case_id(wl_name, layout, op)} N={wl.N} H={wl.H} W={wl.W} C={wl.C} "
          f"k={wl.kH}x{wl.kW} s={wl.stride} d={wl.dilation}", flush=True)
    inp, ref, S = _oracle_case(wl_name, layout, op)
    got = _run_gpu(torch, wl, inp, layout, op)
    _assert_within_bound(got, ref, S, _case_id(wl_name, layout, op))


# Workloads small enough to run under every strategy.
STRAT_WL = [n for n, w in WORKLOADS.items() if "large" not in w.tags]
STRAT_CASES = [(n, l, o, s) for n in STRAT_WL for l in LAYOUTS
               for o in (dw.OP_FWD, dw.OP_INPUT_GRAD)
               for s in (dw.STRATEGY_DIRECT, dw.STRATEGY_TILED, dw.STRATEGY_STREAM)]
SNAME = {dw.STRATEGY_AUTO: "auto", dw.STRATEGY_DIRECT: "direct", dw.STRATEGY_TILED: "tiled",
         dw.STRATEGY_STREAM: "stream"}


@pytest.mark.parametrize("wl_name,layout,op,strategy", STRAT_CASES,
                         ids=[_case_id(*c[:3]) + "-" + SNAME[c[3]] for c in STRAT_CASES])
def test_workload_parity_each_strategy(torch, wl_name, layout, op, strategy):
    wl = WORKLOADS[wl_name]
    name, _, _ = _describe(wl, layout, op, strategy)
    if name is None:
        pytest.skip("no kernel of this strategy for the problem")
    print(f"\n[case] {_case_id(wl_name, layout, op)} kernel={name}", flush=True)
    inp, ref, S = _oracle_case(wl_name, layout, op)
    got = _run_gpu(torch, wl, inp, layout, op, strategy)
    _assert_within_bound(got, ref, S, f"{_case_id(wl_name, layout, op)} {name}")


def _describe(wl, layout, op, strategy, wtype=None):
    wt = wtype if wtype is not None else int(wl.fp16_weights)
    try:
        if wl.general:
            return dw.dwconv2d_describe_ex(op, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride,
                                           wl.dilation, wl.pads, wl.mult, layout, wt,
                                           op == dw.OP_FWD and wl.bias, strategy)
        return dw.dwconv2d_describe(op, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride,
                                    wl.dilation, layout, wt, op == dw.OP_FWD and wl.bias,
                                    strategy)
    except dw.DwconvError as e:
        if e.status == -12:
            return None, None, None
        raise


INT_WL = ["tiny_16x16x8_3x3", "mobilenet_112x112x32_3x3", "mobilenet_s2_224x224x32_3x3",
          "effnet_n1_56x56x128_5x5", "asr_n1_30x19x128_7x7_d2", "asr_n1_1x24x256_1x31",
          "prime_n1_30x19x131_7x7", "large_512x512x256_3x3",
          "mobilenet_s2_xla_224x224x32_3x3", "effnet_n32_56x56x128_5x5_valid",
          "mobilenet_m2_112x112x32_3x3", "reactant_4x4x4_3x3_m2_valid"]
INT_CASES = [(n, l, o, s) for n in INT_WL for l in LAYOUTS for o in (dw.OP_FWD, dw.OP_INPUT_GRAD)
             for s in (dw.STRATEGY_AUTO, dw.STRATEGY_DIRECT)]
INT_CASES += [(n, l, o, dw.STRATEGY_STREAM)
              for n in ("asr_n64_30x19x128_7x7", "asr_n64_30x19x128_7x7_d2",
                        "prime_n64_30x19x131_7x7", "asr_n1_30x19x128_7x7_d2")
              for l in LAYOUTS for o in (dw.OP_FWD, dw.OP_INPUT_GRAD)]


@pytest.mark.parametrize("wl_name,layout,op,strategy", INT_CASES,
                         ids=[_case_id(*c[:3]) + "-" + SNAME[c[3]] for c in INT_CASES])
def test_integer_inputs_bit_exact(torch, wl_name, layout, op, strategy):
    """Integer inputs: every partial sum is exact, so any summation order must
    give the oracle's value bit for bit."""
    wl = WORKLOADS[wl_name]
    if wl.fp16_weights:
        pytest.skip("integer weights are drawn as fp32")
    if _describe(wl, layout, op, strategy)[0] is None:
        pytest.skip("no kernel of this strategy for the problem")
    print(f"\n[case] int {_case_id(wl_name, layout, op)} strategy={strategy}", flush=True)
    inp, ref, _ = _oracle_case(wl_name, layout, op, integer=True)
    got = _run_gpu(torch, wl, inp, layout, op, strategy)
    np.testing.assert_array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("wl_name", ["effnet_n1_56x56x128_5x5_f16w", "effnet_n32_56x56x128_5x5_f16w",
                                     "asr_n1_30x19x128_7x7", "mobilenet_s2_224x224x32_3x3",
                                     "prime_n1_30x19x131_7x7"])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("op", [dw.OP_FWD, dw.OP_INPUT_GRAD])
def test_f16_weights_bitwise_equal_f32_weights(torch, wl_name, layout, op):
    """fp16 weights widen exactly: the f16-weight run equals the f32-weight run
    on the same (fp16-representable) values bit for bit (ggml PR review check)."""
    wl = WORKLOADS[wl_name]
    print(f"\n[case] f16w {_case_id(wl_name, layout, op)}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=1)
    w16 = inp["w"].astype(np.float16)
    w16.flat[0] = np.float16(2.0 ** -24)          # a subnormal weight
    a = dict(inp, w=w16)
    b = dict(inp, w=w16.astype(np.float32))
    ga = _run_gpu(torch, wl, a, layout, op)
    gb = _run_gpu(torch, wl, b, layout, op)
    np.testing.assert_array_equal(ga, gb)


@pytest.mark.parametrize("wl_name", ["large_512x512x256_3x3", "effnet_n32_56x56x128_5x5",
                                     "mobilenet_112x112x32_3x3", "asr_n64_30x19x128_7x7",
                                     "asr_n64_30x19x128_7x7_d2", "prime_n64_30x19x131_7x7"])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_deterministic_and_no_stray_writes(torch, wl_name, layout):
    """Two runs give identical bits; guard bands around the output stay
    untouched and every output element is written."""
    wl = WORKLOADS[wl_name]
    print(f"\n[case] determinism {wl_name} {LNAME[layout]}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=2)
    x, w = _dev(torch, inp["x"]), _dev(torch, inp["w"])
    b = _dev(torch, inp["b"])
    dy = _dev(torch, inp["dy"])
    for op in (dw.OP_FWD, dw.OP_INPUT_GRAD):
        if op == dw.OP_FWD:
            shape = (wl.N, wl.Ho, wl.Wo, wl.C) if layout == NHWC else (wl.N, wl.C, wl.Ho, wl.Wo)
        else:
            shape = (wl.N, wl.H, wl.W, wl.C) if layout == NHWC else (wl.N, wl.C, wl.H, wl.W)
        n = int(np.prod(shape))
        guard = 4096
        results = []
        for rep in range(2):
            buf = torch.full((n + 2 * guard,), float("nan"), device="cuda")
            buf[:guard] = 1234.5
            buf[guard + n:] = -4321.5
            out = buf[guard:guard + n].view(shape)
            if op == dw.OP_FWD:
                dw.dwconv2d_fwd(x, w, b, out, wl.stride, wl.dilation, layout)
            else:
                dw.dwconv2d_input_grad(dy, w, out, wl.stride, wl.dilation, layout)
            torch.cuda.synchronize()
            h = buf.cpu().numpy()
            assert np.all(h[:guard] == 1234.5) and np.all(h[guard + n:] == -4321.5)
            assert not np.isnan(h[guard:guard + n]).any(), "output element not written"
            results.append(h[guard:guard + n].copy())
        np.testing.assert_array_equal(results[0], results[1])


def _random_cases(count=40, seed=1234):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        p = wlmod.random_problem(rng, max_hw=24, max_c=40)
        out.append(p)
    # hand-picked degenerate shapes
    W_ = wlmod.Workload
    U = dict(x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    out += [
        W_("one_pixel", 1, 1, 1, 4, 3, 3, **U), W_("w1", 2, 9, 1, 8, 3, 3, **U),
        W_("h1", 1, 1, 33, 20, 1, 15, **U), W_("k_gt_img", 1, 3, 4, 16, 7, 7, **U),
        W_("c1", 1, 10, 10, 1, 5, 5, **U), W_("c3_s2", 1, 7, 9, 3, 3, 3, stride=2, **U),
        W_("d3", 1, 12, 13, 16, 3, 3, dilation=3, **U), W_("d2_s2", 2, 11, 10, 20, 5, 5, stride=2, dilation=2, **U),
        W_("ragged_c", 1, 17, 37, 68, 3, 3, **U), W_("ragged_c2", 1, 5, 70, 132, 5, 5, **U),
        W_("tall", 1, 200, 3, 16, 3, 3, **U), W_("wide", 1, 3, 300, 16, 3, 3, **U),
        W_("k1", 1, 5, 6, 12, 1, 1, **U), W_("k7x1", 1, 20, 5, 8, 7, 1, **U),
        W_("f16w", 2, 13, 11, 24, 5, 5, fp16_weights=True, **U),
    ]
    return out


RANDOM = _random_cases()


@pytest.mark.parametrize("idx", range(len(RANDOM)), ids=[f"r{i}-{p.name}" for i, p in enumerate(RANDOM)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_random_and_degenerate_shapes(torch, idx, layout):
    import oracle
    wl = RANDOM[idx]
    print(f"\n[case] {wl}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=idx)
    ref_f, S_f = oracle.fwd(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, layout)
    ref_g, S_g = oracle.input_grad(inp["dy"], inp["w"], wl.H, wl.W, wl.stride, wl.dilation, layout)
    for strategy in (dw.STRATEGY_AUTO, dw.STRATEGY_DIRECT, dw.STRATEGY_TILED):
        for op, ref, S in ((dw.OP_FWD, ref_f, S_f), (dw.OP_INPUT_GRAD, ref_g, S_g)):
            name, _, _ = _describe(wl, layout, op, strategy)
            if name is None:
                continue
            got = _run_gpu(torch, wl, inp, layout, op, strategy)
            _assert_within_bound(got, ref, S, f"{wl.name} op={op} {name}")


def test_invalid_arguments_raise_and_leave_output(torch):
    x = torch.randn(1, 8, 8, 4, device="cuda")
    w = torch.randn(4, 2, 2, device="cuda")          # even kernel
    y = torch.full((1, 8, 8, 4), 7.0, device="cuda")
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_fwd(x, w, None, y)
    assert e.value.status == -5
    w3 = torch.randn(4, 3, 3, device="cuda")
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_fwd(x, w3, None, x.view(1, 8, 8, 4))  # in-place
    assert e.value.status == -8
    y3 = torch.full((1, 3, 3, 4), 7.0, device="cuda")
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_launch(dw.OP_FWD, x, w3, None, y3, 8, 8, 3, 1, NHWC)
    assert e.value.status == -3
    assert torch.all(y3 == 7.0)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_runs_on_a_side_stream(torch):
    import oracle
    wl = WORKLOADS["mobilenet_112x112x32_3x3"]
    inp = wlmod.make_inputs(wl, NHWC, seed=5)
    ref, S = oracle.fwd(inp["x"], inp["w"], inp["b"], 1, 1, NHWC)
    s = torch.cuda.Stream()
    x, w, b = _dev(torch, inp["x"]), _dev(torch, inp["w"]), _dev(torch, inp["b"])
    y = torch.empty_like(x)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dw.dwconv2d_fwd(x, w, b, y)
    s.synchronize()
    _assert_within_bound(y.cpu().numpy(), ref, S, "side stream")


# ----------------------------------------------------------------------------
# Explicit padding (negative = crop), even kernels, channel multipliers, at
# random small shapes under every strategy (stride-1 tiled kernels run any
# pads; multipliers run the direct kernels)
# ----------------------------------------------------------------------------
def _random_general_cases(count=36, seed=4321):
    rng = np.random.default_rng(seed)
    U = dict(x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")
    out = []
    while len(out) < count:
        kh, kw = (int(v) for v in rng.choice([1, 2, 3, 4, 5, 7], 2))
        if len(out) % 3 == 0:       # a kernel shape with tiled variants
            kh, kw = [(3, 3), (5, 5), (7, 7), (1, 15)][len(out) % 4]
        s, d = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        if (kh, kw) == (1, 15) or (kh, kw) == (5, 5):
            d = 1
        H, W = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        pads = tuple(int(v) for v in rng.integers(-1, 2 * d * max(kh, kw) // 2 + 2, 4))
        m = int(rng.choice([1, 1, 2, 3]))
        C = int(rng.choice([4, 8, 12, 16, 20, 36, 3, 7]))
        wl = wlmod.Workload(f"g{len(out)}", int(rng.integers(1, 3)), H, W, C, kh, kw, stride=s,
                            dilation=d, pads=pads, mult=m, **U)
        if wl.Ho < 1 or wl.Wo < 1:
            continue
        out.append(wl)
    return out


GENERAL = _random_general_cases()


@pytest.mark.parametrize("idx", range(len(GENERAL)),
                         ids=[f"{p.name}-k{p.kH}x{p.kW}-s{p.stride}-d{p.dilation}-m{p.mult}-"
                              f"p{'_'.join(map(str, p.pads))}" for p in GENERAL])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_random_padded_and_multiplier_shapes(torch, idx, layout):
    wl = GENERAL[idx]
    print(f"\n[case] {wl}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=100 + idx)
    for op in (dw.OP_FWD, dw.OP_INPUT_GRAD):
        ref, S = _oracle(wl, inp, layout, op)
        for strategy in (dw.STRATEGY_AUTO, dw.STRATEGY_DIRECT, dw.STRATEGY_TILED):
            name, _, _ = _describe(wl, layout, op, strategy)
            if name is None:
                continue
            got = _run_gpu(torch, wl, inp, layout, op, strategy)
            _assert_within_bound(got, ref, S, f"{wl.name} op={op} {name}")


def test_xla_same_matches_odd_positions_of_stride1(torch):
    """On the GPU too: the XLA-SAME stride-2 forward equals the stride-1 SAME
    forward kept at the odd positions, bit for bit on integer inputs."""
    wl = WORKLOADS["mobilenet_s2_xla_224x224x32_3x3"]
    for layout in LAYOUTS:
        inp = wlmod.make_inputs(wl, layout, seed=9, integer=True)
        x, w, b = _dev(torch, inp["x"]), _dev(torch, inp["w"]), _dev(torch, inp["b"])
        pads = dw.dwconv2d_same_pads(dw.PAD_XLA_SAME, wl.H, wl.W, wl.kH, wl.kW, 2)
        assert pads == wl.pads
        y2 = dw.fwd(x, w, b, 2, 1, layout, pads=pads)
        y1 = dw.fwd(x, w, b, 1, 1, layout)
        torch.cuda.synchronize()
        a, c = from_layout(y2.cpu().numpy(), layout), from_layout(y1.cpu().numpy(), layout)
        np.testing.assert_array_equal(a, c[:, 1::2, 1::2])
