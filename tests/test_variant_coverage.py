"""Every compiled tiled-kernel variant can be chosen by the planner, and every
(variant, op, multiplier) the planner chooses is checked against the oracle.

The variant tables of csrc/dwconv_internal.h are parsed and each entry's plan
name prefix is derived from its fields (the names `dwconv2d_describe_ex`
reports).  A sweep of small problems (kernel shapes, strides, dilations,
multipliers, channel counts with and without whole 16-byte vectors, image
shapes, both layouts, all three ops) through the describe call (host only)
finds, for every (variant, op, multiplier) that can run, the first problem
that runs it.

* CPU: every table entry is reached by at least one op (a variant no problem
  can select would be compiled for nothing);
* GPU: each (variant, op, multiplier) runs its problem under its strategy
  on integer inputs, where every summation order is exact, and must
  equal the oracle bit for bit.
"""
import os
import re

import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import Workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "depthwise_convolution_amd", "csrc", "dwconv_internal.h")
NTHREADS = max(1, min(16, os.cpu_count() or 1))


def _table(src, name, nfields):
    body = src[src.index(name + "[] = {"):]
    body = body[:body.index("};")]
    pat = r"\{" + r",\s*".join([r"(-?\d+|kNever)"] * nfields) + r"\}"
    return [tuple(-1 if v == "kNever" else int(v) for v in m.groups())
            for m in re.finditer(pat, body)]


def _expected_prefixes():
    """{plan-name prefix: table} for every entry of every tiled variant table."""
    src = open(HEADER).read()
    out = {}

    def nhwc(v, s, m2, wg):
        kh, kw, d, vec, cl, px, g, lv = v
        return (f"{'wgrad_' if wg else ''}tiled_nhwc_s{s}_k{kh}x{kw}_d{d}_v{vec}_cl{cl}_px{px}"
                f"_g{g}{'_l1' if lv == 1 else ''}{'_m2' if m2 else ''}_")

    def nchw(v, s, wg):
        kh, kw, d, q, g, v4 = v
        return (f"{'wgrad_' if wg else ''}tiled_nchw_s{s}_k{kh}x{kw}_d{d}_q{q}_g{g}_"
                f"{'v4' if v4 else 'v1'}_tx")

    for name, s, m2, wg in (("kTiledVariants", 1, False, False),
                            ("kTiledS2Variants", 2, False, False),
                            ("kTiledM2Variants", 1, True, False),
                            ("kWgradVariants", 1, False, True),
                            ("kWgradS2Variants", 2, False, True),
                            ("kWgradM2Variants", 1, True, True)):
        for v in _table(src, name, 8):
            out[nhwc(v, s, m2, wg)] = name
    for name, s, wg in (("kTiledNchwVariants", 1, False), ("kTiledNchwS2Variants", 2, False),
                        ("kWgradNchwVariants", 1, True), ("kWgradNchwS2Variants", 2, True)):
        for v in _table(src, name, 6):
            out[nchw(v, s, wg)] = name
    for kh, kw, d, cl, px, th, nb, minw in _table(src, "kStreamVariants", 8):
        out[f"stream_nhwc_s1_k{kh}x{kw}_d{d}_cl{cl}_px{px}_th{th}_"] = "kStreamVariants"
    for kh, kw, d, px, th, nl, nb, minw in _table(src, "kStreamNchwVariants", 8):
        out[f"stream_nchw_s1_k{kh}x{kw}_d{d}_px{px}_th{th}_nl{nl}_"] = "kStreamNchwVariants"
    for kh, kw, d, px, th, nl, nb, minw in _table(src, "kStreamPlanesVariants", 8):
        out[f"stream_nchw_planes_s1_k{kh}x{kw}_d{d}_px{px}_th{th}_nl{nl}_"] = \
            "kStreamPlanesVariants"
    for kh, kw, d, th, nl, nb, minw in _table(src, "kWgradStreamVariants", 7):
        out[f"wgrad_stream_nchw_s1_k{kh}x{kw}_d{d}_th{th}_nl{nl}_"] = "kWgradStreamVariants"
    for kh, kw, d, px, th, nb, minw in _table(src, "kWgradStreamNhwcVariants", 7):
        out[f"wgrad_stream_nhwc_s1_k{kh}x{kw}_d{d}_px{px}_th{th}"] = "kWgradStreamNhwcVariants"
    return out


def _sweep():
    """{(prefix, op, mult): problem} with problem = (N, H, W, C, kH, kW, s, d, mult,
    layout): a kernel may have an instantiation per multiplier."""
    prefixes = _expected_prefixes()
    found = {}
    for kh, kw, d in ((3, 3, 1), (5, 5, 1), (7, 7, 1), (7, 7, 2), (1, 15, 1), (1, 31, 1),
                      (1, 1, 1)):
        for layout in (wlmod.NHWC, wlmod.NCHW):
            for s in (1, 2):
                for m in (1, 2):
                    for c in (1, 4, 5, 8, 12, 20, 32, 40, 64, 96, 256):
                        for h, w in ((13, 37), (9, 16), (1, 40)):
                            if kh > 1 and h == 1:
                                continue
                            pads = dw.dwconv2d_same_pads(dw.PAD_SAME, h, w, kh, kw, s, d)
                            for op in (dw.OP_FWD, dw.OP_INPUT_GRAD, dw.OP_WEIGHT_GRAD):
                                for st in (dw.STRATEGY_TILED, dw.STRATEGY_STREAM,
                                           dw.STRATEGY_STREAM_PLANES):
                                    try:
                                        name = dw.dwconv2d_describe_ex(
                                            op, 1, h, w, c, kh, kw, s, d, pads, m, layout, 0,
                                            op == dw.OP_FWD, st)[0]
                                    except dw.DwconvError:
                                        continue
                                    for p in prefixes:
                                        if name.startswith(p) and (p, op, m) not in found:
                                            found[(p, op, m)] = (1, h, w, c, kh, kw, s, d, m,
                                                                 layout, st)
    return prefixes, found


PREFIXES, FOUND = _sweep()
CASES = sorted(FOUND.items())


def test_every_variant_is_reachable():
    reached = {p for p, _, _ in FOUND}
    missing = sorted(p for p in PREFIXES if p not in reached)
    assert not missing, f"variants no problem selects: {missing}"
    assert len(PREFIXES) > 50


@pytest.mark.gpu
@pytest.mark.parametrize("key,prob", CASES,
                         ids=[f"{p}op{op}m{m}" for (p, op, m), _ in CASES])
def test_every_variant_matches_oracle(key, prob):
    import torch
    import oracle
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    prefix, op, _ = key
    n, h, w, c, kh, kw, s, d, m, layout, st = prob
    pads = tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, h, w, kh, kw, s, d))
    wl = Workload(name="cover", N=n, H=h, W=w, C=c, kH=kh, kW=kw, stride=s, dilation=d,
                  pads=pads, mult=m)
    print(f"\n[case] {prefix} op={op} {prob}", flush=True)
    inp = wlmod.make_inputs(wl, layout, seed=7, integer=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    if op == dw.OP_FWD:
        ref, _ = oracle.fwd_general(inp["x"], inp["w"], inp["b"], s, d, pads, m, layout,
                                    nthreads=NTHREADS)
        got = dw.fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), s, d, layout, st, pads=pads,
                     mult=m).cpu().numpy()
        np.testing.assert_array_equal(got, ref.astype(np.float32))
    elif op == dw.OP_INPUT_GRAD:
        ref, _ = oracle.input_grad_general(inp["dy"], inp["w"], h, w, s, d, pads, m, layout,
                                           nthreads=NTHREADS)
        got = dw.input_grad(dev(inp["dy"]), dev(inp["w"]), h, w, s, d, layout, st, pads=pads,
                            mult=m).cpu().numpy()
        np.testing.assert_array_equal(got, ref.astype(np.float32))
    else:
        ref_w, _ = oracle.weight_grad_general(inp["x"], inp["dy"], kh, kw, s, d, pads, m, layout,
                                              nthreads=NTHREADS)
        ref_b, _ = oracle.bias_grad(inp["dy"], layout)
        gw, gb = dw.weight_grad(dev(inp["x"]), dev(inp["dy"]), kh, kw, s, d, layout, strategy=st,
                                pads=pads, mult=m)
        np.testing.assert_array_equal(gw.cpu().numpy(), ref_w.astype(np.float32))
        np.testing.assert_array_equal(gb.cpu().numpy(), ref_b.astype(np.float32))
