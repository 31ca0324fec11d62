"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the passage or mathematical fact it checks.  Integer-valued
inputs keep every partial sum exact in float32 and float64, so most checks
here are exact equalities.  None of these tests needs a GPU.
"""
import glob
import json
import os

import numpy as np
import pytest

from depthwise_convolution_amd import workloads as wlmod
from depthwise_convolution_amd.workloads import NHWC, NCHW, to_layout, from_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [NHWC, NCHW]


def _int_problem(rng, N, H, W, C, kH, kW, s, d, layout):
    x = rng.integers(-3, 4, (N, H, W, C)).astype(np.float32)
    w = rng.integers(-3, 4, (C, kH, kW)).astype(np.float32)
    b = rng.integers(-2, 3, (C,)).astype(np.float32)
    Ho, Wo = -(-H // s), -(-W // s)
    dy = rng.integers(-3, 4, (N, Ho, Wo, C)).astype(np.float32)
    return to_layout(x, layout), w, b, to_layout(dy, layout)


SMALL_CASES = [
    # N, H, W, C, kH, kW, s, d
    (1, 5, 5, 1, 3, 3, 1, 1),
    (2, 6, 7, 3, 3, 3, 2, 1),
    (1, 7, 6, 4, 5, 5, 1, 1),
    (1, 9, 8, 2, 5, 3, 2, 2),
    (2, 8, 9, 3, 7, 7, 1, 2),
    (1, 1, 12, 5, 1, 5, 1, 1),
    (1, 1, 11, 2, 1, 7, 2, 1),
    (1, 5, 1, 3, 3, 1, 1, 1),     # W = 1 boundary
    (1, 3, 4, 2, 7, 7, 1, 1),     # kernel larger than the image
    (1, 7, 7, 2, 3, 3, 2, 3),     # odd extents with stride 2, dilation 3
]


# --------------------------------------------------------------------------
# Hand-worked golden examples (tests/golden/*.json, each carries its citation)
# --------------------------------------------------------------------------
def _golden_files():
    return sorted(f for f in glob.glob(os.path.join(GOLDEN, "*.json"))
                  if not f.endswith("half_decode.json")
                  and not os.path.basename(f).startswith("dense_conv"))


@pytest.mark.parametrize("path", _golden_files(), ids=lambda p: os.path.basename(p))
@pytest.mark.parametrize("layout", LAYOUTS)
def test_golden_examples(oracle_mod, path, layout):
    g = json.load(open(path))
    assert g["citation"]
    s, d = g["stride"], g["dilation"]
    x = to_layout(np.array(g["x_nhwc"], np.float32), layout)
    w = np.array(g["w"], np.float32)
    b = np.array(g["b"], np.float32)
    y, _ = oracle_mod.fwd(x, w, b, s, d, layout)
    np.testing.assert_array_equal(from_layout(y, layout), np.array(g["y_nhwc"], np.float64))
    if "dx_nhwc" in g:
        dy = to_layout(np.array(g["dy_nhwc"], np.float32), layout)
        dx, _ = oracle_mod.input_grad(dy, w, g["H"], g["W"], s, d, layout)
        np.testing.assert_array_equal(from_layout(dx, layout), np.array(g["dx_nhwc"], np.float64))
        dx2 = oracle_mod.input_grad_direct(dy, w, g["H"], g["W"], s, d, layout)
        np.testing.assert_array_equal(from_layout(dx2, layout), np.array(g["dx_nhwc"], np.float64))


def test_half_decode_closed_forms(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "half_decode.json")))
    for bits, val in g["cases"]:
        got = oracle_mod.half_to_double(np.uint16(int(bits, 16)))
        want = float(val)
        assert got == want and np.signbit(got) == np.signbit(want), (bits, got, want)


def test_half_decode_all_patterns_match_numpy(oracle_mod):
    """Every binary16 bit pattern decodes to numpy's float16 value (numpy is an
    independent library implementation of the same format)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.half_to_double(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


# --------------------------------------------------------------------------
# P1: direct-sum and reversed-kernel input gradients agree (LeanMlir
#     "Depthwise": the direct formula is equivalent to the reversed-kernel one)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", SMALL_CASES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_gather_equals_direct_input_grad(oracle_mod, case, layout):
    N, H, W, C, kH, kW, s, d = case
    rng = np.random.default_rng(hash(case) % 2**32)
    x, w, b, dy = _int_problem(rng, N, H, W, C, kH, kW, s, d, layout)
    dx_a, _ = oracle_mod.input_grad(dy, w, H, W, s, d, layout)
    dx_b = oracle_mod.input_grad_direct(dy, w, H, W, s, d, layout)
    np.testing.assert_array_equal(dx_a, dx_b)


# --------------------------------------------------------------------------
# P2: depthwise == regular convolution with a kernel that is zero off the
#     channel diagonal (LeanMlir "Depthwise": regular conv minus the sum over c)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", SMALL_CASES[:6])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_depthwise_is_diagonal_dense_conv(oracle_mod, case, layout):
    N, H, W, C, kH, kW, s, d = case
    rng = np.random.default_rng(7 + C)
    x, w, b, _ = _int_problem(rng, N, H, W, C, kH, kW, s, d, layout)
    wd = np.zeros((C, C, kH, kW), np.float32)
    for c in range(C):
        wd[c, c] = w[c]
    y_dense = oracle_mod.dense_conv(x, wd, b, s, d, layout)
    y_dw, _ = oracle_mod.fwd(x, w, b, s, d, layout)
    np.testing.assert_array_equal(y_dw, y_dense)
    if C > 1:
        # an off-diagonal entry must show up (the dense routine does mix channels)
        wd[0, 1, kH // 2, kW // 2] = 1.0
        assert not np.array_equal(oracle_mod.dense_conv(x, wd, b, s, d, layout), y_dw) or \
            not np.any(from_layout(x, layout)[..., 1])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_dense_conv_golden(oracle_mod, layout):
    """The dense routine on a hand-worked two-channel example whose filters
    are nonzero off the channel diagonal (tests/golden/dense_conv_*.json):
    reading x channel o instead of c, or Wd transposed, fails it."""
    g = json.load(open(os.path.join(GOLDEN, "dense_conv_two_channels_1x3.json")))
    assert g["citation"]
    x = to_layout(np.array(g["x_nhwc"], np.float32), layout)
    wd = np.array(g["wd"], np.float32)
    assert wd.shape == (g["Co"], g["C"], g["kH"], g["kW"])
    b = np.array(g["b"], np.float32)
    y = oracle_mod.dense_conv(x, wd, b, g["stride"], g["dilation"], layout)
    np.testing.assert_array_equal(from_layout(y, layout), np.array(g["y_nhwc"], np.float64))
    # the same arithmetic without the bias, by the definition written out here
    x_l = np.array(g["x_nhwc"], np.float64)[0, 0]          # [w][c]
    xp = np.pad(x_l, ((1, 1), (0, 0)))
    want = np.array([[sum(wd[o, c, 0, k] * xp[w + k, c] for c in range(2) for k in range(3))
                      for o in range(2)] for w in range(3)])
    np.testing.assert_array_equal(from_layout(y, layout)[0, 0] - b, want)


# --------------------------------------------------------------------------
# P3: delta kernels.  A centred delta gives the identity plus bias; a delta one
#     row below centre reads the row d below (cross-correlation, offset kh*d-p)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k,d", [((3, 3), 1), ((5, 5), 1), ((7, 7), 2), ((1, 15), 1), ((3, 5), 3)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_delta_kernels(oracle_mod, k, d, layout):
    kH, kW = k
    rng = np.random.default_rng(3)
    N, H, W, C = 2, 11, 13, 3
    xl = rng.standard_normal((N, H, W, C)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, C).astype(np.float32)
    x = to_layout(xl, layout)
    ch, cw = (kH - 1) // 2, (kW - 1) // 2
    w = np.zeros((C, kH, kW), np.float32)
    w[:, ch, cw] = 1.0
    y, _ = oracle_mod.fwd(x, w, b, 1, d, layout)
    want = xl.astype(np.float64) + b.astype(np.float64)
    np.testing.assert_array_equal(from_layout(y, layout), want)
    if kH > 1:
        w = np.zeros((C, kH, kW), np.float32)
        w[:, ch + 1, cw] = 1.0
        y, _ = oracle_mod.fwd(x, w, b, 1, d, layout)
        want = np.broadcast_to(b.astype(np.float64), (N, H, W, C)).copy()
        want[:, :H - d] += xl[:, d:].astype(np.float64)
        np.testing.assert_array_equal(from_layout(y, layout), want)
        # and the input gradient shifts the other way
        dyl = rng.standard_normal((N, H, W, C)).astype(np.float32)
        dx, _ = oracle_mod.input_grad(to_layout(dyl, layout), w, H, W, 1, d, layout)
        want = np.zeros((N, H, W, C))
        want[:, d:] = dyl[:, :H - d]
        np.testing.assert_array_equal(from_layout(dx, layout), want)
    # a delta right of centre reads the column d to the right
    if kW > 1:
        w = np.zeros((C, kH, kW), np.float32)
        w[:, ch, cw + 1] = 1.0
        y, _ = oracle_mod.fwd(x, w, None, 1, d, layout)
        want = np.zeros((N, H, W, C))
        want[:, :, :W - d] = xl[:, :, d:]
        np.testing.assert_array_equal(from_layout(y, layout), want)


# --------------------------------------------------------------------------
# P4: adjoint identity <dy, fwd(x) - b> == <input_grad(dy), x> (LeanMlir
#     "Depthwise": the input VJP is the VJP of the linear part of an affine map)
#     and the weight-VJP analogue <dy, fwd(x;W) - b> == <dW(x,dy), W>
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", SMALL_CASES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_adjoint_identity(oracle_mod, case, layout):
    N, H, W, C, kH, kW, s, d = case
    rng = np.random.default_rng(11 + H * W)
    x, w, b, dy = _int_problem(rng, N, H, W, C, kH, kW, s, d, layout)
    y, _ = oracle_mod.fwd(x, w, b, s, d, layout)
    dx, _ = oracle_mod.input_grad(dy, w, H, W, s, d, layout)
    bb = b.reshape((1, 1, 1, C)) if layout == NHWC else b.reshape((1, C, 1, 1))
    lhs = int(np.sum((y - bb).astype(np.int64) * dy.astype(np.int64)))
    rhs = int(np.sum(dx.astype(np.int64) * x.astype(np.int64)))
    assert lhs == rhs
    dw, _ = oracle_mod.weight_grad(x, dy, kH, kW, s, d, layout)
    rhs_w = int(np.sum(dw.astype(np.int64) * w.astype(np.int64)))
    assert lhs == rhs_w
    db, _ = oracle_mod.bias_grad(dy, layout)
    axes = (0, 1, 2) if layout == NHWC else (0, 2, 3)
    np.testing.assert_array_equal(db, dy.astype(np.float64).sum(axis=axes))


# --------------------------------------------------------------------------
# P5: stride 2 is the even decimation of stride 1, and its input gradient is
#     the stride-1 input gradient of the zero-upsampled cotangent
#     (LeanMlir "Depthwise": stride-2 SAME and its input-VJP)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("hw", [(8, 8), (9, 7), (1, 10), (12, 1)])
@pytest.mark.parametrize("k,d", [((3, 3), 1), ((5, 5), 2), ((1, 7), 1)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_stride2_is_even_decimation(oracle_mod, hw, k, d, layout):
    H, W = hw
    kH, kW = k
    N, C = 2, 3
    rng = np.random.default_rng(5)
    x, w, b, dy = _int_problem(rng, N, H, W, C, kH, kW, 2, d, layout)
    y1, _ = oracle_mod.fwd(x, w, b, 1, d, layout)
    y2, _ = oracle_mod.fwd(x, w, b, 2, d, layout)
    np.testing.assert_array_equal(from_layout(y2, layout), from_layout(y1, layout)[:, ::2, ::2])
    dyl = from_layout(dy, layout)
    up = np.zeros((N, H, W, C), np.float32)
    up[:, ::2, ::2] = dyl
    dx1, _ = oracle_mod.input_grad(to_layout(up, layout), w, H, W, 1, d, layout)
    dx2, _ = oracle_mod.input_grad(dy, w, H, W, 2, d, layout)
    np.testing.assert_array_equal(dx2, dx1)
    # the odd phase (the XLA-SAME variant) is a different function
    up_odd = np.zeros((N, H, W, C), np.float32)
    ho, wo = up[:, 1::2, 1::2].shape[1:3]
    up_odd[:, 1::2, 1::2] = dyl[:, :ho, :wo]
    if ho and wo and np.any(dyl[:, :ho, :wo]):
        dx_odd, _ = oracle_mod.input_grad(to_layout(up_odd, layout), w, H, W, 1, d, layout)
        assert not np.array_equal(dx_odd, dx2)


# --------------------------------------------------------------------------
# P6: layout invariance -- the NHWC result is the transpose of the NCHW result
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", SMALL_CASES)
def test_layout_invariance(oracle_mod, case):
    N, H, W, C, kH, kW, s, d = case
    rng = np.random.default_rng(17)
    xl = rng.standard_normal((N, H, W, C)).astype(np.float32)
    w = rng.standard_normal((C, kH, kW)).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    dyl = rng.standard_normal((N, -(-H // s), -(-W // s), C)).astype(np.float32)
    ya, Sa = oracle_mod.fwd(to_layout(xl, NHWC), w, b, s, d, NHWC)
    yb, Sb = oracle_mod.fwd(to_layout(xl, NCHW), w, b, s, d, NCHW)
    np.testing.assert_array_equal(ya, from_layout(yb, NCHW))
    np.testing.assert_array_equal(Sa, from_layout(Sb, NCHW))
    da, _ = oracle_mod.input_grad(to_layout(dyl, NHWC), w, H, W, s, d, NHWC)
    db, _ = oracle_mod.input_grad(to_layout(dyl, NCHW), w, H, W, s, d, NCHW)
    np.testing.assert_array_equal(da, from_layout(db, NCHW))


# --------------------------------------------------------------------------
# P7: f16 weights give exactly the f32-weight result on f16-representable
#     values (ggml PR review: F16-kernel output == F32-kernel output)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("layout", LAYOUTS)
def test_f16_weights_equal_f32_weights(oracle_mod, layout):
    rng = np.random.default_rng(23)
    N, H, W, C, kH, kW = 2, 9, 10, 5, 5, 5
    x = to_layout(rng.standard_normal((N, H, W, C)).astype(np.float32), layout)
    w16 = (rng.standard_normal((C, kH, kW)) / 5).astype(np.float16)
    w16[0, 0, 0] = np.float16(2.0 ** -24)      # a subnormal
    w16[1, 1, 1] = np.float16(-6.1e-5)          # near the normal/subnormal edge
    w32 = w16.astype(np.float32)
    b = rng.uniform(-0.1, 0.1, C).astype(np.float32)
    for s in (1, 2):
        ya, Sa = oracle_mod.fwd(x, w16, b, s, 1, layout)
        yb, Sb = oracle_mod.fwd(x, w32, b, s, 1, layout)
        np.testing.assert_array_equal(ya, yb)
        dy = to_layout(rng.standard_normal((N, -(-H // s), -(-W // s), C)).astype(np.float32), layout)
        da, _ = oracle_mod.input_grad(dy, w16, H, W, s, 1, layout)
        db, _ = oracle_mod.input_grad(dy, w32, H, W, s, 1, layout)
        np.testing.assert_array_equal(da, db)


# --------------------------------------------------------------------------
# P8: PyTorch's CPU convolution with groups = C (an independent library
#     implementation; cross-correlation with symmetric zero padding)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("case", SMALL_CASES)
def test_matches_torch_cpu(oracle_mod, case):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    N, H, W, C, kH, kW, s, d = case
    rng = np.random.default_rng(29)
    x, w, b, dy = _int_problem(rng, N, H, W, C, kH, kW, s, d, NCHW)
    pad = (d * (kH - 1) // 2, d * (kW - 1) // 2)
    tx = torch.from_numpy(x).double()
    tw = torch.from_numpy(w).double().view(C, 1, kH, kW)
    tb = torch.from_numpy(b).double()
    ty = F.conv2d(tx, tw, tb, stride=s, padding=pad, dilation=d, groups=C)
    y, _ = oracle_mod.fwd(x, w, b, s, d, NCHW)
    np.testing.assert_array_equal(y, ty.numpy())
    tdx = torch.nn.grad.conv2d_input(tx.shape, tw, torch.from_numpy(dy).double(),
                                     stride=s, padding=pad, dilation=d, groups=C)
    dx, _ = oracle_mod.input_grad(dy, w, H, W, s, d, NCHW)
    np.testing.assert_array_equal(dx, tdx.numpy())
    tdw = torch.nn.grad.conv2d_weight(tx, tw.shape, torch.from_numpy(dy).double(),
                                      stride=s, padding=pad, dilation=d, groups=C)
    dw, _ = oracle_mod.weight_grad(x, dy, kH, kW, s, d, NCHW)
    np.testing.assert_array_equal(dw, tdw.numpy().reshape(C, kH, kW))


def test_matches_torch_cpu_random_float(oracle_mod):
    """Float inputs at a workload shape: agreement within the fp32 bound."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    wl = wlmod.WORKLOADS["asr_n1_30x19x128_7x7_d2"]
    inp = wlmod.make_inputs(wl, NCHW, seed=0)
    pad = (wl.dilation * (wl.kH - 1) // 2, wl.dilation * (wl.kW - 1) // 2)
    tw = torch.from_numpy(inp["w"]).double().view(wl.C, 1, wl.kH, wl.kW)
    ty = F.conv2d(torch.from_numpy(inp["x"]).double(), tw, torch.from_numpy(inp["b"]).double(),
                  stride=wl.stride, padding=pad, dilation=wl.dilation, groups=wl.C).numpy()
    y, S = oracle_mod.fwd(inp["x"], inp["w"], inp["b"], wl.stride, wl.dilation, NCHW)
    assert np.all(np.abs(y - ty) <= 1e-12 * (S + 1))


# --------------------------------------------------------------------------
# P9: constant input x = 1: the interior is sum(W) + b, the borders are the
#     partial sums over the taps that land inside the image (zero padding)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k,d", [((3, 3), 1), ((5, 5), 1), ((7, 7), 2), ((1, 31), 1)])
def test_constant_input_border_sums(oracle_mod, k, d):
    kH, kW = k
    rng = np.random.default_rng(31)
    N, H, W, C = 1, 15, 40, 2
    w = rng.integers(-3, 4, (C, kH, kW)).astype(np.float32)
    b = np.array([1.0, -2.0], np.float32)
    y, _ = oracle_mod.fwd(np.ones((N, H, W, C), np.float32), w, b, 1, d, NHWC)
    pH, pW = d * (kH - 1) // 2, d * (kW - 1) // 2
    for h in range(H):
        for x_w in range(W):
            rows = [kh for kh in range(kH) if 0 <= h + kh * d - pH < H]
            cols = [kw for kw in range(kW) if 0 <= x_w + kw * d - pW < W]
            want = w[:, rows][:, :, cols].sum(axis=(1, 2)) + b
            np.testing.assert_array_equal(y[0, h, x_w], want)


# --------------------------------------------------------------------------
# Sum-of-magnitudes output S: for non-negative inputs it equals the value
# --------------------------------------------------------------------------
def test_sum_of_magnitudes(oracle_mod):
    rng = np.random.default_rng(37)
    x = rng.uniform(0, 1, (1, 6, 7, 4)).astype(np.float32)
    w = rng.uniform(0, 1, (4, 3, 3)).astype(np.float32)
    y, S = oracle_mod.fwd(x, w, None, 1, 1, NHWC)
    np.testing.assert_allclose(S, y, rtol=1e-15)
    y2, S2 = oracle_mod.fwd(x, -w, None, 1, 1, NHWC)
    np.testing.assert_allclose(S2, S, rtol=1e-15)
    np.testing.assert_allclose(y2, -y, rtol=1e-15)


def test_workload_table_shapes():
    """The workload table carries the pages' shapes (ggml [W,H,C,N] order)."""
    W = wlmod.WORKLOADS
    assert (W["asr_n1_30x19x128_7x7"].H, W["asr_n1_30x19x128_7x7"].W) == (30, 19)
    assert (W["asr_n1_1x24x128_1x15"].kH, W["asr_n1_1x24x128_1x15"].kW) == (1, 15)
    big = W["large_512x512x256_3x3"]
    assert big.fwd_bytes() == 536_881_152 and big.ig_bytes() == 536_880_128
    assert W["mobilenet_112x112x32_3x3"].fwd_bytes() == 3_212_544
    s2 = W["mobilenet_s2_224x224x32_3x3"]
    assert (s2.Ho, s2.Wo) == (112, 112) and s2.fwd_bytes() == 8_029_440
    assert W["effnet_n1_56x56x128_5x5_f16w"].fwd_bytes() == 3_218_176
    xla = W["mobilenet_s2_xla_224x224x32_3x3"]
    assert (xla.Ho, xla.Wo) == (112, 112) and xla.fwd_bytes() == s2.fwd_bytes()
    m2 = W["mobilenet_m2_112x112x32_3x3"]
    assert m2.Co == 64 and m2.fwd_bytes() == 4 * 112 * 112 * (32 + 64) + 64 * 9 * 4 + 64 * 4
    rl = W["reactant_4x4x4_3x3_m2_valid"]
    assert (rl.Ho, rl.Wo, rl.Co) == (2, 2, 8)
