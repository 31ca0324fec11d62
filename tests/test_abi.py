"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, and rejects every invalid argument before touching a device.

Fake device addresses are used for the error paths; every call here returns
before any HIP runtime call (validation comes first in every entry point).
"""
import ctypes
import os
import re

import pytest

import depthwise_convolution_amd as dw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dwconv.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dwconv2d_\w+)\s*\(", text)))


def _header_defines():
    return dict((m.group(1), int(m.group(2))) for m in
                re.finditer(r"#define\s+(DWCONV_\w+)\s+(-?\d+)", open(HEADER).read()))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dw.LIB_PATH):
        pytest.fail("libdwconv.so is not built (run __graft_entry__.build())")
    return dw.lib()


def test_exports_every_declared_symbol(L):
    names = _header_functions()
    assert set(names) == set(dw.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_binding_constants_match_header():
    d = _header_defines()
    assert d["DWCONV_LAYOUT_NHWC"] == dw.NHWC and d["DWCONV_LAYOUT_NCHW"] == dw.NCHW
    assert d["DWCONV_W_F32"] == dw.W_F32 and d["DWCONV_W_F16"] == dw.W_F16
    assert d["DWCONV_OP_FWD"] == dw.OP_FWD and d["DWCONV_OP_INPUT_GRAD"] == dw.OP_INPUT_GRAD
    assert d["DWCONV_STRATEGY_AUTO"] == dw.STRATEGY_AUTO
    assert d["DWCONV_STRATEGY_DIRECT"] == dw.STRATEGY_DIRECT
    assert d["DWCONV_STRATEGY_TILED"] == dw.STRATEGY_TILED
    codes = {k[len("DWCONV_ERR_"):]: v for k, v in d.items() if k.startswith("DWCONV_ERR_")}
    for name, v in codes.items():
        assert dw.STATUS[v] == name


def test_version_and_strerror(L):
    assert L.dwconv2d_version() >= 100
    for code in dw.STATUS:
        s = L.dwconv2d_strerror(code).decode()
        assert s and s != "unknown status"
    assert L.dwconv2d_strerror(-999).decode() == "unknown status"


# fake but well-aligned device addresses, far apart
X, WP, B, Y = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000
VP = ctypes.c_void_p


def _fwd(L, x=X, w=WP, wt=0, b=B, y=Y, N=1, H=8, W=8, C=4, kH=3, kW=3, s=1, d=1, lay=0):
    return L.dwconv2d_fwd(VP(x) if x else None, VP(w) if w else None, wt,
                          VP(b) if b else None, VP(y) if y else None,
                          N, H, W, C, kH, kW, s, d, lay, None)


def _ig(L, dy=X, w=WP, wt=0, dx=Y, N=1, H=8, W=8, C=4, kH=3, kW=3, s=1, d=1, lay=0):
    return L.dwconv2d_input_grad(VP(dy) if dy else None, VP(w) if w else None, wt,
                                 VP(dx) if dx else None, N, H, W, C, kH, kW, s, d, lay, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(x=0), -1), (dict(w=0), -1), (dict(y=0), -1),
    (dict(N=0), -2), (dict(H=0), -2), (dict(W=-1), -2), (dict(C=0), -2), (dict(kH=0), -2),
    (dict(N=2, H=1 << 15, W=1 << 15, C=1), -2),            # 2^31 elements
    (dict(s=3), -3), (dict(s=0), -3),
    (dict(d=0), -4), (dict(d=1 << 15, kH=5), -4),
    (dict(kH=2), -5), (dict(kW=4), -5),
    (dict(lay=2), -6), (dict(lay=-1), -6),
    (dict(wt=2), -7),
    (dict(y=X + 64), -8),                                  # output inside the input
    (dict(y=WP - 32), -8),                                 # output runs into the weights
    (dict(b=Y + 4), -8),                                   # bias inside the output
    (dict(x=X + 2), -9), (dict(y=Y + 1), -9), (dict(b=B + 2), -9), (dict(w=WP + 2), -9),
])
def test_fwd_rejects(L, kwargs, code):
    assert _fwd(L, **kwargs) == code


def test_f16_weights_need_only_2_byte_alignment(L):
    # a 2-byte aligned f16 pointer passes the alignment check and the call
    # stops at the later overlap check; a 1-byte offset fails alignment
    assert _fwd(L, w=WP + 2, wt=1, y=X + 64) == -8
    assert _fwd(L, w=WP + 1, wt=1, y=X + 64) == -9


@pytest.mark.parametrize("kwargs,code", [
    (dict(dy=0), -1), (dict(dx=0), -1), (dict(H=0), -2), (dict(s=5), -3), (dict(d=-2), -4),
    (dict(kW=6), -5), (dict(lay=3), -6), (dict(wt=-1), -7),
    (dict(dx=X + 4), -8), (dict(dy=X + 1), -9),
])
def test_input_grad_rejects(L, kwargs, code):
    assert _ig(L, **kwargs) == code


def test_launch_rejects_bad_op_strategy_and_bias_on_input_grad(L):
    args = [VP(X), VP(WP), 0, None, VP(Y), 1, 8, 8, 4, 3, 3, 1, 1, 0]
    assert L.dwconv2d_launch(2, *args, 0, None) == -11
    assert L.dwconv2d_launch(0, *args, 7, None) == -12
    args_b = [VP(X), VP(WP), 0, VP(B), VP(Y), 1, 8, 8, 4, 3, 3, 1, 1, 0]
    assert L.dwconv2d_launch(1, *args_b, 0, None) == -11
    # a tiled strategy where no tiled kernel exists (9x9 kernel)
    args9 = [VP(X), VP(WP), 0, None, VP(Y), 1, 32, 32, 16, 9, 9, 1, 1, 0]
    assert L.dwconv2d_launch(0, *args9, 2, None) == -12


# ------------------------------------------------------------- plan selection
def test_describe_selects_kernels():
    name, grid, block = dw.dwconv2d_describe(dw.OP_FWD, 1, 512, 512, 256, 3, 3)
    assert name.startswith("tiled_nhwc_s1_k3x3_d1") and block == 256 and grid >= 1024
    name, _, _ = dw.dwconv2d_describe(dw.OP_INPUT_GRAD, 1, 512, 512, 256, 3, 3)
    assert name.startswith("tiled_nhwc_s1_k3x3_d1") and name.endswith("_ig_f32w")
    name, _, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 224, 224, 32, 3, 3, stride=2)
    assert name.startswith("tiled_nhwc_s2")
    name, _, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 224, 224, 32, 7, 7, stride=2)
    assert name.startswith("direct_nhwc_s2")             # no stride-2 7x7 variant
    name, _, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 30, 19, 131, 7, 7)
    assert name.startswith("tiled_nhwc_s1_k7x7") and "_l1_" in name   # C % 4 != 0: 4-byte staging
    name, _, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 30, 19, 131, 9, 9)
    assert name.startswith("direct_nhwc_s1_v1")          # no tiled 9x9 variant
    name, _, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 16, 16, 8, 3, 3)
    assert name.startswith("direct_nhwc")                # too few channels for a tile
    name, _, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 16, 16, 8, 3, 3, strategy=dw.STRATEGY_TILED)
    assert name.startswith("tiled_nhwc")
    name, _, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 56, 56, 128, 5, 5, wtype=dw.W_F16)
    assert name.endswith("f16w")
    name, grid, _ = dw.dwconv2d_describe(dw.OP_FWD, 1, 56, 56, 128, 5, 5,
                                         strategy=dw.STRATEGY_DIRECT)
    assert name.startswith("direct_nhwc_s1_v4") and grid == (56 * 56 * 32 + 255) // 256
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_describe(dw.OP_FWD, 1, 8, 8, 4, 3, 3, stride=3)
    assert e.value.status == -3


@pytest.mark.parametrize("wl_name", ["large_512x512x256_3x3", "mobilenet_112x112x32_3x3",
                                     "effnet_n32_56x56x128_5x5", "asr_n64_30x19x128_7x7_d2",
                                     "asr_n64_1x24x256_1x31", "asr_n64_1x24x128_1x15",
                                     "asr_n1_30x19x128_7x7", "prime_n64_30x19x131_7x7",
                                     "prime_n64_1x24x131_1x15"])
def test_tiled_grid_covers_problem(wl_name):
    """The tiled grid (row tiles x column tiles x channel tiles x batch) covers
    every output exactly once: recompute it from the tile sizes in the name."""
    from depthwise_convolution_amd.workloads import WORKLOADS
    wl = WORKLOADS[wl_name]
    name, grid, block = dw.dwconv2d_describe(dw.OP_FWD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                             wl.stride, wl.dilation,
                                             strategy=dw.STRATEGY_TILED)
    assert name.startswith("tiled_nhwc") and block == 256
    vec = int(re.search(r"_v(\d+)_", name).group(1))
    cl = int(re.search(r"_cl(\d+)_", name).group(1))
    px = int(re.search(r"_px(\d+)_", name).group(1))
    g = int(re.search(r"_g(\d+)_", name).group(1))
    th = g - (wl.kH - 1) * wl.dilation
    tw, cg = px * 256 // cl, cl * vec
    assert th >= 1 and (cg % 4 == 0 or "_l1_" in name)
    nct, nwt, nst = -(-wl.C // cg), -(-wl.W // tw), -(-wl.H // th)
    assert grid == wl.N * nct * nwt * nst


@pytest.mark.parametrize("wl_name", ["asr_n64_30x19x128_7x7", "asr_n64_30x19x128_7x7_d2",
                                     "prime_n64_30x19x131_7x7", "asr_n1_30x19x128_7x7"])
def test_stream_grid_covers_problem(wl_name):
    """The row-streaming grid: per channel tile, one wave per (image, row
    tile, dilation phase, column block) of the phase sub-grid (rows and
    columns d apart), four waves per workgroup; with dilation 1 and at most
    two full tiles, the last C % 64 channels, when at most 32, form a tail
    tile of 16 or 32 channels per lane group whose waves span 4 or 2 column
    blocks; AUTO takes it only with at least 1024 waves."""
    from depthwise_convolution_amd.workloads import WORKLOADS
    wl = WORKLOADS[wl_name]
    name, grid, block = dw.dwconv2d_describe(dw.OP_FWD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                             wl.stride, wl.dilation,
                                             strategy=dw.STRATEGY_STREAM)
    assert name.startswith("stream_nhwc") and block == 256
    d = wl.dilation
    cl = int(re.search(r"_cl(\d+)_", name).group(1))
    px = int(re.search(r"_px(\d+)_", name).group(1))
    th = int(re.search(r"_th(\d+)_", name).group(1))
    hs, ws = -(-wl.H // d), -(-wl.W // d)
    units = wl.N * -(-hs // th) * d * d * -(-ws // (px * 64 // cl))
    rem, full = wl.C % cl, wl.C // cl
    tcl = 0
    if rem and 2 * rem <= cl and d == 1 and full <= 2:
        tcl = 16 if rem <= 16 and (wl.C % 4 == 0 or full <= 1) else 32
    assert (f"_t{tcl}_" in name) == (tcl > 0)
    nct = wl.C // cl if tcl else -(-wl.C // cl)
    tunits = wl.N * -(-hs // th) * d * d * -(-ws // (px * 64 // tcl)) if tcl else 0
    assert grid == nct * -(-units // 4) + -(-tunits // 4)
    auto = dw.dwconv2d_describe(dw.OP_FWD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW, wl.stride,
                                wl.dilation)[0]
    assert auto.startswith("stream_") == (nct * units + tunits >= 1024)
    # NCHW: lanes along plane columns, planes packed per wave
    name, grid, _ = dw.dwconv2d_describe(dw.OP_FWD, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                         wl.stride, wl.dilation, dw.NCHW,
                                         strategy=dw.STRATEGY_STREAM)
    px = int(re.search(r"_px(\d+)_", name).group(1))
    th = int(re.search(r"_th(\d+)_", name).group(1))
    lpr = int(re.search(r"_lpr(\d+)_", name).group(1))
    assert lpr == min(64, -(-ws // px))
    ppw = (grid * 4) // (d * d * -(-hs // th) * -(-ws // (64 * px)))
    assert 1 <= -(-wl.N * wl.C // max(1, 64 // lpr)) <= grid * 4


@pytest.mark.parametrize("shape,d", [((64, 30, 19, 128), 1), ((64, 30, 19, 128), 2),
                                     ((64, 30, 19, 131), 2), ((2, 13, 19, 131), 1),
                                     ((1, 9, 150, 3), 2), ((3, 40, 41, 5), 1)])
def test_stream_planes_plan(shape, d):
    """The plane-per-lane NCHW plan: one wave per 16 planes x row phase x
    row tile x 20-column block, four waves per workgroup; the staging loads
    per lane cover 16 planes' in-image window columns (5 loads when the
    window or the plane is at most 20 columns wide); AUTO takes it at
    dilation 2 from 1024 waves and never at dilation 1."""
    N, H, W, C = shape
    pads = tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, H, W, 7, 7, 1, d))
    for op in (dw.OP_FWD, dw.OP_INPUT_GRAD):
        name, grid, block = dw.dwconv2d_describe_ex(op, N, H, W, C, 7, 7, 1, d, pads, 1, dw.NCHW,
                                                    0, op == dw.OP_FWD,
                                                    dw.STRATEGY_STREAM_PLANES)
        assert name.startswith(f"stream_nchw_planes_s1_k7x7_d{d}_px5_th5_") and block == 256
        th = 5
        waves = -(-N * C // 16) * d * -(-(-(-H // d)) // th) * -(-W // 20)
        assert grid == -(-waves // 4)
        win = min(20 + 6 * d, W)
        nl = int(re.search(r"_nl(\d+)_", name).group(1))
        assert nl == (5 if 16 * win <= 320 else (7 if d == 1 else 8))
        auto = dw.dwconv2d_describe_ex(op, N, H, W, C, 7, 7, 1, d, pads, 1, dw.NCHW, 0,
                                       op == dw.OP_FWD, dw.STRATEGY_AUTO)[0]
        assert auto.startswith("stream_nchw_planes_") == (d == 2 and waves >= 1024)


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 4, 4)
    w = torch.zeros(4, 3, 3)
    with pytest.raises(ValueError):
        dw.fwd(x, w)


# ------------------------------------------------------------- weight gradient
WS = 0x50_0000_0000


def _wg(L, x=X, dy=B, dw=Y, db=WP, ws=WS, ws_bytes=1 << 30, N=1, H=8, W=8, C=4, kH=3, kW=3,
        s=1, d=1, lay=0, strat=0):
    return L.dwconv2d_weight_grad(VP(x) if x else None, VP(dy) if dy else None,
                                  VP(dw) if dw else None, VP(db) if db else None,
                                  VP(ws) if ws else None, ws_bytes, N, H, W, C, kH, kW, s, d,
                                  lay, strat, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(x=0), -1), (dict(dy=0), -1), (dict(dw=0), -1),
    (dict(H=0), -2), (dict(s=3), -3), (dict(d=0), -4), (dict(kW=2), -5), (dict(lay=5), -6),
    (dict(x=X + 2), -9), (dict(db=WP + 1), -9),
    (dict(ws=0), -13), (dict(ws=WS + 4), -13), (dict(ws_bytes=16), -13),
    (dict(dw=X + 16), -8), (dict(db=B + 8), -8), (dict(ws=Y), -8), (dict(db=WS + 64), -8),
    (dict(strat=9), -12),
])
def test_weight_grad_rejects(L, kwargs, code):
    assert _wg(L, **kwargs) == code


def test_weight_grad_workspace_and_plans():
    n = dw.dwconv2d_weight_grad_workspace_size(1, 512, 512, 256, 3, 3)
    name, grid, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 1, 512, 512, 256, 3, 3)
    assert name.startswith("wgrad_tiled_nhwc") and n > 0 and n % (4 * 256 * 10) == 0
    # each strategy reports the size of its own plans (AUTO: aligned and
    # misaligned pointers, both tiled here; DIRECT: the generic kernel)
    d = dw.dwconv2d_weight_grad_workspace_size(1, 512, 512, 256, 3, 3,
                                                strategy=dw.STRATEGY_DIRECT)
    assert d > 0 and d % (4 * 256 * 10) == 0
    name, _, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 64, 30, 19, 131, 7, 7,
                                      strategy=dw.STRATEGY_TILED)
    assert name.startswith("wgrad_tiled_nhwc") and "_l1_" in name    # any C, 4-byte staging
    name, grid, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 64, 30, 19, 131, 7, 7)
    assert name.startswith("wgrad_stream_nhwc")                      # AUTO: enough waves
    # two 64-channel tiles of 64 * 6 * 4 units (image, 5-row tile, 5-column
    # block) and a 32-lane tail tile for the last 3 channels, whose waves span
    # 2 column blocks (2 * 64 * 6 units), four units per workgroup
    assert name.endswith("_t32") and grid == 2 * (64 * 6 * 4) // 4 + (64 * 6 * 2) // 4
    name, grid, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 64, 30, 19, 128, 7, 7)
    assert "_t" not in name.split("_th")[1] and grid == 2 * (64 * 6 * 4) // 4
    name, _, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 1, 30, 19, 131, 7, 7)
    assert name.startswith("wgrad_tiled_nhwc")                       # AUTO: too few waves
    name, _, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 1, 224, 224, 32, 3, 3, stride=2)
    assert name.startswith("wgrad_tiled_nhwc_s2")
    name, _, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 1, 224, 224, 32, 7, 7, stride=2)
    assert name.startswith("wgrad_direct_nhwc_s2")                  # no stride-2 7x7 tile
    name, _, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 2, 9, 9, 5, 3, 3, layout=dw.NCHW)
    assert name.startswith("wgrad_tiled_nchw_s1")
    name, _, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 2, 9, 9, 5, 3, 3, stride=2,
                                      layout=dw.NCHW)
    assert name.startswith("wgrad_tiled_nchw_s2")
    name, _, _ = dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 2, 9, 9, 5, 7, 7, stride=2,
                                      layout=dw.NCHW)
    assert name.startswith("wgrad_direct_nchw_s2")
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 1, 8, 8, 4, 3, 3, has_bias=True)
    assert e.value.status == -11
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_describe(dw.OP_WEIGHT_GRAD, 1, 8, 8, 4, 9, 9, strategy=dw.STRATEGY_TILED)
    assert e.value.status == -12


def test_launch_rejects_weight_grad_op(L):
    args = [VP(X), VP(WP), 0, None, VP(Y), 1, 8, 8, 4, 3, 3, 1, 1, 0]
    assert L.dwconv2d_launch(2, *args, 0, None) == -11


# ------------------------------------------- explicit padding, channel multiplier
def _pads(*v):
    return (ctypes.c_int * 4)(*v)


def _fwd_ex(L, x=X, w=WP, wt=0, b=B, y=Y, N=1, H=8, W=8, C=4, m=1, kH=3, kW=3, s=1, d=1,
            pads=(1, 1, 1, 1), lay=0, strat=0, op=0):
    return L.dwconv2d_launch_ex(op, VP(x) if x else None, VP(w) if w else None, wt,
                                VP(b) if b else None, VP(y) if y else None,
                                N, H, W, C, m, kH, kW, s, d,
                                _pads(*pads) if pads is not None else None, lay, strat, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(pads=None), -1), (dict(x=0), -1),
    (dict(m=0), -2), (dict(C=0), -2),
    (dict(pads=(-8, 0, 0, 0)), -2),                    # no window position fits (Ho < 1)
    (dict(H=1, pads=(0, 0, 0, 0)), -2),
    (dict(pads=(1 << 16, 0, 0, 0)), -14), (dict(pads=(0, 0, 0, -(1 << 16))), -14),
    (dict(s=3), -3), (dict(d=0), -4), (dict(lay=4), -6), (dict(wt=3), -7),
    (dict(op=2), -11), (dict(op=1), -11),              # weight-grad op; bias with input grad
    (dict(y=X + 64), -8), (dict(x=X + 2), -9), (dict(strat=5), -12),
])
def test_launch_ex_rejects(L, kwargs, code):
    assert _fwd_ex(L, **kwargs) == code


def test_launch_ex_accepts_even_kernels_and_crops(L):
    # even kernels are valid with explicit pads (the SAME entry points reject
    # them), and so are negative pads while a window position still fits; the
    # call stops at the overlap check, after validation
    assert _fwd_ex(L, kH=2, kW=4, pads=(0, 1, 1, 2), y=X + 64) == -8
    assert _fwd_ex(L, pads=(-1, 0, -2, 1), y=X + 64) == -8
    assert _fwd_ex(L, m=3, y=X + 64) == -8
    assert _fwd(L, kH=2, y=X + 64) == -5


def test_same_pads_and_out_extents():
    """The host helpers against the oracle's own pad rules (XLA-SAME: the
    stride-1 SAME result kept at the odd positions)."""
    import oracle
    for H, W in ((8, 8), (7, 10), (1, 5), (224, 224)):
        for k in ((3, 3), (5, 5), (7, 7), (1, 15), (3, 1)):
            for s in (1, 2):
                for d in (1, 2):
                    same = dw.dwconv2d_same_pads(dw.PAD_SAME, H, W, k[0], k[1], s, d)
                    assert same == oracle.same_pads(H, W, k[0], k[1], s, d)
                    xla = dw.dwconv2d_same_pads(dw.PAD_XLA_SAME, H, W, k[0], k[1], s, d)
                    assert xla == oracle.xla_same_pads(H, W, k[0], k[1], s, d)
                    for pads in (same, xla):
                        want = oracle.out_extents_padded(H, W, k[0], k[1], s, d, pads)
                        if min(want) < 1:
                            with pytest.raises(dw.DwconvError) as e:
                                dw.dwconv2d_out_extents(H, W, k[0], k[1], s, d, pads)
                            assert e.value.status == -2
                        else:
                            assert dw.dwconv2d_out_extents(H, W, k[0], k[1], s, d, pads) == want
                    assert dw.dwconv2d_out_extents(H, W, k[0], k[1], s, d, same) == \
                        (-(-H // s), -(-W // s))
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_same_pads(dw.PAD_SAME, 8, 8, 2, 3)
    assert e.value.status == -5
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv2d_same_pads(7, 8, 8, 3, 3)
    assert e.value.status == -14


def test_describe_ex_plans():
    """Same plans as the SAME entry points for SAME pads; tiled kernels with
    any pads and the multipliers they take; direct kernels for the other
    multipliers and for shapes without a tile; even kernels run direct."""
    same = dw.dwconv2d_describe(dw.OP_FWD, 1, 512, 512, 256, 3, 3)
    assert dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 512, 512, 256, 3, 3, pads=(1, 1, 1, 1)) == same
    name, grid, _ = dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 512, 512, 256, 3, 3, pads=(0, 0, 0, 0))
    assert name.startswith("tiled_nhwc_s1") and grid < same[1]   # 510 x 510 outputs
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_INPUT_GRAD, 1, 56, 56, 128, 5, 5,
                                         pads=(0, 4, 3, 1), layout=dw.NCHW)
    assert name.startswith("tiled_nchw_s1")
    name, grid, _ = dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 112, 112, 32, 3, 3, mult=2)
    assert name.startswith("tiled_nhwc_s1") and "_m2_" in name     # multiplier 2: tiled
    name, grid, _ = dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 112, 112, 32, 3, 3, mult=3)
    assert name.startswith("direct_nhwc_s1_v1") and grid == (112 * 112 * 96 + 255) // 256
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 112, 112, 30, 3, 3, mult=2)
    assert name.startswith("direct_nhwc")                          # C % 4 != 0
    name, grid, _ = dw.dwconv2d_describe_ex(dw.OP_INPUT_GRAD, 1, 112, 112, 32, 3, 3, mult=2,
                                            layout=dw.NCHW)
    assert name.startswith("tiled_nchw_s1") and "_m2_" in name    # dx sums 2 dy planes
    name, grid, _ = dw.dwconv2d_describe_ex(dw.OP_INPUT_GRAD, 1, 112, 112, 32, 3, 3, mult=3,
                                            layout=dw.NCHW)
    assert name.startswith("direct_nchw_s1") and grid == (112 * 112 * 32 + 255) // 256
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 16, 16, 32, 2, 2, pads=(0, 1, 0, 1))
    assert name.startswith("direct_nhwc")
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 224, 224, 32, 3, 3, stride=2,
                                         pads=dw.dwconv2d_same_pads(dw.PAD_XLA_SAME, 224, 224,
                                                                    3, 3, 2))
    assert name.startswith("tiled_nhwc_s2")
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_INPUT_GRAD, 1, 224, 224, 32, 3, 3, stride=2,
                                         pads=(0, 1, 0, 1), layout=dw.NCHW)
    assert name.startswith("tiled_nchw_s2") and "_v1_" in name   # upsampled: 4-byte staging
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_FWD, 1, 56, 56, 32, 7, 7, stride=2,
                                         pads=(3, 3, 3, 3), layout=dw.NCHW)
    assert name.startswith("direct_nchw_s2")                     # no stride-2 7x7 tile
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_WEIGHT_GRAD, 1, 64, 64, 32, 3, 3,
                                         pads=(0, 2, 2, 0))
    assert name.startswith("wgrad_tiled_nhwc")
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_WEIGHT_GRAD, 1, 64, 64, 32, 3, 3, mult=2)
    assert name.startswith("wgrad_tiled_nhwc") and "_m2_" in name
    name, _, _ = dw.dwconv2d_describe_ex(dw.OP_WEIGHT_GRAD, 1, 64, 64, 32, 3, 3, mult=4)
    assert name.startswith("wgrad_direct")
    a = dw.dwconv2d_weight_grad_workspace_size_ex(2, 9, 9, 5, 3, 3, mult=3, layout=dw.NCHW)
    assert a % (4 * 15 * 10) == 0 and a > 0


def test_tiled_nchw_staging_covers_every_tap():
    """The NCHW tile stages columns [w0 - hl, w0 - hl + twl) of each row: for
    any left pad the columns a thread reads, w - left + kw*d for its outputs,
    must fall inside that window (checked by recomputing the planner's hl,
    twl rule for every tile width the planner picks)."""
    for k, d, v4 in (((3, 3), 1, 4), ((5, 5), 1, 4), ((7, 7), 2, 4), ((1, 31), 1, 1),
                     ((7, 7), 1, 1)):
        for left in range(-5, 3 * d * (k[1] - 1)):
            hl = -((-left) & ~3) if v4 == 4 else left
            assert hl >= left and hl - left < v4
            for tw in (32, 64, 256, 512):
                span = (hl - left) + tw + d * (k[1] - 1)
                twl = (span + v4 - 1) // v4 * v4
                # first column read (output 0, tap 0) and last (output tw-1, last tap)
                first = (0 - left) - (0 - hl)
                last = (tw - 1 - left + d * (k[1] - 1)) - (0 - hl)
                assert 0 <= first and last < twl
                extra = (d * (k[1] - 1) + 3 + 3) // 4 * 4 if v4 == 4 else d * (k[1] - 1)
                assert twl <= tw + extra


# ------------------------------------------------------------- fused epilogues
G_, BE, MU, VA = 0x60_0000_0000, 0x61_0000_0000, 0x62_0000_0000, 0x63_0000_0000


def _bn_act(L, x=X, w=WP, b=B, g=G_, be=BE, mu=MU, va=VA, eps=1e-5, act=2, y=Y, C=4, m=1,
            pads=(1, 1, 1, 1)):
    vp = lambda a: VP(a) if a else None
    return L.dwconv2d_fwd_bn_act_ex(vp(x), vp(w), 0, vp(b), vp(g), vp(be), vp(mu), vp(va), eps,
                                    act, vp(y), 1, 8, 8, C, m, 3, 3, 1, 1, _pads(*pads), 0, 0,
                                    None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(act=4), -15), (dict(act=-1), -15), (dict(g=0), -15), (dict(va=0, mu=0), -15),
    (dict(eps=-1.0), -15), (dict(eps=float("inf")), -15), (dict(eps=float("nan")), -15),
    (dict(g=G_ + 2), -9), (dict(y=MU + 4), -8), (dict(y=X + 64), -8), (dict(x=0), -1),
    (dict(pads=(-8, 0, 0, 0)), -2),
])
def test_fwd_bn_act_rejects(L, kwargs, code):
    assert _bn_act(L, **kwargs) == code


def test_fwd_bn_act_without_batchnorm_validates_like_forward(L):
    # no BatchNorm arrays: eps is not looked at; the call stops at the overlap check
    assert _bn_act(L, g=0, be=0, mu=0, va=0, eps=float("nan"), y=X + 64) == -8
    assert _bn_act(L, act=0, y=X + 64) == -8


def _sgd(L, x=X, dy=B, w=Y, b=WP, lr=0.1, dw=0, db=0, ws=WS, ws_bytes=1 << 30, C=4, m=1):
    vp = lambda a: VP(a) if a else None
    return L.dwconv2d_weight_grad_sgd_ex(vp(x), vp(dy), vp(w), vp(b), lr, vp(dw), vp(db), vp(ws),
                                         ws_bytes, 1, 8, 8, C, m, 3, 3, 1, 1, _pads(1, 1, 1, 1),
                                         0, 0, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(w=0), -1), (dict(x=0), -1), (dict(lr=float("nan")), -15), (dict(lr=float("inf")), -15),
    (dict(w=Y + 2), -9), (dict(ws=0), -13), (dict(ws_bytes=16), -13),
    (dict(w=X + 16), -8), (dict(b=B + 8), -8), (dict(dw=Y + 4), -8), (dict(db=WS + 32), -8),
])
def test_weight_grad_sgd_rejects(L, kwargs, code):
    assert _sgd(L, **kwargs) == code


def test_binding_shares_torch_hip_runtime():
    """Loading the library through the binding before anything imports torch
    must still leave one HIP runtime in the process (the one torch uses), so
    that torch's streams and pointers are valid in the library's launches."""
    import subprocess
    import sys
    code = ("import depthwise_convolution_amd as dw; dw.lib(); import torch; "
            "print(len({l.split()[-1] for l in open('/proc/self/maps') "
            "if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


@pytest.mark.parametrize("off", [4, 8, 12])
def test_plans_for_tensors_off_16_byte_alignment(off):
    """A tensor view whose address is 4, 8 or 12 bytes past a 16-byte boundary
    (a contiguous view at a storage offset of 1-3 floats) gets kernels that use
    no 16-byte access: 4-byte staging (`_l1`, `_v1`) or 1-channel direct
    kernels; at a multiple of 16 the plan is the aligned one."""
    def name(op, layout, C, k, addr, s=1, d=1, H=56, W=56, mult=1, bias=False,
             st=dw.STRATEGY_AUTO):
        return dw.dwconv2d_describe_addr_ex(op, 2, H, W, C, k, k, stride=s, dilation=d,
                                            mult=mult, layout=layout, has_bias=bias,
                                            strategy=st, addr_bits=addr)[0]
    T = dw.STRATEGY_TILED
    for k, d in ((3, 1), (5, 1), (7, 1), (7, 2)):
        for op in (dw.OP_FWD, dw.OP_INPUT_GRAD, dw.OP_WEIGHT_GRAD):
            # NHWC: C % 4 == 0 takes 16-byte staging only when aligned
            a = name(op, dw.NHWC, 128, k, 0, d=d, st=T)
            u = name(op, dw.NHWC, 128, k, off, d=d, st=T)
            assert "_l1" not in a and ("_l1" in u or "_v1" in u), (a, u)
            assert name(op, dw.NHWC, 128, k, 16 + 32 * off, d=d, st=T) == a
            # NCHW: whole 16-byte rows (W % 4 == 0) only when aligned
            a = name(op, dw.NCHW, 32, k, 0, d=d, st=T)
            u = name(op, dw.NCHW, 32, k, off, d=d, st=T)
            assert "_v4" in a and "_v4" not in u, (a, u)
    # the row-streaming kernels use 4-byte accesses only: the same plan at
    # any 4-byte alignment
    for lay in (dw.NHWC, dw.NCHW):
        for k, d in ((7, 1), (7, 2)):
            a = name(dw.OP_FWD, lay, 128, k, 0, d=d, st=dw.STRATEGY_STREAM)
            assert a.startswith("stream_") and \
                name(dw.OP_FWD, lay, 128, k, off, d=d, st=dw.STRATEGY_STREAM) == a
    # the bias takes part in the forward's choice (its 4-channel loads)
    assert "_l1" in name(dw.OP_FWD, dw.NHWC, 128, 3, off, bias=True)
    # stride 2, and multiplier 2 (16-byte only): the 4-byte or direct kernels
    assert "_l1" in name(dw.OP_FWD, dw.NHWC, 64, 3, off, s=2)
    assert name(dw.OP_FWD, dw.NHWC, 32, 3, off, mult=2).startswith("direct_nhwc_s1_v1")
    assert "_v1" in name(dw.OP_FWD, dw.NCHW, 32, 3, off, s=2)
    # direct kernels: 4-channel vectors only when aligned
    a = dw.dwconv2d_describe_addr_ex(dw.OP_FWD, 1, 9, 9, 8, 3, 3, layout=dw.NHWC,
                                     strategy=dw.STRATEGY_DIRECT, addr_bits=0)[0]
    u = dw.dwconv2d_describe_addr_ex(dw.OP_FWD, 1, 9, 9, 8, 3, 3, layout=dw.NHWC,
                                     strategy=dw.STRATEGY_DIRECT, addr_bits=off)[0]
    assert "_v4_" in a and "_v1_" in u


def test_weight_grad_noalloc_rejects_before_touching_the_gpu(L):
    """The allocation-free weight gradient validates like the workspace form,
    and a problem whose partial sums need more than the library's scratch
    array (its workspace size above DWCONV_SCRATCH_BYTES) is refused with
    DWCONV_ERR_SCRATCH before any runtime call (fake addresses here)."""
    assert dw.SCRATCH_BYTES == 16 << 20
    text = open(HEADER).read()
    assert re.search(r"#define\s+DWCONV_SCRATCH_BYTES\s+\(16LL << 20\)", text)
    f = L.dwconv2d_weight_grad_noalloc_ex
    x, g, wgt = 0x10000, 0x40000000000, 0x80000000000
    big = (64, 112, 112, 256, 7, 7)                  # 43.75 MiB of partial sums (NHWC)
    pads = dw._pads_arg(dw.dwconv2d_same_pads(dw.PAD_SAME, 112, 112, 7, 7))
    need = dw.dwconv2d_weight_grad_workspace_size_ex(*big[:4], 7, 7, 1, 1, None, 1, dw.NHWC)
    assert need > dw.SCRATCH_BYTES
    N, H, W, C, kH, kW = big
    assert f(x, g, wgt, None, N, H, W, C, 1, kH, kW, 1, 1, pads, dw.NHWC, 0, None) == -16
    assert L.dwconv2d_strerror(-16).decode().startswith("allocation-free")
    # ordinary argument errors come first
    assert f(None, g, wgt, None, 1, 8, 8, 4, 1, 3, 3, 1, 1, pads, dw.NHWC, 0, None) == -1
    assert f(x, g, wgt, None, 1, 8, 8, 4, 1, 3, 3, 3, 1, pads, dw.NHWC, 0, None) == -3
    assert f(x, g, wgt, None, 1, 8, 8, 4, 1, 3, 3, 1, 1, None, dw.NHWC, 0, None) == -1
    assert f(x, g, wgt, None, 1, 8, 8, 4, 1, 3, 3, 1, 1, pads, 5, 0, None) == -6
    assert f(x, g, wgt, None, 1, 8, 8, 4, 1, 3, 3, 1, 1, pads, dw.NHWC, 9, None) == -12


@pytest.mark.parametrize("C", [3, 16, 24, 32, 33, 40, 64, 65, 67, 96, 128, 129, 131, 132, 144,
                               150, 160, 161, 195, 196, 259])
@pytest.mark.parametrize("op", ["fwd", "wgrad"])
def test_stream_tail_tile_rule(C, op):
    """The row-streaming NHWC walks' tail tile, for 64x30x19xC 7x7: the last
    C % 64 channels (at most 32 of them) run with 16 channels per lane group
    when there is at most one full tile or C % 4 == 0, else with 32, and only
    with dilation 1 and at most two full tiles (the measured region); the grid
    is the full tiles' workgroups plus the tail's, whose waves span 64 / lanes
    column blocks of 5 columns."""
    opc = dw.OP_FWD if op == "fwd" else dw.OP_WEIGHT_GRAD
    for d in (1, 2):
        pads = tuple(dw.dwconv2d_same_pads(dw.PAD_SAME, 30, 19, 7, 7, 1, d))
        name, grid, _ = dw.dwconv2d_describe_ex(opc, 64, 30, 19, C, 7, 7, 1, d, pads, 1, dw.NHWC,
                                                0, op == "fwd", dw.STRATEGY_STREAM)
        rem, full = C % 64, C // 64
        tcl = 0
        if rem and 2 * rem <= 64 and d == 1 and full <= 2:
            tcl = 16 if rem <= 16 and (C % 4 == 0 or full <= 1) else 32
        if tcl:
            assert (f"_t{tcl}_" if op == "fwd" else f"_t{tcl}") in name, name
        else:
            assert "_t16" not in name and "_t32" not in name, name
        th = 5 if d == 1 else 8
        hs, ws = -(-30 // d), -(-19 // d)
        units = 64 * -(-hs // th) * d * d * -(-ws // 5)
        nct = full if tcl else -(-C // 64)
        tunits = 64 * -(-hs // th) * d * d * -(-ws // (5 * 64 // tcl)) if tcl else 0
        assert grid == nct * -(-units // 4) + -(-tunits // 4), (name, grid)
