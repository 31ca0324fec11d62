"""Depthwise 2-D convolution for MI355X (gfx950): Python binding of libdwconv.

The binding only marshals arguments: every step of the computation runs in
the HIP kernels of ``libdwconv.so`` (see ``include/dwconv.h`` for the C ABI).
PyTorch provides device memory and the current stream.  If the library has
not been built, every call raises ``RuntimeError``: there is no fallback.

Names mirror the C ABI: ``dwconv2d_fwd``, ``dwconv2d_input_grad``,
``dwconv2d_launch``, ``dwconv2d_describe``, ``dwconv2d_weight_grad``,
``dwconv2d_weight_grad_workspace_size``, ``dwconv2d_strerror``,
``dwconv2d_version``, and the general forms with explicit padding and a
channel multiplier: ``dwconv2d_same_pads``, ``dwconv2d_out_extents``,
``dwconv2d_launch_ex``, ``dwconv2d_describe_ex``, ``dwconv2d_weight_grad_ex``,
``dwconv2d_weight_grad_workspace_size_ex``; the fused epilogues
``dwconv2d_fwd_bn_act_ex`` (BatchNorm + activation in the forward's store)
and ``dwconv2d_weight_grad_sgd_ex`` (SGD step in the weight-gradient
reduction).  ``fwd``, ``input_grad`` and
``weight_grad`` are the same calls with the outputs (and the workspace)
allocated here; given ``pads`` or ``mult`` they use the general forms.

Tensor shapes: NHWC tensors are ``(N, H, W, C)``, NCHW tensors
``(N, C, H, W)``; weights ``(mult*C, kH, kW)`` float32 or float16; bias
``(mult*C,)``; ``pads`` is ``(top, bottom, left, right)``.
"""
import ctypes
import functools
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdwconv.so")

# enumerations of include/dwconv.h
NHWC, NCHW = 0, 1
W_F32, W_F16 = 0, 1
OP_FWD, OP_INPUT_GRAD, OP_WEIGHT_GRAD = 0, 1, 2
STRATEGY_AUTO, STRATEGY_DIRECT, STRATEGY_TILED, STRATEGY_STREAM = 0, 1, 2, 3
STRATEGY_STREAM_PLANES = 4
PAD_SAME, PAD_XLA_SAME = 0, 1
ACT_NONE, ACT_RELU, ACT_RELU6, ACT_SILU = 0, 1, 2, 3
STATUS = {
    0: "OK", -1: "NULL_PTR", -2: "BAD_DIM", -3: "BAD_STRIDE", -4: "BAD_DILATION",
    -5: "EVEN_KERNEL", -6: "BAD_LAYOUT", -7: "BAD_WTYPE", -8: "ALIAS", -9: "MISALIGNED",
    -10: "LAUNCH", -11: "BAD_OP", -12: "BAD_STRATEGY", -13: "WORKSPACE", -14: "BAD_PAD",
    -15: "BAD_EPILOGUE", -16: "SCRATCH",
}
SCRATCH_BYTES = 16 << 20     # DWCONV_SCRATCH_BYTES
EXPORTS = ("dwconv2d_fwd", "dwconv2d_input_grad", "dwconv2d_launch", "dwconv2d_describe",
           "dwconv2d_weight_grad", "dwconv2d_weight_grad_workspace_size",
           "dwconv2d_strerror", "dwconv2d_version",
           "dwconv2d_same_pads", "dwconv2d_out_extents", "dwconv2d_launch_ex",
           "dwconv2d_describe_ex", "dwconv2d_weight_grad_workspace_size_ex",
           "dwconv2d_weight_grad_ex", "dwconv2d_fwd_bn_act_ex", "dwconv2d_weight_grad_sgd_ex",
           "dwconv2d_describe_addr_ex", "dwconv2d_weight_grad_noalloc_ex")

_lib = None


class DwconvError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_strerror(status)})")


def lib():
    """The loaded libdwconv.so (ctypes), with argument types set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libdwconv.so not found at {LIB_PATH}: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()'); there is no fallback path")
    # torch carries its own copy of the HIP runtime.  Importing it first makes
    # this library bind to that copy (same soname), so torch's streams and
    # allocations are valid in its launches; loaded the other way round the
    # process would hold two HIP runtimes, and a launch on a torch stream
    # would be rejected by the wrong one.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    i, vp, ll = ctypes.c_int, ctypes.c_void_p, ctypes.c_longlong
    L.dwconv2d_fwd.argtypes = [vp, vp, i, vp, vp] + [i] * 9 + [vp]
    L.dwconv2d_input_grad.argtypes = [vp, vp, i, vp] + [i] * 9 + [vp]
    L.dwconv2d_launch.argtypes = [i, vp, vp, i, vp, vp] + [i] * 10 + [vp]
    L.dwconv2d_describe.argtypes = [i] * 13 + [ctypes.c_char_p, i, ctypes.POINTER(ll),
                                               ctypes.POINTER(i)]
    L.dwconv2d_weight_grad_workspace_size.argtypes = [i] * 10 + [ctypes.POINTER(ll)]
    L.dwconv2d_weight_grad.argtypes = [vp, vp, vp, vp, vp, ll] + [i] * 10 + [vp]
    ip = ctypes.POINTER(i)
    L.dwconv2d_same_pads.argtypes = [i] * 7 + [ip]
    L.dwconv2d_out_extents.argtypes = [i] * 6 + [ip, ip, ip]
    L.dwconv2d_launch_ex.argtypes = [i, vp, vp, i, vp, vp] + [i] * 9 + [ip, i, i, vp]
    L.dwconv2d_describe_ex.argtypes = [i] * 12 + [ip, i, i, ctypes.c_char_p, i,
                                                  ctypes.POINTER(ll), ip]
    L.dwconv2d_describe_addr_ex.argtypes = [i] * 12 + [ip, i, i, ctypes.c_ulonglong,
                                                       ctypes.c_char_p, i, ctypes.POINTER(ll), ip]
    L.dwconv2d_weight_grad_workspace_size_ex.argtypes = [i] * 9 + [ip, i, i, ctypes.POINTER(ll)]
    L.dwconv2d_weight_grad_ex.argtypes = [vp, vp, vp, vp, vp, ll] + [i] * 9 + [ip, i, i, vp]
    L.dwconv2d_weight_grad_noalloc_ex.argtypes = [vp, vp, vp, vp] + [i] * 9 + [ip, i, i, vp]
    f32 = ctypes.c_float
    L.dwconv2d_fwd_bn_act_ex.argtypes = ([vp, vp, i, vp, vp, vp, vp, vp, f32, i, vp] + [i] * 9 +
                                         [ip, i, i, vp])
    L.dwconv2d_weight_grad_sgd_ex.argtypes = ([vp, vp, vp, vp, f32, vp, vp, vp, ll] + [i] * 9 +
                                              [ip, i, i, vp])
    L.dwconv2d_strerror.argtypes = [i]
    L.dwconv2d_strerror.restype = ctypes.c_char_p
    for f in EXPORTS:
        if f != "dwconv2d_strerror":
            getattr(L, f).restype = i
    _lib = L
    return L


def _strerror(status):
    try:
        return lib().dwconv2d_strerror(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def dwconv2d_strerror(status):
    return _strerror(status)


def dwconv2d_version():
    return lib().dwconv2d_version()


# ---------------------------------------------------------------- marshalling
def _layout_code(layout):
    if layout in (NHWC, "nhwc", "NHWC"):
        return NHWC
    if layout in (NCHW, "nchw", "NCHW"):
        return NCHW
    raise ValueError(f"unknown layout {layout!r}")


def _dims(t, layout):
    if t.dim() != 4:
        raise ValueError("activation tensors must be 4-D")
    if layout == NHWC:
        n, h, w, c = t.shape
    else:
        n, c, h, w = t.shape
    return int(n), int(h), int(w), int(c)


def _shape(layout, n, h, w, c):
    return (n, h, w, c) if layout == NHWC else (n, c, h, w)


def _check_dev(t, name, dtypes):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _wtype(w):
    import torch
    _check_dev(w, "w", (torch.float32, torch.float16))
    if w.dim() != 3:
        raise ValueError("w must be (C, kH, kW)")
    return W_F16 if w.dtype == torch.float16 else W_F32


def _stream(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    # a plain int converts to the c_void_p argument type
    return None if t is None else t.data_ptr()


def _check_status(st, what):
    if st != 0:
        raise DwconvError(st, what)


def _prepare(op, inp, w, b, out, H, W, stride, dilation, layout):
    import torch
    lay = _layout_code(layout)
    _check_dev(inp, "input", (torch.float32,))
    _check_dev(out, "output", (torch.float32,))
    wt = _wtype(w)
    C, kH, kW = (int(v) for v in w.shape)
    if b is not None:
        _check_dev(b, "b", (torch.float32,))
        if tuple(b.shape) != (C,):
            raise ValueError("b must be (C,)")
    Ho, Wo = -(-H // stride), -(-W // stride)
    N = int(inp.shape[0])
    big, small = _shape(lay, N, H, W, C), _shape(lay, N, Ho, Wo, C)
    want_in, want_out = (big, small) if op == OP_FWD else (small, big)
    if tuple(inp.shape) != want_in or tuple(out.shape) != want_out:
        raise ValueError(f"shape mismatch: input {tuple(inp.shape)} (want {want_in}), "
                         f"output {tuple(out.shape)} (want {want_out})")
    if not (inp.device == out.device == w.device) or (b is not None and b.device != out.device):
        raise ValueError("all tensors must be on the same device")
    return lay, wt, N, C, kH, kW


def dwconv2d_launch(op, inp, w, b, out, H, W, stride=1, dilation=1, layout=NHWC,
                    strategy=STRATEGY_AUTO, stream=None):
    """Enqueue op (OP_FWD / OP_INPUT_GRAD) under `strategy` into `out`."""
    lay, wt, N, C, kH, kW = _prepare(op, inp, w, b, out, H, W, stride, dilation, layout)
    st = lib().dwconv2d_launch(op, _ptr(inp), _ptr(w), wt, _ptr(b), _ptr(out), N, H, W, C,
                               kH, kW, stride, dilation, lay, strategy, _stream(out, stream))
    _check_status(st, "dwconv2d_launch")
    return out


def dwconv2d_fwd(x, w, b, y, stride=1, dilation=1, layout=NHWC, stream=None):
    """y = depthwise_conv(x; w, b), written into the preallocated y."""
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    lay, wt, N, C, kH, kW = _prepare(OP_FWD, x, w, b, y, H, W, stride, dilation, lay)
    st = lib().dwconv2d_fwd(_ptr(x), _ptr(w), wt, _ptr(b), _ptr(y), N, H, W, C, kH, kW,
                            stride, dilation, lay, _stream(y, stream))
    _check_status(st, "dwconv2d_fwd")
    return y


def dwconv2d_input_grad(dy, w, dx, stride=1, dilation=1, layout=NHWC, stream=None):
    """dx = input gradient of depthwise_conv for cotangent dy, into preallocated dx."""
    lay = _layout_code(layout)
    N, H, W, C = _dims(dx, lay)
    lay, wt, N, C, kH, kW = _prepare(OP_INPUT_GRAD, dy, w, None, dx, H, W, stride, dilation,
                                     lay)
    st = lib().dwconv2d_input_grad(_ptr(dy), _ptr(w), wt, _ptr(dx), N, H, W, C, kH, kW,
                                   stride, dilation, lay, _stream(dx, stream))
    _check_status(st, "dwconv2d_input_grad")
    return dx


def dwconv2d_describe(op, N, H, W, C, kH, kW, stride=1, dilation=1, layout=NHWC,
                      wtype=W_F32, has_bias=False, strategy=STRATEGY_AUTO):
    """(kernel name, grid, block) that a launch with these arguments would use."""
    name = ctypes.create_string_buffer(128)
    grid, block = ctypes.c_longlong(0), ctypes.c_int(0)
    st = lib().dwconv2d_describe(op, wtype, int(bool(has_bias)), N, H, W, C, kH, kW, stride,
                                 dilation, _layout_code(layout), strategy, name, 128,
                                 ctypes.byref(grid), ctypes.byref(block))
    _check_status(st, "dwconv2d_describe")
    return name.value.decode(), grid.value, block.value


# ------------------------------------------------------------- conveniences
def fwd(x, w, b=None, stride=1, dilation=1, layout=NHWC, strategy=STRATEGY_AUTO, stream=None,
        pads=None, mult=1):
    """Allocate y and run the forward pass (general form when pads or mult given)."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    if pads is None and mult == 1:
        y = torch.empty(_shape(lay, N, -(-H // stride), -(-W // stride), C),
                        dtype=torch.float32, device=x.device)
        return dwconv2d_launch(OP_FWD, x, w, b, y, H, W, stride, dilation, lay, strategy,
                               stream)
    kH, kW = int(w.shape[1]), int(w.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    Ho, Wo = dwconv2d_out_extents(H, W, kH, kW, stride, dilation, pads)
    y = torch.empty(_shape(lay, N, Ho, Wo, mult * C), dtype=torch.float32, device=x.device)
    return dwconv2d_launch_ex(OP_FWD, x, w, b, y, H, W, stride, dilation, pads, mult, lay,
                              strategy, stream)


def input_grad(dy, w, H, W, stride=1, dilation=1, layout=NHWC, strategy=STRATEGY_AUTO,
               stream=None, pads=None, mult=1):
    """Allocate dx of forward-input extents (H, W) and run the input gradient."""
    import torch
    lay = _layout_code(layout)
    N, _, _, Cy = _dims(dy, lay)
    if pads is None and mult == 1:
        dx = torch.empty(_shape(lay, N, H, W, Cy), dtype=torch.float32, device=dy.device)
        return dwconv2d_launch(OP_INPUT_GRAD, dy, w, None, dx, H, W, stride, dilation, lay,
                               strategy, stream)
    kH, kW = int(w.shape[1]), int(w.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    dx = torch.empty(_shape(lay, N, H, W, Cy // mult), dtype=torch.float32, device=dy.device)
    return dwconv2d_launch_ex(OP_INPUT_GRAD, dy, w, None, dx, H, W, stride, dilation, pads,
                              mult, lay, strategy, stream)


def dwconv2d_weight_grad_workspace_size(N, H, W, C, kH, kW, stride=1, dilation=1, layout=NHWC,
                                        strategy=STRATEGY_AUTO):
    """Workspace bytes dwconv2d_weight_grad needs for these arguments."""
    out = ctypes.c_longlong(0)
    st = lib().dwconv2d_weight_grad_workspace_size(N, H, W, C, kH, kW, stride, dilation,
                                                   _layout_code(layout), strategy,
                                                   ctypes.byref(out))
    _check_status(st, "dwconv2d_weight_grad_workspace_size")
    return out.value


def dwconv2d_weight_grad(x, dy, dw, db, workspace, stride=1, dilation=1, layout=NHWC,
                         strategy=STRATEGY_AUTO, stream=None):
    """dw (and db unless None) = weight / bias gradients for input x and cotangent dy."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    _check_dev(x, "x", (torch.float32,))
    _check_dev(dy, "dy", (torch.float32,))
    _check_dev(dw, "dw", (torch.float32,))
    if dw.dim() != 3 or int(dw.shape[0]) != C:
        raise ValueError("dw must be (C, kH, kW)")
    kH, kW = int(dw.shape[1]), int(dw.shape[2])
    if db is not None:
        _check_dev(db, "db", (torch.float32,))
        if tuple(db.shape) != (C,):
            raise ValueError("db must be (C,)")
    Ho, Wo = -(-H // stride), -(-W // stride)
    if tuple(dy.shape) != _shape(lay, N, Ho, Wo, C):
        raise ValueError(f"dy shape {tuple(dy.shape)} != {_shape(lay, N, Ho, Wo, C)}")
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().dwconv2d_weight_grad(_ptr(x), _ptr(dy), _ptr(dw), _ptr(db), _ptr(workspace),
                                    nbytes, N, H, W, C, kH, kW, stride, dilation, lay, strategy,
                                    _stream(dw, stream))
    _check_status(st, "dwconv2d_weight_grad")
    return dw, db


def weight_grad(x, dy, kH, kW, stride=1, dilation=1, layout=NHWC, with_bias=True,
                strategy=STRATEGY_AUTO, stream=None, pads=None, mult=1):
    """Allocate dW (mult*C, kH, kW), db (mult*C,) and the workspace; run the
    weight gradient (general form when pads or mult given)."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    general = pads is not None or mult != 1
    if general:
        pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
        nbytes = dwconv2d_weight_grad_workspace_size_ex(N, H, W, C, kH, kW, stride, dilation,
                                                        pads, mult, lay, strategy)
    else:
        nbytes = dwconv2d_weight_grad_workspace_size(N, H, W, C, kH, kW, stride, dilation, lay,
                                                     strategy)
    ws = torch.empty(max(1, (nbytes + 15) // 16) * 4, dtype=torch.float32, device=x.device)
    dw = torch.empty((mult * C, kH, kW), dtype=torch.float32, device=x.device)
    db = torch.empty((mult * C,), dtype=torch.float32, device=x.device) if with_bias else None
    if general:
        return dwconv2d_weight_grad_ex(x, dy, dw, db, ws, stride, dilation, pads, mult, lay,
                                       strategy, stream)
    return dwconv2d_weight_grad(x, dy, dw, db, ws, stride, dilation, lay, strategy, stream)


# ------------------------------------------- explicit padding, channel multiplier
def _pads_arg(pads):
    if pads is None or len(pads) != 4:
        raise ValueError("pads must be (top, bottom, left, right)")
    return _pads_array(tuple(int(v) for v in pads))


@functools.lru_cache(maxsize=256)
def _pads_array(pads):
    # read-only for the library (const int *), so one array per pads tuple serves every call
    return (ctypes.c_int * 4)(*pads)


def _pads_or_same(pads, H, W, kH, kW, stride, dilation):
    if pads is None:
        return _same_pads_cached(H, W, kH, kW, stride, dilation)
    return tuple(int(v) for v in pads)


@functools.lru_cache(maxsize=1024)
def _same_pads_cached(H, W, kH, kW, stride, dilation):
    return dwconv2d_same_pads(PAD_SAME, H, W, kH, kW, stride, dilation)


def dwconv2d_same_pads(mode, H, W, kH, kW, stride=1, dilation=1):
    """(top, bottom, left, right) of PAD_SAME or PAD_XLA_SAME."""
    out = (ctypes.c_int * 4)()
    st = lib().dwconv2d_same_pads(mode, H, W, kH, kW, stride, dilation, out)
    _check_status(st, "dwconv2d_same_pads")
    return tuple(out)


def dwconv2d_out_extents(H, W, kH, kW, stride, dilation, pads):
    """(Ho, Wo) of a padded problem."""
    return _out_extents_cached(int(H), int(W), int(kH), int(kW), int(stride), int(dilation),
                               tuple(int(v) for v in pads))


@functools.lru_cache(maxsize=1024)
def _out_extents_cached(H, W, kH, kW, stride, dilation, pads):
    ho, wo = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().dwconv2d_out_extents(H, W, kH, kW, stride, dilation, _pads_arg(pads),
                                    ctypes.byref(ho), ctypes.byref(wo))
    _check_status(st, "dwconv2d_out_extents")
    return ho.value, wo.value


def _prepare_ex(op, inp, w, b, out, H, W, stride, dilation, pads, mult, layout):
    import torch
    lay = _layout_code(layout)
    _check_dev(inp, "input", (torch.float32,))
    _check_dev(out, "output", (torch.float32,))
    wt = _wtype(w)
    Co, kH, kW = (int(v) for v in w.shape)
    if mult < 1 or Co % mult != 0:
        raise ValueError("w must be (mult*C, kH, kW)")
    C = Co // mult
    if b is not None:
        _check_dev(b, "b", (torch.float32,))
        if tuple(b.shape) != (Co,):
            raise ValueError("b must be (mult*C,)")
    Ho, Wo = dwconv2d_out_extents(H, W, kH, kW, stride, dilation, pads)
    N = int(inp.shape[0])
    big, small = _shape(lay, N, H, W, C), _shape(lay, N, Ho, Wo, Co)
    want_in, want_out = (big, small) if op == OP_FWD else (small, big)
    if tuple(inp.shape) != want_in or tuple(out.shape) != want_out:
        raise ValueError(f"shape mismatch: input {tuple(inp.shape)} (want {want_in}), "
                         f"output {tuple(out.shape)} (want {want_out})")
    if not (inp.device == out.device == w.device) or (b is not None and b.device != out.device):
        raise ValueError("all tensors must be on the same device")
    return lay, wt, N, C, kH, kW


def dwconv2d_launch_ex(op, inp, w, b, out, H, W, stride=1, dilation=1, pads=None, mult=1,
                       layout=NHWC, strategy=STRATEGY_AUTO, stream=None):
    """Enqueue op (OP_FWD / OP_INPUT_GRAD) with explicit pads and channel multiplier."""
    kH, kW = int(w.shape[1]), int(w.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    lay, wt, N, C, kH, kW = _prepare_ex(op, inp, w, b, out, H, W, stride, dilation, pads, mult,
                                        layout)
    st = lib().dwconv2d_launch_ex(op, _ptr(inp), _ptr(w), wt, _ptr(b), _ptr(out), N, H, W, C,
                                  mult, kH, kW, stride, dilation, _pads_arg(pads), lay, strategy,
                                  _stream(out, stream))
    _check_status(st, "dwconv2d_launch_ex")
    return out


def dwconv2d_describe_ex(op, N, H, W, C, kH, kW, stride=1, dilation=1, pads=None, mult=1,
                         layout=NHWC, wtype=W_F32, has_bias=False, strategy=STRATEGY_AUTO):
    """(kernel name, grid, block) of a general-form launch."""
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    name = ctypes.create_string_buffer(128)
    grid, block = ctypes.c_longlong(0), ctypes.c_int(0)
    st = lib().dwconv2d_describe_ex(op, wtype, int(bool(has_bias)), N, H, W, C, mult, kH, kW,
                                    stride, dilation, _pads_arg(pads), _layout_code(layout),
                                    strategy, name, 128, ctypes.byref(grid), ctypes.byref(block))
    _check_status(st, "dwconv2d_describe_ex")
    return name.value.decode(), grid.value, block.value


def dwconv2d_describe_addr_ex(op, N, H, W, C, kH, kW, stride=1, dilation=1, pads=None, mult=1,
                              layout=NHWC, wtype=W_F32, has_bias=False, strategy=STRATEGY_AUTO,
                              addr_bits=0):
    """(kernel name, grid, block) of a general-form launch whose tensor
    addresses OR together to `addr_bits` (0: all 16-byte aligned)."""
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    name = ctypes.create_string_buffer(128)
    grid, block = ctypes.c_longlong(0), ctypes.c_int(0)
    st = lib().dwconv2d_describe_addr_ex(op, wtype, int(bool(has_bias)), N, H, W, C, mult, kH,
                                         kW, stride, dilation, _pads_arg(pads),
                                         _layout_code(layout), strategy, int(addr_bits), name,
                                         128, ctypes.byref(grid), ctypes.byref(block))
    _check_status(st, "dwconv2d_describe_addr_ex")
    return name.value.decode(), grid.value, block.value


def dwconv2d_weight_grad_workspace_size_ex(N, H, W, C, kH, kW, stride=1, dilation=1, pads=None,
                                           mult=1, layout=NHWC, strategy=STRATEGY_AUTO):
    """Workspace bytes of dwconv2d_weight_grad_ex."""
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    out = ctypes.c_longlong(0)
    st = lib().dwconv2d_weight_grad_workspace_size_ex(N, H, W, C, mult, kH, kW, stride,
                                                      dilation, _pads_arg(pads),
                                                      _layout_code(layout), strategy,
                                                      ctypes.byref(out))
    _check_status(st, "dwconv2d_weight_grad_workspace_size_ex")
    return out.value


def dwconv2d_weight_grad_ex(x, dy, dw, db, workspace, stride=1, dilation=1, pads=None, mult=1,
                            layout=NHWC, strategy=STRATEGY_AUTO, stream=None):
    """dw (mult*C, kH, kW) and db (mult*C,) unless None, general form."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    _check_dev(x, "x", (torch.float32,))
    _check_dev(dy, "dy", (torch.float32,))
    _check_dev(dw, "dw", (torch.float32,))
    if dw.dim() != 3 or int(dw.shape[0]) != mult * C:
        raise ValueError("dw must be (mult*C, kH, kW)")
    kH, kW = int(dw.shape[1]), int(dw.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    if db is not None:
        _check_dev(db, "db", (torch.float32,))
        if tuple(db.shape) != (mult * C,):
            raise ValueError("db must be (mult*C,)")
    Ho, Wo = dwconv2d_out_extents(H, W, kH, kW, stride, dilation, pads)
    if tuple(dy.shape) != _shape(lay, N, Ho, Wo, mult * C):
        raise ValueError(f"dy shape {tuple(dy.shape)} != {_shape(lay, N, Ho, Wo, mult * C)}")
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().dwconv2d_weight_grad_ex(_ptr(x), _ptr(dy), _ptr(dw), _ptr(db), _ptr(workspace),
                                       nbytes, N, H, W, C, mult, kH, kW, stride, dilation,
                                       _pads_arg(pads), lay, strategy, _stream(dw, stream))
    _check_status(st, "dwconv2d_weight_grad_ex")
    return dw, db



def dwconv2d_weight_grad_noalloc_ex(x, dy, dw, db, stride=1, dilation=1, pads=None, mult=1,
                                    layout=NHWC, strategy=STRATEGY_AUTO, stream=None):
    """dwconv2d_weight_grad_ex with the partial sums in the library's own
    scratch array (no workspace, no allocation): for callers that cannot
    allocate.  Calls that overlap on one GPU race on that array."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    _check_dev(x, "x", (torch.float32,))
    _check_dev(dy, "dy", (torch.float32,))
    _check_dev(dw, "dw", (torch.float32,))
    if dw.dim() != 3 or int(dw.shape[0]) != mult * C:
        raise ValueError("dw must be (mult*C, kH, kW)")
    kH, kW = int(dw.shape[1]), int(dw.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    if db is not None:
        _check_dev(db, "db", (torch.float32,))
        if tuple(db.shape) != (mult * C,):
            raise ValueError("db must be (mult*C,)")
    Ho, Wo = dwconv2d_out_extents(H, W, kH, kW, stride, dilation, pads)
    if tuple(dy.shape) != _shape(lay, N, Ho, Wo, mult * C):
        raise ValueError(f"dy shape {tuple(dy.shape)} != {_shape(lay, N, Ho, Wo, mult * C)}")
    st = lib().dwconv2d_weight_grad_noalloc_ex(_ptr(x), _ptr(dy), _ptr(dw), _ptr(db), N, H, W,
                                               C, mult, kH, kW, stride, dilation,
                                               _pads_arg(pads), lay, strategy,
                                               _stream(dw, stream))
    _check_status(st, "dwconv2d_weight_grad_noalloc_ex")
    return dw, db


# ------------------------------------------------------------- fused epilogues
def _act_code(act):
    names = {"none": ACT_NONE, "relu": ACT_RELU, "relu6": ACT_RELU6, "silu": ACT_SILU}
    if isinstance(act, str):
        if act.lower() not in names:
            raise ValueError(f"unknown activation {act!r}")
        return names[act.lower()]
    return int(act)


def dwconv2d_fwd_bn_act_ex(x, w, b, y, bn=None, eps=1e-5, act=ACT_NONE, stride=1, dilation=1,
                           pads=None, mult=1, layout=NHWC, strategy=STRATEGY_AUTO, stream=None):
    """y = act(BatchNorm(conv(x; w, b))) in one pass; bn = (gamma, beta, mean, var)
    float32 GPU tensors of mult*C elements, or None."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    kH, kW = int(w.shape[1]), int(w.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    lay, wt, N, C, kH, kW = _prepare_ex(OP_FWD, x, w, b, y, H, W, stride, dilation, pads, mult,
                                        lay)
    ptrs = [None] * 4
    if bn is not None:
        if len(bn) != 4:
            raise ValueError("bn must be (gamma, beta, mean, var)")
        for k, t in enumerate(bn):
            _check_dev(t, ("gamma", "beta", "mean", "var")[k], (torch.float32,))
            if tuple(t.shape) != (mult * C,):
                raise ValueError("BatchNorm arrays must be (mult*C,)")
            ptrs[k] = _ptr(t)
    st = lib().dwconv2d_fwd_bn_act_ex(_ptr(x), _ptr(w), wt, _ptr(b), *ptrs, float(eps),
                                      _act_code(act), _ptr(y), N, H, W, C, mult, kH, kW, stride,
                                      dilation, _pads_arg(pads), lay, strategy, _stream(y, stream))
    _check_status(st, "dwconv2d_fwd_bn_act_ex")
    return y


def fwd_bn_act(x, w, b=None, bn=None, eps=1e-5, act=ACT_NONE, stride=1, dilation=1,
               layout=NHWC, strategy=STRATEGY_AUTO, stream=None, pads=None, mult=1):
    """Allocate y and run the forward with the fused BatchNorm / activation."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    kH, kW = int(w.shape[1]), int(w.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    Ho, Wo = dwconv2d_out_extents(H, W, kH, kW, stride, dilation, pads)
    y = torch.empty(_shape(lay, N, Ho, Wo, mult * C), dtype=torch.float32, device=x.device)
    return dwconv2d_fwd_bn_act_ex(x, w, b, y, bn, eps, act, stride, dilation, pads, mult, lay,
                                  strategy, stream)


def dwconv2d_weight_grad_sgd_ex(x, dy, w, b, lr, workspace, dw=None, db=None, stride=1,
                                dilation=1, pads=None, mult=1, layout=NHWC,
                                strategy=STRATEGY_AUTO, stream=None):
    """In place: w -= lr * dW, b -= lr * db (b may be None); dw, db optionally
    receive the gradients."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    for name, t in (("x", x), ("dy", dy), ("w", w)):
        _check_dev(t, name, (torch.float32,))
    if w.dim() != 3 or int(w.shape[0]) != mult * C:
        raise ValueError("w must be (mult*C, kH, kW) float32")
    kH, kW = int(w.shape[1]), int(w.shape[2])
    for name, t, shape in (("b", b, (mult * C,)), ("dw", dw, tuple(w.shape)),
                           ("db", db, (mult * C,))):
        if t is not None:
            _check_dev(t, name, (torch.float32,))
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must be {shape}")
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    Ho, Wo = dwconv2d_out_extents(H, W, kH, kW, stride, dilation, pads)
    if tuple(dy.shape) != _shape(lay, N, Ho, Wo, mult * C):
        raise ValueError(f"dy shape {tuple(dy.shape)} != {_shape(lay, N, Ho, Wo, mult * C)}")
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().dwconv2d_weight_grad_sgd_ex(_ptr(x), _ptr(dy), _ptr(w), _ptr(b), float(lr),
                                           _ptr(dw), _ptr(db), _ptr(workspace), nbytes, N, H, W,
                                           C, mult, kH, kW, stride, dilation, _pads_arg(pads), lay,
                                           strategy, _stream(w, stream))
    _check_status(st, "dwconv2d_weight_grad_sgd_ex")
    return w, b


def weight_grad_sgd(x, dy, w, b, lr, stride=1, dilation=1, layout=NHWC, strategy=STRATEGY_AUTO,
                    stream=None, pads=None, mult=1):
    """Allocate the workspace and apply the fused SGD step to w (and b) in place."""
    import torch
    lay = _layout_code(layout)
    N, H, W, C = _dims(x, lay)
    kH, kW = int(w.shape[1]), int(w.shape[2])
    pads = _pads_or_same(pads, H, W, kH, kW, stride, dilation)
    nbytes = dwconv2d_weight_grad_workspace_size_ex(N, H, W, C, kH, kW, stride, dilation, pads,
                                                    mult, lay, strategy)
    ws = torch.empty(max(1, (nbytes + 15) // 16) * 4, dtype=torch.float32, device=x.device)
    return dwconv2d_weight_grad_sgd_ex(x, dy, w, b, lr, ws, None, None, stride, dilation, pads,
                                       mult, lay, strategy, stream)
