"""CPU oracle for depthwise 2-D convolution (numpy-facing ctypes wrapper).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the entry module's
``smoke()`` and the CPU-baseline leg of ``bench.py`` may import this package.
It shares nothing with the HIP path (``depthwise_convolution_amd``); the only
code both sides see is the seeded input generator, which holds none of the
method's arithmetic.

The general routines (``*_general``) take explicit per-side padding
``pads = (top, bottom, left, right)`` (negative pads crop) and a channel multiplier ``mult``
(output channel ``o`` reads input channel ``o // mult``; weights
``(mult*C, kH, kW)``); ``same_pads`` and ``xla_same_pads`` give the two SAME
paddings as explicit pads.

All arithmetic is in ``dwconv_oracle.c`` (double-precision accumulation, one
output at a time, the plain definitions from the LeanMlir "Depthwise" page:
forward equation, reversed-kernel and direct input-gradient forms, stride-2 as
the even decimation of stride 1 and its zero-upsampled backward, regular
convolution for comparison, weight and bias gradients).  This module only
marshals numpy arrays.

Array shapes follow the layout: NHWC arrays are ``(N, H, W, C)``, NCHW arrays
``(N, C, H, W)``; weights are ``(C, kH, kW)`` float32 or float16.
"""
import ctypes
import os

import numpy as np

NHWC, NCHW = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdwconv_oracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i = ctypes.c_int
_vp = ctypes.c_void_p


def _configure(lib):
    lib.dwo_half_to_double.restype = ctypes.c_double
    lib.dwo_half_to_double.argtypes = [ctypes.c_uint16]
    lib.dwo_fwd.argtypes = [_f32p, _vp, _i, _vp, _f64p, _vp] + [_i] * 10
    lib.dwo_input_grad.argtypes = [_f32p, _vp, _i, _f64p, _vp] + [_i] * 10
    lib.dwo_input_grad_direct.argtypes = [_f32p, _vp, _i, _f64p] + [_i] * 9
    lib.dwo_dense_conv.argtypes = [_f32p, _f32p, _vp, _f64p] + [_i] * 10
    lib.dwo_weight_grad.argtypes = [_f32p, _f32p, _f64p, _vp] + [_i] * 10
    lib.dwo_bias_grad.argtypes = [_f32p, _f64p, _vp] + [_i] * 5
    lib.dwo_fwd_general.argtypes = [_f32p, _vp, _i, _vp, _f64p, _vp] + [_i] * 15
    lib.dwo_input_grad_general.argtypes = [_f32p, _vp, _i, _f64p, _vp] + [_i] * 15
    lib.dwo_weight_grad_general.argtypes = [_f32p, _f32p, _f64p, _vp] + [_i] * 15
    for f in ("dwo_fwd", "dwo_input_grad", "dwo_input_grad_direct",
              "dwo_dense_conv", "dwo_weight_grad", "dwo_bias_grad", "dwo_version",
              "dwo_fwd_general", "dwo_input_grad_general", "dwo_weight_grad_general"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def swap_library(path):
    """Point this module at another build of the oracle source (used by the
    test that plants mistakes in a copy of the oracle).  Returns the library
    that was active before, to be restored with ``restore_library``."""
    prev = _load()
    globals()["_lib"] = _configure(ctypes.CDLL(path))
    return prev


def restore_library(prev):
    globals()["_lib"] = prev


def out_extent(n, s):
    return (n + s - 1) // s


def _nhwc_dims(shape, layout):
    if layout == NHWC:
        n, h, w, c = shape
    else:
        n, c, h, w = shape
    return n, h, w, c


def _shape(layout, n, h, w, c):
    return (n, h, w, c) if layout == NHWC else (n, c, h, w)


def _weights(w):
    w = np.ascontiguousarray(w)
    if w.dtype == np.float16:
        return w, 1
    if w.dtype == np.float32:
        return w, 0
    raise TypeError("weights must be float32 or float16")


def _ptr(a):
    return None if a is None else a.ctypes.data


def parity_bound(S):
    """Elementwise acceptance bound for a float32 result: 1e-5*S + 1e-6,
    where S is the sum of |products| that entered the element."""
    return 1e-5 * S + 1e-6


def half_to_double(bits):
    """Decode IEEE binary16 bit patterns (uint16) to float64."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([lib.dwo_half_to_double(int(v)) for v in flat], dtype=np.float64)
    return out.reshape(np.shape(bits))


def fwd(x, w, b=None, stride=1, dilation=1, layout=NHWC, nthreads=1, with_sum=True):
    """Forward depthwise conv. Returns (y, S) as float64 (S None if not asked)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    w, wt = _weights(w)
    N, H, W, C = _nhwc_dims(x.shape, layout)
    kH, kW = w.shape[1], w.shape[2]
    assert w.shape[0] == C
    bb = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    Ho, Wo = out_extent(H, stride), out_extent(W, stride)
    y = np.empty(_shape(layout, N, Ho, Wo, C), np.float64)
    S = np.empty_like(y) if with_sum else None
    lib.dwo_fwd(x, _ptr(w), wt, _ptr(bb), y, _ptr(S), N, H, W, C, kH, kW,
                stride, dilation, layout, nthreads)
    return y, S


def input_grad(dy, w, H, W, stride=1, dilation=1, layout=NHWC, nthreads=1, with_sum=True):
    """Input gradient (reversed-kernel form). H, W are the forward input extents."""
    lib = _load()
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    w, wt = _weights(w)
    N, Ho, Wo, C = _nhwc_dims(dy.shape, layout)
    assert (Ho, Wo) == (out_extent(H, stride), out_extent(W, stride))
    kH, kW = w.shape[1], w.shape[2]
    dx = np.empty(_shape(layout, N, H, W, C), np.float64)
    S = np.empty_like(dx) if with_sum else None
    lib.dwo_input_grad(dy, _ptr(w), wt, dx, _ptr(S), N, H, W, C, kH, kW,
                       stride, dilation, layout, nthreads)
    return dx, S


def input_grad_direct(dy, w, H, W, stride=1, dilation=1, layout=NHWC):
    """Input gradient, direct sum over output positions (small inputs only)."""
    lib = _load()
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    w, wt = _weights(w)
    N, Ho, Wo, C = _nhwc_dims(dy.shape, layout)
    kH, kW = w.shape[1], w.shape[2]
    dx = np.empty(_shape(layout, N, H, W, C), np.float64)
    lib.dwo_input_grad_direct(dy, _ptr(w), wt, dx, N, H, W, C, kH, kW,
                              stride, dilation, layout)
    return dx


def dense_conv(x, wd, b=None, stride=1, dilation=1, layout=NHWC):
    """Regular convolution with a full [Co][C][kH][kW] float32 kernel."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    wd = np.ascontiguousarray(wd, dtype=np.float32)
    N, H, W, C = _nhwc_dims(x.shape, layout)
    Co, Ci, kH, kW = wd.shape
    assert Ci == C
    bb = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    Ho, Wo = out_extent(H, stride), out_extent(W, stride)
    y = np.empty(_shape(layout, N, Ho, Wo, Co), np.float64)
    lib.dwo_dense_conv(x, wd, _ptr(bb), y, N, H, W, C, Co, kH, kW,
                       stride, dilation, layout)
    return y


def weight_grad(x, dy, kH, kW, stride=1, dilation=1, layout=NHWC, nthreads=1):
    """dW[c,kh,kw] = sum over batch and output positions of x * dy. Returns (dW, S)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    N, H, W, C = _nhwc_dims(x.shape, layout)
    dw = np.empty((C, kH, kW), np.float64)
    S = np.empty_like(dw)
    lib.dwo_weight_grad(x, dy, dw, _ptr(S), N, H, W, C, kH, kW,
                        stride, dilation, layout, nthreads)
    return dw, S


def bias_grad(dy, layout=NHWC):
    """db[c] = sum over batch and positions of dy. Returns (db, S)."""
    lib = _load()
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    N, Ho, Wo, C = _nhwc_dims(dy.shape, layout)
    db = np.empty((C,), np.float64)
    S = np.empty_like(db)
    lib.dwo_bias_grad(dy, db, _ptr(S), N, Ho, Wo, C, layout)
    return db, S


# ---------------------------------------------------------------------------
# Explicit padding and channel multiplier
# ---------------------------------------------------------------------------
def same_pads(H, W, kH, kW, stride=1, dilation=1):
    """Symmetric SAME padding (the LeanMlir forward equation's p = d*(k-1)/2 on
    every side, odd kernels) as explicit (top, bottom, left, right) pads."""
    assert kH % 2 == 1 and kW % 2 == 1
    ph, pw = dilation * (kH - 1) // 2, dilation * (kW - 1) // 2
    return (ph, ph, pw, pw)


def xla_same_pads(H, W, kH, kW, stride=1, dilation=1):
    """The LeanMlir page's stride-2 XLA-SAME as explicit pads: the stride-1
    SAME result kept at the ODD positions.  Output row ho then reads input
    rows 2*ho + 1 + kh*d - p, i.e. a top pad of p - 1; a bottom pad of p
    makes the output extent floor(H/2), the number of odd positions.  (On
    even extents with at least two taps per axis this is XLA's own SAME
    padding.)  At stride 1 it is the symmetric SAME padding."""
    ph, pw = same_pads(H, W, kH, kW, 1, dilation)[0::2]
    if stride == 1:
        return (ph, ph, pw, pw)
    assert stride == 2
    return (ph - 1, ph, pw - 1, pw)


def out_extents_padded(H, W, kH, kW, stride, dilation, pads):
    """Window positions that fit the padded input along each axis."""
    t, b, l, r = pads
    Ho = (H + t + b - dilation * (kH - 1) - 1) // stride + 1
    Wo = (W + l + r - dilation * (kW - 1) - 1) // stride + 1
    return Ho, Wo


def fwd_general(x, w, b=None, stride=1, dilation=1, pads=None, mult=1, layout=NHWC,
                nthreads=1, with_sum=True):
    """Forward with explicit pads and channel multiplier.  x has C input
    channels, w is (mult*C, kH, kW), b (mult*C,) or None.  pads None means
    symmetric SAME.  Returns (y, S) with mult*C output channels."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    w, wt = _weights(w)
    N, H, W, C = _nhwc_dims(x.shape, layout)
    kH, kW = w.shape[1], w.shape[2]
    assert w.shape[0] == mult * C
    if pads is None:
        pads = same_pads(H, W, kH, kW, stride, dilation)
    Ho, Wo = out_extents_padded(H, W, kH, kW, stride, dilation, pads)
    assert Ho >= 1 and Wo >= 1
    bb = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    y = np.empty(_shape(layout, N, Ho, Wo, mult * C), np.float64)
    S = np.empty_like(y) if with_sum else None
    lib.dwo_fwd_general(x, _ptr(w), wt, _ptr(bb), y, _ptr(S), N, H, W, C, mult, kH, kW,
                        stride, dilation, pads[0], pads[2], Ho, Wo, layout, nthreads)
    return y, S


def input_grad_general(dy, w, H, W, stride=1, dilation=1, pads=None, mult=1, layout=NHWC,
                       nthreads=1, with_sum=True):
    """Input gradient of fwd_general.  H, W are the forward input extents;
    dy has mult*C channels.  Returns (dx, S) with C channels."""
    lib = _load()
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    w, wt = _weights(w)
    N, Ho, Wo, Co = _nhwc_dims(dy.shape, layout)
    assert Co % mult == 0 and w.shape[0] == Co
    C = Co // mult
    kH, kW = w.shape[1], w.shape[2]
    if pads is None:
        pads = same_pads(H, W, kH, kW, stride, dilation)
    assert (Ho, Wo) == out_extents_padded(H, W, kH, kW, stride, dilation, pads)
    dx = np.empty(_shape(layout, N, H, W, C), np.float64)
    S = np.empty_like(dx) if with_sum else None
    lib.dwo_input_grad_general(dy, _ptr(w), wt, dx, _ptr(S), N, H, W, C, mult, kH, kW,
                               stride, dilation, pads[0], pads[2], Ho, Wo, layout, nthreads)
    return dx, S


def weight_grad_general(x, dy, kH, kW, stride=1, dilation=1, pads=None, mult=1,
                        layout=NHWC, nthreads=1):
    """dW of fwd_general: (mult*C, kH, kW).  Returns (dW, S)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    N, H, W, C = _nhwc_dims(x.shape, layout)
    if pads is None:
        pads = same_pads(H, W, kH, kW, stride, dilation)
    Ho, Wo = out_extents_padded(H, W, kH, kW, stride, dilation, pads)
    assert _nhwc_dims(dy.shape, layout) == (N, Ho, Wo, mult * C)
    dw = np.empty((mult * C, kH, kW), np.float64)
    S = np.empty_like(dw)
    lib.dwo_weight_grad_general(x, dy, dw, _ptr(S), N, H, W, C, mult, kH, kW,
                                stride, dilation, pads[0], pads[2], Ho, Wo, layout, nthreads)
    return dw, S


# ---------------------------------------------------------------------------
# Epilogue fusions and the SGD step
# ---------------------------------------------------------------------------
ACT_NONE, ACT_RELU, ACT_RELU6, ACT_SILU = 0, 1, 2, 3


def _chan(v, layout, ndim=4):
    """Per-channel vector shaped to broadcast over an activation array."""
    v = np.asarray(v, np.float64)
    return v.reshape((1, 1, 1, -1)) if layout == NHWC else v.reshape((1, -1, 1, 1))


def batchnorm_act(z, bn=None, eps=1e-5, act=ACT_NONE, layout=NHWC):
    """Inference-form BatchNorm and activation applied to a convolution result
    z (float64), per output channel.  bn = (gamma, beta, mean, var) or None:
        t = (z - mean) * gamma / sqrt(var + eps) + beta
    act: ACT_NONE (t), ACT_RELU max(t, 0), ACT_RELU6 min(max(t, 0), 6),
    ACT_SILU t * sigmoid(t) = t / (1 + exp(-t)).  The LeanMlir page names
    the fused depthwise + BatchNorm codegen only; these are the textbook
    definitions of the layers of the networks it names (MobileNetV2: ReLU6,
    EfficientNet: SiLU).  Returns (y, inv) with inv = gamma / sqrt(var + eps)
    per channel (ones without BatchNorm)."""
    z = np.asarray(z, np.float64)
    if bn is not None:
        gamma, beta, mean, var = (np.asarray(v, np.float64) for v in bn)
        inv = gamma / np.sqrt(var + np.float64(np.float32(eps)))
        t = (z - _chan(mean, layout)) * _chan(inv, layout) + _chan(beta, layout)
    else:
        inv = None
        t = z
    if act == ACT_NONE:
        y = t
    elif act == ACT_RELU:
        y = np.maximum(t, 0.0)
    elif act == ACT_RELU6:
        y = np.minimum(np.maximum(t, 0.0), 6.0)
    elif act == ACT_SILU:
        with np.errstate(over="ignore"):
            y = t / (1.0 + np.exp(-t))
    else:
        raise ValueError(act)
    return y, inv


def sgd_step(w, b, dw, db, lr):
    """The LeanMlir page's SGD steps for the depthwise weights and bias:
    W - lr * dW and b - lr * db (float64)."""
    w_new = np.asarray(w, np.float64) - np.float64(np.float32(lr)) * np.asarray(dw, np.float64)
    b_new = None if b is None else (np.asarray(b, np.float64)
                                    - np.float64(np.float32(lr)) * np.asarray(db, np.float64))
    return w_new, b_new
