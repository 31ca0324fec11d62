"""Workload table and seeded synthetic input generators.

This module holds no convolution arithmetic: it only names problem shapes and
draws random arrays.  It is the one piece of code that both the HIP path's
tests/bench and the CPU oracle's callers share.

Shapes are the ones the pages time or test: the ggml PR's perf table
(llama.cpp PR #21565, "Performance (Apple M5)": [W,H,C,N] = [19,30,128,1] 7x7,
[24,1,128,1] 1x15, [24,1,256,1] 1x31, [512,512,256,1] 3x3, [112,112,32,1] 3x3,
[56,56,128,1] 5x5), the ASR shapes and edge cases of its review thread
(dilation, prime channel count, batch > 1), the MobileNetV2 stride-2
downsampling of the LeanMlir "Depthwise" page (SAME and XLA-SAME), and the
grouped "4 => 8, groups = 4" layer of Reactant.jl issue 331 (a channel
multiplier).  No dataset stands behind any of them: every value is drawn
here.

A workload's padding is SAME (d*(k-1)/2 on every side) unless it names
explicit ``pads = (top, bottom, left, right)``; ``mult`` output channels are
computed per input channel.  The output extents below are only the sizes of
the arrays to draw (window positions that fit the padded input).

Draw order and dtype: numpy ``default_rng(seed)``, in the order x, W, b, dy,
each drawn in float64 over the logical [N, H, W, C] (or [C, kH, kW]) shape and
cast to float32; fp16 weights are rounded to float16 (round-to-nearest-even)
and the float32 weights of such a workload carry the same rounded values.
NCHW tensors are the transposes of the same logical draws, so a workload holds
the same numbers in both layouts.
"""
from dataclasses import dataclass, field
import numpy as np

NHWC, NCHW = 0, 1
LAYOUT_NAMES = {NHWC: "nhwc", NCHW: "nchw"}


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    W: int
    C: int
    kH: int
    kW: int
    stride: int = 1
    dilation: int = 1
    x_dist: str = "normal1"      # "normal1": N(0,1); "uniform1": U(-1,1)
    w_dist: str = "normal_fan"   # "normal_fan": N(0, 1/(kH*kW)); "uniform1": U(-1,1)
    dy_dist: str = "normal1"
    fp16_weights: bool = False
    bias: bool = True
    pads: tuple = None           # (top, bottom, left, right); None = SAME
    mult: int = 1                # output channels per input channel
    tags: tuple = field(default=())

    @property
    def general(self):
        """True when the workload needs the explicit-padding / multiplier form."""
        return self.pads is not None or self.mult != 1

    @property
    def Ho(self):
        if self.pads is None:
            return (self.H + self.stride - 1) // self.stride
        t, b = self.pads[0], self.pads[1]
        return (self.H + t + b - self.dilation * (self.kH - 1) - 1) // self.stride + 1

    @property
    def Wo(self):
        if self.pads is None:
            return (self.W + self.stride - 1) // self.stride
        l, r = self.pads[2], self.pads[3]
        return (self.W + l + r - self.dilation * (self.kW - 1) - 1) // self.stride + 1

    @property
    def Co(self):
        return self.mult * self.C

    @property
    def wbytes(self):
        return self.Co * self.kH * self.kW * (2 if self.fp16_weights else 4)

    def fwd_bytes(self):
        """Algorithmic bytes of one forward: x + y + W + b."""
        return (4 * self.N * self.H * self.W * self.C + 4 * self.N * self.Ho * self.Wo * self.Co
                + self.wbytes + (4 * self.Co if self.bias else 0))

    def ig_bytes(self):
        """Algorithmic bytes of one input gradient: dy + dx + W."""
        return (4 * self.N * self.Ho * self.Wo * self.Co + 4 * self.N * self.H * self.W * self.C
                + self.wbytes)

    def wgrad_bytes(self):
        """Algorithmic bytes of the weight + bias gradient: x + dy + dW + db."""
        return (4 * self.N * self.H * self.W * self.C + 4 * self.N * self.Ho * self.Wo * self.Co
                + 4 * self.Co * self.kH * self.kW + 4 * self.Co)

    def fwd_flops(self):
        return 2 * self.N * self.Ho * self.Wo * self.Co * self.kH * self.kW


def _w(name, N, H, W, C, k, **kw):
    kh, kwid = k
    return Workload(name=name, N=N, H=H, W=W, C=C, kH=kh, kW=kwid, **kw)


_U = dict(x_dist="uniform1", w_dist="uniform1", dy_dist="uniform1")

# The configurations the tests and the bench run.
WORKLOADS = {w.name: w for w in [
    _w("tiny_16x16x8_3x3", 1, 16, 16, 8, (3, 3), **_U, tags=("tiny",)),
    _w("mobilenet_112x112x32_3x3", 1, 112, 112, 32, (3, 3), tags=("target",)),
    _w("mobilenet_s2_224x224x32_3x3", 1, 224, 224, 32, (3, 3), stride=2),
    _w("effnet_n1_56x56x128_5x5", 1, 56, 56, 128, (5, 5)),
    _w("effnet_n1_56x56x128_5x5_f16w", 1, 56, 56, 128, (5, 5), fp16_weights=True),
    _w("effnet_n32_56x56x128_5x5", 32, 56, 56, 128, (5, 5)),
    _w("effnet_n32_56x56x128_5x5_f16w", 32, 56, 56, 128, (5, 5), fp16_weights=True),
    _w("asr_n1_30x19x128_7x7", 1, 30, 19, 128, (7, 7), **_U),
    _w("asr_n64_30x19x128_7x7", 64, 30, 19, 128, (7, 7), **_U),
    _w("asr_n1_30x19x128_7x7_d2", 1, 30, 19, 128, (7, 7), dilation=2, **_U),
    _w("asr_n64_30x19x128_7x7_d2", 64, 30, 19, 128, (7, 7), dilation=2, **_U),
    _w("asr_n1_1x24x128_1x15", 1, 1, 24, 128, (1, 15), **_U),
    _w("asr_n64_1x24x128_1x15", 64, 1, 24, 128, (1, 15), **_U),
    _w("asr_n1_1x24x256_1x31", 1, 1, 24, 256, (1, 31), **_U),
    _w("asr_n64_1x24x256_1x31", 64, 1, 24, 256, (1, 31), **_U),
    # the two remaining (C, kernel) pairings of the 1 x 24 rows, parity only
    _w("asr_n1_1x24x256_1x15", 1, 1, 24, 256, (1, 15), **_U, tags=("parity_only",)),
    _w("asr_n1_1x24x128_1x31", 1, 1, 24, 128, (1, 31), **_U, tags=("parity_only",)),
    # prime channel count edge case
    _w("prime_n1_30x19x131_7x7", 1, 30, 19, 131, (7, 7), **_U),
    _w("prime_n64_30x19x131_7x7", 64, 30, 19, 131, (7, 7), **_U),
    _w("prime_n1_1x24x131_1x15", 1, 1, 24, 131, (1, 15), **_U, tags=("parity_only",)),
    _w("prime_n64_1x24x131_1x15", 64, 1, 24, 131, (1, 15), **_U, tags=("parity_only",)),
    _w("large_512x512x256_3x3", 1, 512, 512, 256, (3, 3), tags=("target", "large")),
    # explicit padding: the page's stride-2 XLA-SAME (odd positions kept) on
    # the MobileNetV2 downsampling shape, and VALID (no padding) at stride 1
    _w("mobilenet_s2_xla_224x224x32_3x3", 1, 224, 224, 32, (3, 3), stride=2,
       pads=(0, 1, 0, 1), tags=("general",)),
    _w("effnet_n32_56x56x128_5x5_valid", 32, 56, 56, 128, (5, 5), pads=(0, 0, 0, 0),
       tags=("general",)),
    # channel multiplier: the Reactant.jl layer (4 => 8, groups = 4, 3x3, no
    # padding, 4x4 input) and a multiplier of 2 on the MobileNet shape
    _w("reactant_4x4x4_3x3_m2_valid", 1, 4, 4, 4, (3, 3), pads=(0, 0, 0, 0), mult=2, **_U,
       tags=("general", "parity_only")),
    _w("mobilenet_m2_112x112x32_3x3", 1, 112, 112, 32, (3, 3), mult=2, tags=("general",)),
]}


def _draw(rng, dist, shape, k=None):
    if dist == "normal1":
        return rng.standard_normal(shape)
    if dist == "uniform1":
        return rng.uniform(-1.0, 1.0, shape)
    if dist == "normal_fan":
        return rng.standard_normal(shape) / np.sqrt(k)
    if dist == "int3":
        return rng.integers(-3, 4, shape).astype(np.float64)
    if dist == "int2":
        return rng.integers(-2, 3, shape).astype(np.float64)
    raise ValueError(dist)


def to_layout(a_nhwc, layout):
    """Logical [N,H,W,C] array -> contiguous array in `layout`."""
    if layout == NHWC:
        return np.ascontiguousarray(a_nhwc)
    return np.ascontiguousarray(np.transpose(a_nhwc, (0, 3, 1, 2)))


def from_layout(a, layout):
    """Array in `layout` -> logical [N,H,W,C] view."""
    if layout == NHWC:
        return a
    return np.transpose(a, (0, 2, 3, 1))


def make_inputs(wl: Workload, layout=NHWC, seed=0, integer=False):
    """Seeded inputs of a workload: dict with x, w, b (or None), dy.

    With ``integer=True`` every value is a small integer (x, W, dy in
    {-3..3}, b in {-2..2}); then all partial sums are exact in float32.
    """
    rng = np.random.default_rng(seed)
    kk = wl.kH * wl.kW
    xs = (wl.N, wl.H, wl.W, wl.C)
    ys = (wl.N, wl.Ho, wl.Wo, wl.Co)
    ws = (wl.Co, wl.kH, wl.kW)
    if integer:
        x = _draw(rng, "int3", xs)
        w = _draw(rng, "int3", ws)
        b = _draw(rng, "int2", (wl.Co,))
        dy = _draw(rng, "int3", ys)
    else:
        x = _draw(rng, wl.x_dist, xs)
        w = _draw(rng, wl.w_dist, ws, kk)
        b = rng.uniform(-0.1, 0.1, (wl.Co,))
        dy = _draw(rng, wl.dy_dist, ys)
    x = x.astype(np.float32)
    dy = dy.astype(np.float32)
    if wl.fp16_weights:
        w = w.astype(np.float16)
    else:
        w = w.astype(np.float32)
    b = b.astype(np.float32) if wl.bias else None
    return {"x": to_layout(x, layout), "w": np.ascontiguousarray(w), "b": b,
            "dy": to_layout(dy, layout)}


def random_problem(rng, max_hw=20, max_c=13):
    """A random small problem description for sweep tests (no data)."""
    k_h = int(rng.choice([1, 3, 5, 7]))
    k_w = int(rng.choice([1, 3, 5, 7]))
    return Workload(name="rand", N=int(rng.integers(1, 3)), H=int(rng.integers(1, max_hw)),
                    W=int(rng.integers(1, max_hw)), C=int(rng.integers(1, max_c)),
                    kH=k_h, kW=k_w, stride=int(rng.integers(1, 3)),
                    dilation=int(rng.integers(1, 3)), x_dist="uniform1", w_dist="uniform1",
                    dy_dist="uniform1")
