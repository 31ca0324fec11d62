"""Maximum sizes: tensors just under the 2^31-element limit and over the tiled
kernels' 2 GiB addressing limit, checked on sampled output rows.

The GPU runs the whole problem; the oracle recomputes each sampled output row
from a crop of the input (the rows that window reads, with the crop's own
explicit pads: the image's SAME pad at an image edge, 0 inside), which is the
same sum by definition, so it can check any row of a tensor it could not
hold whole.  Inputs are drawn on the device with a seeded generator.
"""
import numpy as np
import pytest

import depthwise_convolution_amd as dw
from depthwise_convolution_amd.workloads import NHWC, NCHW

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return t


def _rows(t_, layout, r0, r1):
    """Rows [r0, r1) of an activation tensor, as a contiguous host array."""
    if layout == NHWC:
        return t_[:, r0:r1].contiguous().cpu().numpy()
    return t_[:, :, r0:r1].contiguous().cpu().numpy()


@pytest.mark.parametrize("shape,layout", [
    ((1, 2896, 2896, 256), NHWC),      # 2,147,024,896 elements: just under 2^31
    ((1, 1536, 1536, 256), NCHW),      # 2.4 GB: past the tiled kernels' 2 GiB limit
    ((1, 1536, 1536, 256), NHWC),
])
def test_max_size_sampled_rows(torch, shape, layout):
    import oracle
    N, H, W, C = shape
    k, p = 3, 1
    print(f"\n[case] max size {shape} layout={layout}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dims = (N, H, W, C) if layout == NHWC else (N, C, H, W)
    x = torch.randn(dims, device="cuda", generator=g)
    wt = (torch.randn((C, k, k), device="cuda", generator=g) / 3).contiguous()
    b = torch.rand((C,), device="cuda", generator=g) * 0.2 - 0.1
    name = dw.dwconv2d_describe(dw.OP_FWD, N, H, W, C, k, k, 1, 1, layout)[0]
    assert name.startswith("direct"), name         # beyond the tiled kernels' limit
    y = dw.fwd(x, wt, b, 1, 1, layout)
    torch.cuda.synchronize()
    w_h, b_h = wt.cpu().numpy(), b.cpu().numpy()
    rng = np.random.default_rng(11)
    samples = sorted(set([0, H - 1] + [int(r) for r in rng.integers(1, H - 1, 6)]))
    for r in samples:
        r0, r1 = max(0, r - p), min(H, r + p + 1)
        pads = (p - (r - r0), p - (r1 - 1 - r), p, p)   # SAME pad only where the crop is the edge
        xc = _rows(x, layout, r0, r1)
        ref, S = oracle.fwd_general(xc, w_h, b_h, 1, 1, pads, 1, layout, nthreads=16)
        got = _rows(y, layout, r, r + 1)
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= 1e-5 * S + 1e-6), f"row {r}: max err {err.max():.3g}"
    del y
    # the input gradient of the same size, sampled the same way (stride 1, SAME:
    # the reversed-kernel form over dy rows r-1..r+1)
    dy = x                                                # any seeded tensor of dy's shape
    dx = dw.input_grad(dy, wt, H, W, 1, 1, layout)
    torch.cuda.synchronize()
    for r in samples:
        r0, r1 = max(0, r - p), min(H, r + p + 1)
        pads = (p - (r - r0), p - (r1 - 1 - r), p, p)
        dyc = _rows(dy, layout, r0, r1)
        # dx row r of the full problem is the forward with the reversed kernel
        # over the dy crop (SAME stride 1: dx = correlation of dy with W flipped)
        wflip = np.ascontiguousarray(w_h[:, ::-1, ::-1])
        ref, S = oracle.fwd_general(dyc, wflip, None, 1, 1, pads, 1, layout, nthreads=16)
        got = _rows(dx, layout, r, r + 1)
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= 1e-5 * S + 1e-6), f"dx row {r}: max err {err.max():.3g}"
    del dx, x
    torch.cuda.empty_cache()
