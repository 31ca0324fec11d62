"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU:
a flipped kernel, a dropped dilation in the padding, the odd stride phase, a
dropped bias or tap, a wrong channel, a transposed index, a broken f16
decode), builds it, and runs the pin checks of ``test_oracle_pins`` against
it.  At least one pin must fail for every mutant; the unmodified source must
pass the same checks.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dwconv_oracle.c")

# (name, old text, new text, which occurrence (0-based) or None for all)
MUTANTS = [
    ("fwd_flipped_kernel",
     "(acc_t)x[at(layout, C, H, W, n, c, hi, wi)] *\n                                        (acc_t)wtap(w, wtype, kH, kW, c, kh, kw)",
     "(acc_t)x[at(layout, C, H, W, n, c, hi, wi)] *\n                                        (acc_t)wtap(w, wtype, kH, kW, c, kH - 1 - kh, kW - 1 - kw)", 0),
    ("padding_ignores_dilation", "const int pH = d * (kH - 1) / 2, pW = d * (kW - 1) / 2;",
     "const int pH = (kH - 1) / 2, pW = (kW - 1) / 2;", None),
    ("fwd_odd_stride_phase", "const int hi = ho * s + kh * d - pH;",
     "const int hi = ho * s + (s - 1) + kh * d - pH;", 0),
    ("fwd_drops_bias", "acc_t acc = b ? (acc_t)b[c] : 0, sabs = 0;",
     "acc_t acc = 0, sabs = 0;", 0),
    ("fwd_drops_last_column_tap", "for (int kw = 0; kw < kW; ++kw) {\n                        const int wi = wo * s + kw * d - pW;",
     "for (int kw = 0; kw < kW - 1; ++kw) {\n                        const int wi = wo * s + kw * d - pW;", 0),
    ("fwd_uses_filter_of_channel_0", "wtap(w, wtype, kH, kW, c, kh, kw);",
     "wtap(w, wtype, kH, kW, 0, kh, kw);", 0),
    ("ig_kernel_not_reversed", "wtap(w, wtype, kH, kW, c, kH - 1 - kh, kW - 1 - kw)",
     "wtap(w, wtype, kH, kW, c, kh, kw)", 0),
    ("ig_odd_upsample_phase", "if (th < 0 || th >= H || th % s != 0)",
     "if (th < 0 || th >= H || th % s != s - 1)", 0),
    ("ig_wrong_tap_sign", "const int th = h + kh * d - pH;", "const int th = h - kh * d + pH;", 0),
    ("nhwc_index_h_w_transposed", "return (((size_t)n * H + h) * W + w) * C + c;",
     "return (((size_t)n * W + w) * H + h) * C + c;", 0),
    ("nchw_index_c_h_transposed", "return (((size_t)n * C + c) * H + h) * W + w;",
     "return (((size_t)n * H + h) * C + c) * W + w;", 0),
    ("half_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);", 0),
    ("half_exponent_bias", "v = ldexp((double)(1024 + f), e - 25);",
     "v = ldexp((double)(1024 + f), e - 24);", 0),
    ("half_read_as_raw_bits", "return dwo_half_to_double(((const uint16_t *)w)[i]);",
     "return (double)((const uint16_t *)w)[i];", 0),
    ("general_fwd_reads_channel_o_mod_C",
     "const int n = (int)(no / Co), o = (int)(no % Co), c = o / m;",
     "const int n = (int)(no / Co), o = (int)(no % Co), c = o % C;", 0),
    ("general_fwd_top_pad_sign", "const int hi = ho * s + kh * d - pt;",
     "const int hi = ho * s + kh * d + pt;", 0),
    ("general_fwd_left_pad_for_rows", "const int hi = ho * s + kh * d - pt;",
     "const int hi = ho * s + kh * d - pl;", 0),
    ("general_ig_odd_phase", "if (eh < 0 || eh % s != 0 || eh / s >= Ho)",
     "if (eh < 0 || eh % s != s - 1 || eh / s >= Ho)", 0),
    ("general_ig_one_replica_only", "for (int j = 0; j < m; ++j) {",
     "for (int j = 0; j < 1; ++j) {", 0),
    ("general_ig_row_bound_uses_H", "if (eh < 0 || eh % s != 0 || eh / s >= Ho)",
     "if (eh < 0 || eh % s != 0 || eh >= H)", 0),
    ("general_wgrad_reads_channel_o", "const int o = (int)(t / ((long)kH * kW)), c = o / m;",
     "const int o = (int)(t / ((long)kH * kW)), c = o % C;", 0),
    ("general_wgrad_left_pad_sign", "const int wi = wo * s + kw * d - pl;",
     "const int wi = wo * s + kw * d + pl;", 1),
    ("dense_reads_x_channel_o",
     "acc += (double)x[at(layout, C, H, W, n, c, hi, wi)] *\n                                       (double)wd[",
     "acc += (double)x[at(layout, C, H, W, n, o, hi, wi)] *\n                                       (double)wd[", 0),
    ("dense_filter_transposed", "(double)wd[(((size_t)o * C + c) * kH + kh) * kW + kw];",
     "(double)wd[(((size_t)c * Co + o) * kH + kh) * kW + kw];", 0),
    ("weight_grad_swaps_dy_index", "(double)dy[at(layout, C, Ho, Wo, n, c, ho, wo)];\n                    acc += p;",
     "(double)dy[at(layout, C, Ho, Wo, n, c, wo % Ho, ho % Wo)];\n                    acc += p;", 0),
]


def _mutate(src, old, new, which):
    assert old in src, old
    if which is None:
        return src.replace(old, new)
    parts = src.split(old)
    assert len(parts) > which + 1
    return old.join(parts[:which + 1]) + new + old.join(parts[which + 1:])


def _build(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-std=c99", "-O1", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-o", so, c, "-lm"], check=True)
    return so


def _all_pins_pass(om):
    """Run a representative selection of the pins; True if all pass."""
    import json
    checks = []
    for path in pins._golden_files():
        for layout in pins.LAYOUTS:
            checks.append(lambda p=path, l=layout: pins.test_golden_examples(om, p, l))
    checks.append(lambda: pins.test_half_decode_closed_forms(om))
    for layout in pins.LAYOUTS:
        checks.append(lambda l=layout: pins.test_dense_conv_golden(om, l))
    for case in pins.SMALL_CASES[:5]:
        for layout in pins.LAYOUTS:
            checks.append(lambda c=case, l=layout: pins.test_adjoint_identity(om, c, l))
            checks.append(lambda c=case, l=layout: pins.test_gather_equals_direct_input_grad(om, c, l))
        checks.append(lambda c=case: pins.test_layout_invariance(om, c))
    checks.append(lambda: pins.test_f16_weights_equal_f32_weights(om, pins.NHWC))
    checks.append(lambda: pins.test_delta_kernels(om, (7, 7), 2, pins.NHWC))
    checks.append(lambda: pins.test_stride2_is_even_decimation(om, (9, 7), (3, 3), 1, pins.NHWC))
    try:
        import torch  # noqa: F401
        for case in pins.SMALL_CASES[:5]:
            checks.append(lambda c=case: pins.test_matches_torch_cpu(om, c))
    except ImportError:
        pass
    from tests import test_oracle_general_pins as gp
    checks.append(lambda: gp.test_xla_same_pads_values(om))
    checks.append(lambda: gp.test_symmetric_backward_is_wrong_for_xla_forward(om))
    checks.append(lambda: gp.test_reactant_grouped_layer_shapes(om))
    for layout in pins.LAYOUTS:
        checks.append(lambda l=layout: gp.test_xla_same_stride2_is_odd_decimation(
            om, (8, 6), (3, 3), 1, l))
        checks.append(lambda l=layout: gp.test_multiplier_is_replicated_depthwise(om, 2, l))
        for case in gp.GENERAL_CASES:
            checks.append(lambda c=case, l=layout: gp.test_general_adjoint_identities(om, c, l))
    checks.append(lambda: gp.test_symmetric_pads_reduce_to_same(om, (1, 7, 6, 2, 3, 3, 2, 1),
                                                              pins.NHWC))
    try:
        import torch  # noqa: F401
        for case in gp.GENERAL_CASES:
            checks.append(lambda c=case: gp.test_general_matches_torch_cpu(om, c))
    except ImportError:
        pass
    for chk in checks:
        try:
            chk()
        except AssertionError:
            return False
    return True


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="dwo_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmodified_source_passes(workdir):
    so = _build(open(SRC).read(), workdir, "orig")
    prev = oracle.swap_library(so)
    try:
        assert _all_pins_pass(oracle)
    finally:
        oracle.restore_library(prev)


# a planted mistake may drive a pin's arithmetic to non-finite values: that is
# one of the ways it gets caught, not a problem of the test
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(workdir, mut):
    name, old, new, which = mut
    so = _build(_mutate(open(SRC).read(), old, new, which), workdir, name)
    prev = oracle.swap_library(so)
    try:
        assert not _all_pins_pass(oracle), f"mutant {name} passed every pin"
    finally:
        oracle.restore_library(prev)
