"""The measurement summaries of bench.py on synthetic rocprofv3 CSVs (host
only): dispatches are assigned to table rows in issue order, also when two
workloads launch the same run-time shaped kernel on the same grid; the
counter calibration uses the 256 MiB copies and not smaller copies that share
their grid; the detail table renders every row."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import depthwise_convolution_amd as dw  # noqa: E402
from depthwise_convolution_amd import workloads  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
          "Start_Timestamp", "End_Timestamp"]
WGRAD_NCHW = ("void dwconv::(anonymous namespace)::k_wgrad_tiled_nchw(float const*, float "
              "const*, float*, dwconv::(anonymous namespace)::WgradNchwArgs)")
REDUCE = ("void dwconv::(anonymous namespace)::k_wgrad_reduce<8>(float const*, float*, float*, "
          "int, int, int, float*, float*, float)")
FLUSH = "void at::native::reduce_kernel<512, 1>(at::native::ReduceOp)"
COPY = "__amd_rocclr_copyBuffer"


def _grid(wl, layout, op):
    opc = {"fwd": dw.OP_FWD, "ig": dw.OP_INPUT_GRAD, "wgrad": dw.OP_WEIGHT_GRAD}[op]
    _, grid, block = dw.dwconv2d_describe_ex(opc, wl.N, wl.H, wl.W, wl.C, wl.kH, wl.kW,
                                             wl.stride, wl.dilation, wl.pads, wl.mult, layout,
                                             0, op == "fwd")
    return grid * block


def _tiled_nhwc_name(mode):
    return ("void dwconv::(anonymous namespace)::k_tiled_nhwc<float, 3, 3, 1, 4, 32, 1, 8, 4, "
            f"{mode}, 1, 1>(float const*, void const*, float const*, float*, "
            "dwconv::(anonymous namespace)::TiledArgs, dwconv::EpiArgs)")


@pytest.fixture(scope="module")
def rows():
    """Two NCHW weight gradients that run the same run-time shaped kernel on
    the same grid, with an NHWC forward between them (as in the table)."""
    a = workloads.WORKLOADS["asr_n64_1x24x128_1x15"]
    big = workloads.WORKLOADS["large_512x512x256_3x3"]
    ga, gb = _grid(a, workloads.NCHW, "wgrad"), _grid(big, workloads.NCHW, "wgrad")
    assert ga == gb, "the case needs one kernel and one grid for both workloads"
    return a, big, ga


def test_shared_kernel_rows_are_split_by_issue_order(rows):
    a, big, g = rows
    gf = _grid(big, workloads.NHWC, "fwd")
    seq = [(WGRAD_NCHW, g, 1.0), (REDUCE, 256, 9.0), (WGRAD_NCHW, g, 1.0), (FLUSH, 512, 7.0),
           (WGRAD_NCHW, g, 1.0), (REDUCE, 256, 9.0),
           (_tiled_nhwc_name(0), gf, 5.0), (_tiled_nhwc_name(0), gf, 5.0), (FLUSH, 512, 7.0),
           (WGRAD_NCHW, g, 2.0), (REDUCE, 256, 9.0), (WGRAD_NCHW, g, 2.0)]
    order = [(a, workloads.NCHW, "wgrad"), (big, workloads.NHWC, "fwd"),
             (big, workloads.NCHW, "wgrad")]
    got = bench._assign_rows(dw, order, seq)
    assert [v for _, _, v in got] == [[1.0, 1.0, 1.0], [5.0, 5.0], [2.0, 2.0]]
    # the forward's mode is read from the template arguments: an input-gradient
    # kernel of the same shape and grid is not the forward
    seq_ig = [(_tiled_nhwc_name(1), gf, 3.0)]
    assert bench._assign_rows(dw, [(big, workloads.NHWC, "fwd")], seq_ig)[0][2] == []


def test_row_without_dispatches_takes_nothing(rows):
    a, big, g = rows
    gf = _grid(big, workloads.NHWC, "fwd")
    seq = [(_tiled_nhwc_name(0), gf, 5.0), (FLUSH, 512, 7.0), (_tiled_nhwc_name(1), gf, 3.0),
           (WGRAD_NCHW, g, 2.0)]
    order = [(big, workloads.NHWC, "fwd"), (a, workloads.NCHW, "wgrad"),
             (big, workloads.NHWC, "ig"), (big, workloads.NCHW, "wgrad")]
    got = bench._assign_rows(dw, order, seq)
    # the second row ran nothing (the next dwconv kernel is the third row's):
    # it must not skip ahead and take the last row's dispatch of the kernel
    # the two share
    assert [v for _, _, v in got] == [[5.0], [], [3.0], [2.0]]


def _write_csv(path, counter, dispatches):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, value) in enumerate(dispatches):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid,
                        "Counter_Name": counter, "Counter_Value": value,
                        "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + 500})


def test_counter_table_calibrates_on_the_large_copies(tmp_path, rows):
    _, big, _ = rows
    gf = _grid(big, workloads.NHWC, "fwd")
    alg = bench.op_bytes(big, "fwd")
    # small same-bytes copies share the big copies' grid; the big ones read
    # 128 MiB of FETCH_SIZE and write 256 MiB of WRITE_SIZE per 256 MiB copy
    fetch = [(COPY, 131072, 800.0)] * 5 + [(_tiled_nhwc_name(0), gf, alg / 2 / 1024)] * 3 + \
            [(COPY, 131072, 131072.0)] * 5
    write = [(COPY, 131072, 1600.0)] * 5 + [(_tiled_nhwc_name(0), gf, alg / 2 / 1024)] * 3 + \
            [(COPY, 131072, 262144.0)] * 5
    fc, wc = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(fc, "FETCH_SIZE", fetch)
    _write_csv(wc, "WRITE_SIZE", write)
    detail = tmp_path / "d.json"
    detail.write_text(json.dumps({"per_config": [
        {"workload": big.name, "layout": "nhwc", "op": "fwd"}]}))
    text, table, (sf, sw) = bench.counter_table(str(fc), str(wc), str(detail))
    assert sf == pytest.approx(2.0) and sw == pytest.approx(1.0)
    rec = table[(big.name, "nhwc", "fwd")]
    # read alg/2 bytes x 2.0, written alg/2 bytes x 1.0
    assert rec["hbm_bytes_per_launch"] == pytest.approx(1.5 * alg, rel=1e-6)
    assert "5 / 5 runtime copies" in text


def test_detail_table_renders_every_row(tmp_path):
    rows_ = [{"workload": "w1", "layout": "nhwc", "op": op, "kernel": "k", "us": 1.0,
              "cold_us": 2.0, "floor_us": 0.5, "bound": "hbm", "frac_of_bound": 0.5,
              "GBs": 10.0, "pct_hbm_peak": 0.1} for op in ("fwd", "ig", "wgrad")]
    rows_[0]["copy_same_bytes_us"] = 0.9
    rows_[0].update(cpu_us=100.0, cpu_threads=16, cpu_us_1thread=900.0)
    detail = tmp_path / "d.json"
    detail.write_text(json.dumps({"per_config": rows_,
                                  "launch_floor": {"empty_launch_us": 1.5, "event_pair_us": 6.0}}))
    text = bench.detail_table(str(detail))
    assert text.count("| w1 | nhwc |") == 3
    assert "100.0 (16)" in text and "Launch floor: empty kernel back to back 1.5 us" in text


def test_every_bench_row_plan_has_a_kernel_family():
    """Every plan the per-workload table runs (each workload, layout and op,
    and each kernel the strategies can select for the 7x7 windows) names a
    kernel family the trace and counter summaries know, so no row is left
    without its kernel."""
    names = set()
    for wl in workloads.WORKLOADS.values():
        for layout in (workloads.NHWC, workloads.NCHW):
            for op in bench.OPS:
                if op.startswith("wgrad") and wl.fp16_weights:
                    continue
                names.add(bench._row_matcher(dw, wl, layout, op)[0])
    for st in (dw.STRATEGY_TILED, dw.STRATEGY_STREAM, dw.STRATEGY_STREAM_PLANES,
               dw.STRATEGY_DIRECT):
        for d in (1, 2):
            for layout in (workloads.NHWC, workloads.NCHW):
                try:
                    names.add(dw.dwconv2d_describe(dw.OP_FWD, 64, 30, 19, 128, 7, 7, 1, d, layout,
                                                   strategy=st)[0])
                except dw.DwconvError:
                    pass
    missing = sorted(n for n in names if bench.kernel_family(n) is None)
    assert not missing, missing
    assert bench.kernel_family("stream_nchw_planes_s1_k7x7_d2_px5_th5_nl5_fwd_f32w") == \
        "k_stream_nchw_planes"

