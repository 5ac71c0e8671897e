"""CPU test of the rocprofv3 harness (rocprof_report.py report) on small CSVs
written here in rocprofv3's own column layout, with round numbers whose
reductions are known: copy-scaled HBM bytes, the headline kernels' average
durations over the benchmark's own launches only, TFLOP/s and GB/s against
the MI355X peaks, MfmaUtil medians, and the traffic file bench.py reads."""
from __future__ import annotations

import csv
import json
import os

import pytest

import rocprof_report as R
import workloads as W
from bench import decode_bytes, prefill_flops

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
                "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
                "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
                "Counter_Value", "Start_Timestamp", "End_Timestamp"]
PREFILL = "void fattn::(anonymous namespace)::fwd_bf16_kernel<128>(fattn::(anonymous namespace)::Params)"
DECODE = ("void fattn::(anonymous namespace)::decode_split_kernel<128, 8, true>"
          "(fattn::(anonymous namespace)::SplitParams)")
COPY = "__amd_rocclr_copyBuffer"
FILL = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char> >(int)"


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols, quoting=csv.QUOTE_NONNUMERIC)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, 0) for c in cols})


def _trace_row(i, name, grid, start_ns, dur_us, wg):
    return {"Kind": "KERNEL_DISPATCH", "Agent_Id": "Agent 1", "Dispatch_Id": i, "Kernel_Name": name,
            "Correlation_Id": i, "Start_Timestamp": start_ns, "End_Timestamp": start_ns + int(dur_us * 1000),
            "Workgroup_Size_X": wg, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1,
            "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1}


def _counter_rows(i, name, grid, counters):
    return [{"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": "Agent 1", "Grid_Size": grid,
             "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v} for c, v in counters.items()]


@pytest.fixture
def collected(tmp_path):
    d = tmp_path / "prof"
    steps, warmup, settle = 3, 1, 2
    # trace: two settle steps and one warmup step (500 us, 700 us: not timed),
    # the timed steps (300 us prefill, 400 us decode), then later legs with the
    # same kernels and grids that must not count (900 / 100 us)
    rows, t, i = [], 10 ** 9, 0
    for s in range(settle + warmup + steps):
        dp, dd = (500.0, 700.0) if s < settle + warmup else (300.0, 400.0)
        rows.append(_trace_row(i, PREFILL, R.PREFILL_GRID, t, dp, 256)); i += 1; t += 10 ** 6
        rows.append(_trace_row(i, DECODE, R.DECODE_GRID, t, dd, 512)); i += 1; t += 10 ** 6
    rows.append(_trace_row(i, PREFILL, R.PREFILL_GRID, t, 900.0, 256)); i += 1; t += 10 ** 6
    rows.append(_trace_row(i, DECODE, R.DECODE_GRID, t, 100.0, 512)); i += 1
    _write(str(d / "trace" / "run_kernel_trace.csv"), TRACE_COLS, rows)
    # matrix-core counters: MfmaUtil 40 / 50 / 60 % over three prefill dispatches
    rows = []
    for j, u in enumerate((40.0, 60.0, 50.0)):
        rows += _counter_rows(j, PREFILL, R.PREFILL_GRID,
                              {"MfmaUtil": u, "MfmaFlopsBF16": 2.8e11, "GRBM_GUI_ACTIVE": 1e6})
    _write(str(d / "mfma" / "run_counter_collection.csv"), COUNTER_COLS, rows)
    # copy: FETCH_SIZE reads half the copied bytes (scale 2), WRITE_SIZE all (scale 1);
    # the fill kernel before it moves little and is ignored
    for kind, val in (("fetch", 524288.0), ("write", 1048576.0)):
        cname = "FETCH_SIZE" if kind == "fetch" else "WRITE_SIZE"
        rows = _counter_rows(0, FILL, 1 << 26, {cname: 29.0})
        for j in (1, 2, 3):
            rows += _counter_rows(j, COPY, 131072, {cname: val})
        _write(str(d / f"{kind}_copy" / "run_counter_collection.csv"), COUNTER_COLS, rows)
    for leg, name, grid, fk, wk in (("prefill", PREFILL, R.PREFILL_GRID, 250000.0, 65536.0),
                                    ("decode", DECODE, R.DECODE_GRID, 1081344.0, 256.0)):
        for kind, cname, val in (("fetch", "FETCH_SIZE", fk), ("write", "WRITE_SIZE", wk)):
            rows = []
            for j in (1, 2, 3):
                rows += _counter_rows(j, name, grid, {cname: val})
            _write(str(d / f"{kind}_{leg}" / "run_counter_collection.csv"), COUNTER_COLS, rows)
    bench_line = {"steps": steps, "warmup": warmup, "settle": {"ms": 200.0, "steps": settle},
                  "roofline": {"avg_launch_us": 301.0, "achieved": 913.0},
                  "decode": {"avg_call_us": 401.0, "value": 5524.0}}
    passes = {name: {"cmd": f"rocprofv3 ... {name}", "returncode": 0,
                     "bench": bench_line if name == "trace" else {}} for name, _, _ in R.PASSES}
    with open(d / "manifest.json", "w") as f:
        json.dump({"sources": {"fwd_bf16.hip": "aaaa", "decode_kv.hip": "bbbb"}, "passes": passes}, f)
    return str(d)


def test_report_reduces_traces_and_counters(collected, tmp_path):
    out = str(tmp_path / "profiles")
    R.report(collected, out)
    vals = {}
    with open(os.path.join(out, "hbm_traffic.txt")) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    assert float(vals["copy_fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["copy_write_scale"]) == pytest.approx(1.0)
    assert int(vals["prefill_hbm_bytes_per_launch"]) == 250000 * 1024 * 2 + 65536 * 1024
    assert int(vals["decode_hbm_bytes_per_launch"]) == 1081344 * 1024 * 2 + 256 * 1024
    assert vals["prefill_source_sha256"] == "aaaa" and vals["decode_source_sha256"] == "bbbb"

    pre = open(os.path.join(out, "fwd_bf16_mha_causal_b2_h32_s4096_d128.md")).read()
    tflops = prefill_flops(W.MHA_CAUSAL) / 300e-6 / 1e12  # warmup and later launches are not counted
    assert "| 3 | 300.0 | 300.0 | 300.0 |" in pre
    assert f"{tflops:.1f}" in pre and f"{tflops / R.PEAK_BF16_TFLOPS:.1%}" in pre
    assert "MfmaUtil, median of 3 dispatches): 50.0%" in pre
    dec = open(os.path.join(out, "decode_int8_b32_hq32_hkv8_skv32768_d128.md")).read()
    gbs = decode_bytes(W.INT8_DECODE) / 400e-6 / 1e9
    assert "| 3 | 400.0 | 400.0 | 400.0 |" in dec and f"{gbs:.1f}" in dec
    table = open(os.path.join(out, "kernels_bench_run.md")).read()
    assert "| `fwd_bf16_kernel<128>` | 524288 | 7 |" in table  # every dispatch in the overall table
    assert "| 50.0% | 280.000 |" in table


def test_short_kernel_names():
    assert R.short_kernel_name(PREFILL) == "fwd_bf16_kernel<128>"
    assert R.short_kernel_name(DECODE) == "decode_split_kernel<128, 8, true>"
    assert R.short_kernel_name("void fattn::(anonymous namespace)::bwd_reduce_kernel(P, long)") == \
        "bwd_reduce_kernel"
