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
DECODE = ("void fattn::(anonymous namespace)::decode_split_kernel<128, 8, true, true>"
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
    # LDS / stall / instruction counters of the prefill and of the backward's
    # kernels: GRBM_GUI_ACTIVE 8e6 summed over 8 XCDs -> 1e6 active cycles,
    # 2.56e8 CU-cycles, 1.024e9 SIMD-cycles
    cu, simd = 2.56e8, 1.024e9
    wc = 7.0 * cu / 4  # 7 waves per CU, in quad-cycles
    lds_vals = {"SQ_LDS_IDX_ACTIVE": 0.25 * cu, "SQ_LDS_BANK_CONFLICT": 0.004 * cu, "SQ_LDS_ADDR_CONFLICT": 0.0,
                "SQ_WAIT_INST_LDS": 0.08 * wc, "SQ_WAVE_CYCLES": wc, "SQ_WAIT_ANY": 0.23 * wc,
                "GRBM_GUI_ACTIVE": 8e6}
    inst_vals = {"SQ_ACTIVE_INST_VALU": 0.4 * simd / 4, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * simd,
                 "SQ_INSTS_VALU": 7.15e6, "SQ_INSTS_MFMA": 1e6, "SQ_INSTS_LDS": 1.52e6, "GRBM_GUI_ACTIVE": 8e6}
    BWD = {"pre": "void fattn::(anonymous namespace)::bwd_pre_kernel<128>(fattn::(anonymous namespace)::BwdParams)",
           "dq": "void fattn::(anonymous namespace)::bwd_dq_kernel<128>(fattn::(anonymous namespace)::BwdParams)",
           "dkdv": "void fattn::(anonymous namespace)::bwd_dkdv_kernel<128>(fattn::(anonymous namespace)::BwdParams)"}
    for pname, names, vals in (("lds_prefill", [PREFILL], lds_vals), ("inst_prefill", [PREFILL], inst_vals),
                               ("lds_bwd", list(BWD.values()), lds_vals), ("inst_bwd", list(BWD.values()), inst_vals),
                               ("bwd_mfma", list(BWD.values()), {"MfmaUtil": 35.0, "MfmaFlopsBF16": 5e11,
                                                                 "GRBM_GUI_ACTIVE": 8e6}),
                               ("fetch_bwd", list(BWD.values()), {"FETCH_SIZE": 262144.0}),
                               ("write_bwd", list(BWD.values()), {"WRITE_SIZE": 65536.0})):
        rows = []
        for j in (1, 2, 3):
            for n in names:
                rows += _counter_rows(10 * j + names.index(n), n, R.PREFILL_GRID, vals)
        _write(str(d / pname / "run_counter_collection.csv"), COUNTER_COLS, rows)
    # backward trace: 3 settle calls and 2 warmup calls (slow), then 5 timed calls
    rows, t, i = [], 10 ** 9, 0
    rows.append(_trace_row(i, PREFILL, R.PREFILL_GRID, t, 300.0, 256)); i += 1; t += 10 ** 6
    for c in range(3 + 2 + 5):
        slow = c < 5
        for n, dur in (("pre", 25.0), ("dq", 400.0), ("dkdv", 600.0)):
            rows.append(_trace_row(i, BWD[n], 524288, t, dur * (2 if slow else 1), 256)); i += 1; t += 10 ** 6
    _write(str(d / "bwd_trace" / "run_kernel_trace.csv"), TRACE_COLS, rows)
    bwd_line = {"avg_us": 1030.0, "TFLOP/s": 667.0, "steps": 5, "warmup": 2, "settle": {"ms": 200.0, "steps": 3}}
    bench_line = {"steps": steps, "warmup": warmup, "settle": {"ms": 200.0, "steps": settle},
                  "roofline": {"avg_launch_us": 301.0, "achieved": 913.0},
                  "decode": {"avg_call_us": 401.0, "value": 5524.0}}
    passes = {name: {"cmd": f"rocprofv3 ... {name}", "returncode": 0,
                     "bench": bench_line if name == "trace" else bwd_line if name == "bwd_trace" else {}}
              for name, _, _ in R.PASSES}
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


def test_report_counter_and_backward_summaries(collected, tmp_path):
    out = str(tmp_path / "profiles")
    R.report(collected, out)
    ctr = open(os.path.join(out, "fwd_bf16_counters_mha_causal_b2_h32_s4096_d128.md")).read()
    # MfmaUtil 50.0% (mfma pass), matrix busy 50.0%, VALU 40.0%, sum 90.0%, LDS 25.0%,
    # conflicts 0.40%, 7.0 waves per CU, 23.0% waiting, 8.0% on LDS, 6.15 / 1.52 per product
    assert ("| `fwd_bf16_kernel<128>` | 50.0% | 50.0% | 40.0% | 90.0% | 25.0% | 0.40% | 7.0 | 23.0% | "
            "8.0% | 6.15 / 1.52 |") in ctr
    bwd = open(os.path.join(out, "bwd_mha_causal_b2_h32_s4096_d128.md")).read()
    # the timed calls only: 600 + 400 + 25 us
    assert "| `bwd_dkdv_kernel<128>` | 5 | 600.0 | 600.0 | 600.0 |" in bwd
    assert "| `bwd_pre_kernel<128>` | 5 | 25.0 | 25.0 | 25.0 |" in bwd
    tf = 2.5 * prefill_flops(W.MHA_CAUSAL) / 1025e-6 / 1e12
    assert f"Sum of the kernels' averages: 1025.0 us per backward, {tf:.1f} TFLOP/s" in bwd
    assert "| `bwd_dkdv_kernel<128>` | 35.0% | 50.0% | 40.0% | 90.0% |" in bwd
    # 262144 KiB read x 2 (copy scale), 65536 KiB written x 1
    assert f"| `bwd_dq_kernel<128>` | {262144 * 1024 * 2 / 1e6:.1f} | {65536 * 1024 / 1e6:.1f} |" in bwd


def test_short_kernel_names():
    assert R.short_kernel_name(PREFILL) == "fwd_bf16_kernel<128>"
    assert R.short_kernel_name(DECODE) == "decode_split_kernel<128, 8, true, true>"
    assert R.short_kernel_name("void fattn::(anonymous namespace)::bwd_reduce_kernel(P, long)") == \
        "bwd_reduce_kernel"
