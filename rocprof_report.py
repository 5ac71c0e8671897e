"""rocprofv3 harness of libfattn: collects kernel traces and hardware counters
of the benchmark on an MI355X and reduces them to the summaries in profiles/.

    python rocprof_report.py collect DIR   # on the GPU machine: runs the passes
    python rocprof_report.py report DIR    # reads DIR's CSVs, rewrites profiles/

``collect`` runs one rocprofv3 process per pass (kernel trace, matrix-core
counters, HBM read and write counters of a plain 1 GiB copy, of the prefill
leg and of the decode leg, LDS / stall / instruction counters of the
prefill leg, then a kernel trace and the same counters of the backward),
each as a child process under its own time limit, and writes DIR/manifest.json with the exact commands, the
bench's JSON line of each pass and the hash of every kernel source.

``report`` reduces what collect left:
  * the kernel trace: dispatches, average / min / max duration of every
    libfattn kernel, grouped by kernel and grid; for the prefill and decode
    kernels of the benchmark workloads, TFLOP/s or GB/s from the average
    duration against the MI355X peaks (2.5 PFLOP/s dense bf16, 8 TB/s HBM);
  * the counters: MfmaUtil (matrix pipes busy over active cycles) and the
    bf16 matrix work executed (MfmaFlopsBF16) per kernel and grid;
  * HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
    prefill and decode kernels, each scaled by the same counter's reading
    for the copy of a known size, against the algorithmic bytes.
It writes profiles/kernels_bench_run.md, profiles/hbm_traffic.txt (read by
bench.py for roofline.traffic, keyed by kernel-source hash) and the two
headline summaries profiles/fwd_bf16_mha_causal_b2_h32_s4096_d128.md and
profiles/decode_int8_b32_hq32_hkv8_skv32768_d128.md, the prefill kernel's LDS,
stall and overlap counters (profiles/fwd_bf16_counters_mha_causal_b2_h32_s4096_d128.md)
and the backward's kernel trace, counters and HBM traffic
(profiles/bwd_mha_causal_b2_h32_s4096_d128.md).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "tiled_exact_attention_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30  # bench.py --only copy: one 1 GiB device-to-device copy per call

# (pass name, rocprofv3 options, bench.py arguments).  Counter passes stay
# within one hardware pass (FETCH_SIZE uses 3 TCC counters, WRITE_SIZE 2).
# Counter passes skip the bench's clock-settle phase (the counters are
# ratios per dispatch; under the profiler every dispatch is serialised).
BENCH_SHORT = ["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--settle-ms", "0"]
BWD_SHORT = ["--only", "bwd", "--steps", "2", "--warmup", "1", "--settle-ms", "0"]
PREFILL_SHORT = ["--only", "prefill"] + BENCH_SHORT
# SQ counters for the stall / overlap tables (at most 8 SQ and 2 GRBM per pass)
LDS_COUNTERS = ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_WAIT_INST_LDS",
                "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "GRBM_GUI_ACTIVE"]
INST_COUNTERS = ["SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                 "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]
PASSES = [
    ("trace", ["--kernel-trace", "--stats"], ["--steps", "10", "--warmup", "2", "--no-cpu-baseline"]),
    ("mfma", ["--pmc", "MfmaUtil", "MfmaFlopsBF16", "GRBM_GUI_ACTIVE"], BENCH_SHORT),
    ("fetch_copy", ["--pmc", "FETCH_SIZE"], ["--only", "copy", "--steps", "2", "--warmup", "1"]),
    ("write_copy", ["--pmc", "WRITE_SIZE"], ["--only", "copy", "--steps", "2", "--warmup", "1"]),
    ("fetch_prefill", ["--pmc", "FETCH_SIZE"], PREFILL_SHORT),
    ("write_prefill", ["--pmc", "WRITE_SIZE"], PREFILL_SHORT),
    ("fetch_decode", ["--pmc", "FETCH_SIZE"], ["--only", "decode"] + BENCH_SHORT),
    ("write_decode", ["--pmc", "WRITE_SIZE"], ["--only", "decode"] + BENCH_SHORT),
    ("lds_prefill", ["--pmc"] + LDS_COUNTERS, PREFILL_SHORT),
    ("inst_prefill", ["--pmc"] + INST_COUNTERS, PREFILL_SHORT),
    ("bwd_trace", ["--kernel-trace", "--stats"], ["--only", "bwd", "--steps", "5", "--warmup", "2"]),
    ("bwd_mfma", ["--pmc", "MfmaUtil", "MfmaFlopsBF16", "GRBM_GUI_ACTIVE"], BWD_SHORT),
    ("lds_bwd", ["--pmc"] + LDS_COUNTERS, BWD_SHORT),
    ("inst_bwd", ["--pmc"] + INST_COUNTERS, BWD_SHORT),
    ("fetch_bwd", ["--pmc", "FETCH_SIZE"], BWD_SHORT),
    ("write_bwd", ["--pmc", "WRITE_SIZE"], BWD_SHORT),
]

# The benchmark's headline kernels: the MHA causal prefill (B2 H32 S4096
# d128: 2048 blocks of 256 threads) and the int8 decode (B32 Hq32 Hkv8
# Skv32768 d128: one 512-thread workgroup per (batch, kv head)).
PREFILL_KERNEL = re.compile(r"fwd_bf16_kernel<128>")
PREFILL_GRID = 2048 * 256
DECODE_KERNEL = re.compile(r"decode_split_kernel<128, ?8, ?true, ?true>")  # varlen: <..., false>, same grid
DECODE_GRID = 32 * 8 * 512
LIBRARY_KERNEL = re.compile(r"(fwd_bf16|fwd_f32|decode_split|decode_merge|bwd_\w+|kv_quant)_kernel")


def log(msg):
    print(msg, flush=True)


def source_hashes():
    out = {}
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(path, "rb") as f:
            out[os.path.basename(path)] = hashlib.sha256(f.read()).hexdigest()[:16]
    return out


# ------------------------------------------------------------------ collect

def collect(outdir, timeout_s=300):
    os.makedirs(outdir, exist_ok=True)
    manifest = {"sources": source_hashes(), "passes": {}}
    for name, prof_opts, bench_args in PASSES:
        pdir = os.path.join(outdir, name)
        cmd = (["rocprofv3"] + prof_opts + ["--output-format", "csv", "-d", pdir, "-o", "run", "--",
                                           sys.executable, "bench.py"] + bench_args)
        log(f"pass {name}: {' '.join(cmd)}")
        t0 = time.time()
        res = subprocess.run(["timeout", "-s", "KILL", str(timeout_s)] + cmd, cwd=ROOT,
                             capture_output=True, text=True)
        lines = [l for l in res.stdout.splitlines() if l.startswith("{")]
        bench_line = json.loads(lines[-1]) if lines else None
        with open(os.path.join(outdir, f"{name}.log"), "w") as f:
            f.write(res.stdout + "\n--- stderr ---\n" + res.stderr)
        # rocprofv3 can end with a fault of its own after a complete run: the
        # pass counts when the program's own last line (the JSON) was printed
        ok = bench_line is not None
        log(f"  {name}: exit {res.returncode}, {time.time() - t0:.0f} s, "
            f"{'bench line captured' if ok else 'NO bench line'}")
        manifest["passes"][name] = {"cmd": " ".join(["rocprofv3"] + prof_opts +
                                                    ["--output-format", "csv", "-d", "<dir>", "-o", "run",
                                                     "--", "python", "bench.py"] + bench_args),
                                    "returncode": res.returncode, "bench": bench_line}
        if not ok:
            with open(os.path.join(outdir, "manifest.json"), "w") as f:
                json.dump(manifest, f, indent=1)
            raise SystemExit(f"pass {name} failed (exit {res.returncode}); see {name}.log")
    with open(os.path.join(outdir, "manifest.json"), "w") as f:
        json.dump(manifest, f, indent=1)
    log(f"collected {len(PASSES)} passes into {outdir}")


# ------------------------------------------------------------------- report

def _read_csv(pattern_dir, suffix):
    """Rows of every CSV under pattern_dir whose name ends with suffix."""
    rows = []
    for path in sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _col(row, *names):
    """Value of the first column present among names (case-insensitive)."""
    low = {k.lower(): v for k, v in row.items() if k is not None}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in columns {sorted(low)}")


def short_kernel_name(name):
    """'void fattn::(anonymous namespace)::fwd_bf16_kernel<128>(...)' -> 'fwd_bf16_kernel<128>'."""
    m = re.search(r"(\w+_kernel)(<[^()]*>)?", name)
    if not m:
        return name.strip()
    args = [a.strip() for a in (m.group(2) or "<>")[1:-1].split(",") if a.strip()]
    return m.group(1) + (f"<{', '.join(args)}>" if args else "")


def _grid(row):
    """Total work-items of a dispatch (grid size x * y * z, or Grid_Size)."""
    try:
        return int(float(_col(row, "Grid_Size")))
    except KeyError:
        x = int(float(_col(row, "Grid_Size_X")))
        y = int(float(_col(row, "Grid_Size_Y")))
        z = int(float(_col(row, "Grid_Size_Z")))
        return x * y * z


def kernel_trace(pdir):
    """{(kernel, grid): [duration_us, ...]} of libfattn dispatches, in launch order."""
    out = {}
    for row in _read_csv(pdir, "kernel_trace.csv"):
        name = _col(row, "Kernel_Name")
        if not LIBRARY_KERNEL.search(name):
            continue
        start = int(_col(row, "Start_Timestamp"))
        dur = (int(_col(row, "End_Timestamp")) - start) / 1e3
        out.setdefault((short_kernel_name(name), _grid(row)), []).append((start, dur))
    return {k: [d for _, d in sorted(v)] for k, v in out.items()}


def counters(pdir):
    """{(kernel, grid): {counter: [value per dispatch, ...]}} of libfattn dispatches."""
    per_dispatch = {}
    for row in _read_csv(pdir, "counter_collection.csv"):
        name = _col(row, "Kernel_Name")
        if not LIBRARY_KERNEL.search(name):
            continue
        key = (short_kernel_name(name), _grid(row))
        disp = _col(row, "Dispatch_Id", "Correlation_Id")
        cname = _col(row, "Counter_Name")
        per_dispatch.setdefault(key, {}).setdefault(cname, {})
        d = per_dispatch[key][cname]
        d[disp] = d.get(disp, 0.0) + float(_col(row, "Counter_Value"))
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per_dispatch.items()}


def copy_counter(pdir, counter):
    """Median per-dispatch value of a counter for the copy kernel (the only
    dispatches of the copy pass that move 1 GiB)."""
    vals = {}
    for row in _read_csv(pdir, "counter_collection.csv"):
        if _col(row, "Counter_Name") != counter:
            continue
        disp = _col(row, "Dispatch_Id", "Correlation_Id")
        vals[(_col(row, "Kernel_Name"), disp)] = vals.get((_col(row, "Kernel_Name"), disp), 0.0) + \
            float(_col(row, "Counter_Value"))
    # the copy dispatches are the ones with the largest reading
    best = max(vals.values())
    big = [v for v in vals.values() if v >= 0.5 * best]
    return statistics.median(big)


def _match(d, kernel_re, grid):
    vals = [v for (k, g), v in d.items() if kernel_re.search(k) and g == grid]
    if not vals:
        raise KeyError(f"no dispatch of {kernel_re.pattern} with grid {grid}")
    return vals[0]


def algorithmic():
    """Algorithmic FLOP of the MHA prefill and bytes of the int8 decode."""
    sys.path.insert(0, ROOT)
    import workloads as W
    from bench import decode_bytes, prefill_flops
    wp, wd = W.MHA_CAUSAL, W.INT8_DECODE
    qkvo = 4 * wp.B * wp.Sq * wp.Hq * wp.d * 2
    return prefill_flops(wp), qkvo, decode_bytes(wd)


def stall_rows(lds, inst, mfma, kernel_re):
    """Per (kernel, grid) matching kernel_re: medians over dispatches of the
    LDS, wait and instruction counters, as fractions.  GRBM_GUI_ACTIVE is
    summed over the 8 XCDs, so one XCD's active cycles are an eighth of it:
    CU-cycles = that x 256 CUs, SIMD-cycles = that x 1024 SIMDs.  The wave
    counters and SQ_ACTIVE_INST_VALU count quad-cycles."""
    rows = []
    for key in sorted(set(lds) | set(inst)):
        if not kernel_re.search(key[0]):
            continue
        m = lambda d, c: statistics.median(d[key][c]) if key in d and d[key].get(c) else None
        g_l, g_i = m(lds, "GRBM_GUI_ACTIVE"), m(inst, "GRBM_GUI_ACTIVE")
        cu = g_l / 8 * 256 if g_l else None
        simd = g_i / 8 * 1024 if g_i else None
        r = {"kernel": key[0], "grid": key[1]}
        if cu:
            r["lds_busy"] = m(lds, "SQ_LDS_IDX_ACTIVE") / cu
            r["bank_conflict"] = m(lds, "SQ_LDS_BANK_CONFLICT") / cu
            r["addr_conflict"] = m(lds, "SQ_LDS_ADDR_CONFLICT") / cu
            wc = m(lds, "SQ_WAVE_CYCLES")
            r["waves_per_cu"] = 4 * wc / cu
            r["wait_any"] = m(lds, "SQ_WAIT_ANY") / wc
            r["wait_lds"] = m(lds, "SQ_WAIT_INST_LDS") / wc
        if simd:
            r["mfma_busy"] = m(inst, "SQ_VALU_MFMA_BUSY_CYCLES") / simd
            r["valu_active"] = 4 * m(inst, "SQ_ACTIVE_INST_VALU") / simd
            nm = m(inst, "SQ_INSTS_MFMA")
            r["valu_per_mfma"] = (m(inst, "SQ_INSTS_VALU") - nm) / nm if nm else None
            r["lds_per_mfma"] = m(inst, "SQ_INSTS_LDS") / nm if nm else None
        mu = m(mfma, "MfmaUtil")
        r["mfma_util"] = mu / 100 if mu is not None else None
        rows.append(r)
    return rows


def _pct(x, digits=1):
    return "-" if x is None else f"{100 * x:.{digits}f}%"


def stall_table(rows):
    out = ["| kernel | MfmaUtil | matrix busy | VALU active | busy sum | LDS busy | bank conflicts "
           "| waves per CU | waves waiting | waiting to issue LDS | VALU / LDS instr per product |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        busy = (r["mfma_busy"] + r["valu_active"]) if "mfma_busy" in r else None
        ratio = (f"{r['valu_per_mfma']:.2f} / {r['lds_per_mfma']:.2f}"
                 if r.get("valu_per_mfma") is not None else "-")
        waves = f"{r['waves_per_cu']:.1f}" if "waves_per_cu" in r else "-"
        out.append(f"| `{r['kernel']}` | {_pct(r.get('mfma_util'))} | {_pct(r.get('mfma_busy'))} | "
                   f"{_pct(r.get('valu_active'))} | {_pct(busy)} | {_pct(r.get('lds_busy'))} | "
                   f"{_pct(r.get('bank_conflict'), 2)} | {waves} | {_pct(r.get('wait_any'))} | "
                   f"{_pct(r.get('wait_lds'))} | {ratio} |")
    return out


def report(indir, outdir=PROFILES):
    with open(os.path.join(indir, "manifest.json")) as f:
        man = json.load(f)
    passes = man["passes"]
    flops, prefill_alg_bytes, decode_alg_bytes = algorithmic()

    trace = kernel_trace(os.path.join(indir, "trace"))
    mf = counters(os.path.join(indir, "mfma"))

    # HBM traffic: copy-scaled FETCH_SIZE / WRITE_SIZE (KiB per dispatch)
    fetch_scale = COPY_BYTES / (copy_counter(os.path.join(indir, "fetch_copy"), "FETCH_SIZE") * 1024)
    write_scale = COPY_BYTES / (copy_counter(os.path.join(indir, "write_copy"), "WRITE_SIZE") * 1024)
    traffic = {}
    for leg, kre, grid in (("prefill", PREFILL_KERNEL, PREFILL_GRID), ("decode", DECODE_KERNEL, DECODE_GRID)):
        fk = statistics.median(_match(counters(os.path.join(indir, f"fetch_{leg}")), kre, grid)["FETCH_SIZE"])
        wk = statistics.median(_match(counters(os.path.join(indir, f"write_{leg}")), kre, grid)["WRITE_SIZE"])
        traffic[leg] = (fk, wk, fk * 1024 * fetch_scale + wk * 1024 * write_scale)

    os.makedirs(outdir, exist_ok=True)
    src = man["sources"]
    with open(os.path.join(outdir, "hbm_traffic.txt"), "w") as f:
        f.write("# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch),\n"
                "# each scaled by the same counter's reading for a plain 1 GiB device copy.\n"
                "# Written by: python rocprof_report.py collect <dir> && python rocprof_report.py report <dir>\n"
                "# Passes (repo root, one counter per run):\n")
        for name in ("fetch_copy", "write_copy", "fetch_prefill", "write_prefill", "fetch_decode", "write_decode"):
            f.write(f"#   {passes[name]['cmd']}\n")
        f.write(f"copy_fetch_scale: {fetch_scale:.4f}\ncopy_write_scale: {write_scale:.4f}\n")
        f.write("prefill_kernel: fwd_bf16_kernel<128> (MHA causal B2 H32 S4096 d128)\n")
        f.write(f"prefill_fetch_kib_raw: {traffic['prefill'][0]:.1f}\nprefill_write_kib_raw: {traffic['prefill'][1]:.1f}\n")
        f.write(f"prefill_hbm_bytes_per_launch: {traffic['prefill'][2]:.0f}\n")
        f.write(f"prefill_source_sha256: {src['fwd_bf16.hip']}\n")
        f.write("decode_kernels: decode_split_kernel<128, 8, true, true> (B32 Hq32 Hkv8 Skv32768 d128, merged in the "
                "workgroup, non-temporal cache loads)\n")
        f.write(f"decode_fetch_kib_raw: {traffic['decode'][0]:.1f}\ndecode_write_kib_raw: {traffic['decode'][1]:.1f}\n")
        f.write(f"decode_hbm_bytes_per_launch: {traffic['decode'][2]:.0f}\n")
        f.write(f"decode_source_sha256: {src['decode_kv.hip']}\n")

    # every libfattn kernel of the bench run: trace and matrix-core counters
    lines = ["# Kernels of one benchmark run on MI355X: durations and matrix-core utilisation", "",
             "Written by `python rocprof_report.py report <dir>` from the passes below (repo root).", "",
             f"    {passes['trace']['cmd']}", f"    {passes['mfma']['cmd']}", "",
             "Durations are from the kernel trace; `MfmaUtil` is rocprofv3's derived metric (matrix pipes "
             "busy over the kernel's active cycles, at the clock the chip ran), `MfmaFlopsBF16` the bf16 "
             "matrix work the dispatch executed.  Rows are (kernel, grid size in work-items).", "",
             "| kernel | grid | dispatches | avg us | min us | max us | MfmaUtil median | executed bf16 GFLOP |",
             "|---|---|---|---|---|---|---|---|"]
    for (k, g), durs in sorted(trace.items(), key=lambda kv: -sum(kv[1])):
        c = mf.get((k, g), {})
        mu = f"{statistics.median(c['MfmaUtil']):.1f}%" if c.get("MfmaUtil") else "-"
        fl = f"{statistics.median(c['MfmaFlopsBF16']) / 1e9:.3f}" if c.get("MfmaFlopsBF16") else "-"
        lines.append(f"| `{k}` | {g} | {len(durs)} | {statistics.mean(durs):.1f} | {min(durs):.1f} | "
                     f"{max(durs):.1f} | {mu} | {fl} |")
    with open(os.path.join(outdir, "kernels_bench_run.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # headline summaries.  The benchmark runs its settle steps, W warmup
    # steps and then its K timed steps (prefill launch, decode call) before
    # anything else; later legs reuse the same kernels and grids (back-to-back
    # prefills, the backward's forward, the varlen decode), so the timed
    # steps' dispatches are the K that follow the settle and warmup steps.
    bench = passes["trace"]["bench"] or {}
    w0 = int((bench.get("settle") or {}).get("steps", 0)) + int(bench.get("warmup", 0))
    timed = slice(w0, w0 + int(bench.get("steps", 0))) if bench.get("steps") else slice(None)
    pdur = _match(trace, PREFILL_KERNEL, PREFILL_GRID)[timed]
    pavg = statistics.mean(pdur)
    pmf = _match(mf, PREFILL_KERNEL, PREFILL_GRID) if any(
        PREFILL_KERNEL.search(k) and g == PREFILL_GRID for k, g in mf) else {}
    ptf = flops / (pavg * 1e-6) / 1e12
    fk, wk, tot = traffic["prefill"]
    with open(os.path.join(outdir, "fwd_bf16_mha_causal_b2_h32_s4096_d128.md"), "w") as f:
        f.write("# fwd_bf16_kernel<128>: MHA causal prefill, B=2, H=32, S=4096, d=128, bf16\n\n"
                "Written by `python rocprof_report.py report <dir>`.  Kernel trace (repo root):\n\n"
                f"    {passes['trace']['cmd']}\n\n"
                "| kernel | dispatches | avg us | min us | max us | TFLOP/s at avg | of 2.5 PFLOP/s |\n"
                "|---|---|---|---|---|---|---|\n"
                f"| `fwd_bf16_kernel<128>` (the bench's timed steps) | {len(pdur)} | {pavg:.1f} | {min(pdur):.1f} | {max(pdur):.1f} | "
                f"{ptf:.1f} | {ptf / PEAK_BF16_TFLOPS:.1%} |\n\n"
                f"Algorithmic work: {flops} FLOP per launch (4*d per visible query/key pair per head).\n")
        rl = bench.get("roofline", {})
        if rl:
            f.write(f"The bench line of the same run (HIP events around each launch of the timed steps): "
                    f"{rl.get('avg_launch_us')} us average per launch, {rl.get('achieved')} TFLOP/s.\n")
        if pmf.get("MfmaUtil"):
            f.write(f"\nMatrix pipes busy (MfmaUtil, median of {len(pmf['MfmaUtil'])} dispatches): "
                    f"{statistics.median(pmf['MfmaUtil']):.1f}%; executed bf16 matrix work "
                    f"{statistics.median(pmf['MfmaFlopsBF16']) / 1e9:.3f} GFLOP per launch.\n")
        f.write(f"\nHBM traffic (copy-scaled FETCH_SIZE {fk:.1f} KiB x {fetch_scale:.4f} and WRITE_SIZE "
                f"{wk:.1f} KiB x {write_scale:.4f}): {tot / 1e6:.1f} MB per launch against "
                f"{prefill_alg_bytes / 1e6:.1f} MB of algorithmic q, k, v, o ({tot / prefill_alg_bytes:.2f}x).\n")

    ddur = _match(trace, DECODE_KERNEL, DECODE_GRID)[timed]
    davg = statistics.mean(ddur)
    dgbs = decode_alg_bytes / (davg * 1e-6) / 1e9
    fk, wk, tot = traffic["decode"]
    with open(os.path.join(outdir, "decode_int8_b32_hq32_hkv8_skv32768_d128.md"), "w") as f:
        f.write("# decode_split_kernel<128, 8, true, true>: int8-cache decode, B=32, Hq=32, Hkv=8, Skv=32768, d=128\n\n"
                "One launch per call: the 8 splits of each (batch, kv head) stream are the waves of one "
                "workgroup and are merged in LDS.  Written by `python rocprof_report.py report <dir>`.  "
                "Kernel trace (repo root):\n\n"
                f"    {passes['trace']['cmd']}\n\n"
                "| kernel | dispatches | avg us | min us | max us | GB/s at avg | of 8 TB/s |\n"
                "|---|---|---|---|---|---|---|\n"
                f"| `decode_split_kernel<128, 8, true, true>` (the bench's timed steps) | {len(ddur)} | {davg:.1f} | {min(ddur):.1f} | "
                f"{max(ddur):.1f} | {dgbs:.1f} | {dgbs / PEAK_HBM_GBS:.1%} |\n\n"
                f"Algorithmic bytes: {decode_alg_bytes} per call (int8 K and V, fp32 scales, bf16 q and o).\n")
        dec = bench.get("decode", {})
        if dec:
            f.write(f"The bench line of the same run (HIP events around each call): {dec.get('avg_call_us')} us "
                    f"average per call, {dec.get('value')} GB/s.\n")
        f.write(f"\nHBM traffic (copy-scaled FETCH_SIZE {fk:.1f} KiB and WRITE_SIZE {wk:.1f} KiB): "
                f"{tot / 1e6:.1f} MB per call against {decode_alg_bytes / 1e6:.1f} MB algorithmic "
                f"({tot / decode_alg_bytes:.3f}x).\n")
    # LDS, stall and overlap counters of the prefill kernel(s)
    lds_p = counters(os.path.join(indir, "lds_prefill"))
    inst_p = counters(os.path.join(indir, "inst_prefill"))
    rows = stall_rows(lds_p, inst_p, mf, re.compile(r"fwd_bf16_kernel"))
    with open(os.path.join(outdir, "fwd_bf16_counters_mha_causal_b2_h32_s4096_d128.md"), "w") as f:
        f.write("# fwd_bf16_kernel: LDS, wave stalls and matrix / vector overlap, MI355X\n\n"
                "Written by `python rocprof_report.py report <dir>` from three counter passes of the "
                "prefill leg and the bench run's matrix-core pass (repo root):\n\n")
        for name in ("lds_prefill", "inst_prefill", "mfma"):
            f.write(f"    {passes[name]['cmd']}\n")
        f.write(f"\nMedians over dispatches; rows are (kernel, grid size in work-items), the MHA causal "
                f"B2 H32 S4096 d128 launch is grid {PREFILL_GRID}.  GRBM_GUI_ACTIVE is summed over the 8 XCDs, "
                "so one XCD's active cycles are an eighth of it: CU-cycles = that x 256, SIMD-cycles = that x "
                "1024.  Matrix busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD-cycles (the same ratio as MfmaUtil, "
                "from another pass); VALU active = 4 x SQ_ACTIVE_INST_VALU (quad-cycles) / SIMD-cycles; "
                "LDS busy and bank conflicts per CU-cycle; waves waiting and waiting to issue an LDS "
                "instruction per wave-cycle (SQ_WAIT_ANY, SQ_WAIT_INST_LDS over SQ_WAVE_CYCLES); VALU "
                "(non-matrix) and LDS instructions per matrix product from SQ_INSTS_*.  A busy sum near 100% "
                "means the matrix and vector work of a SIMD hardly overlap.\n\n")
        f.write("\n".join(stall_table(rows)) + "\n")
        f.write("\n| kernel | grid |\n|---|---|\n" + "".join(f"| `{r['kernel']}` | {r['grid']} |\n" for r in rows))

    # the backward of the MHA workload
    btrace = kernel_trace(os.path.join(indir, "bwd_trace"))
    bmf = counters(os.path.join(indir, "bwd_mfma"))
    brows = stall_rows(counters(os.path.join(indir, "lds_bwd")), counters(os.path.join(indir, "inst_bwd")),
                       bmf, re.compile(r"bwd_\w+_kernel"))
    bfe = counters(os.path.join(indir, "fetch_bwd"))
    bwr = counters(os.path.join(indir, "write_bwd"))
    bb = passes["bwd_trace"]["bench"] or {}
    b0 = int((bb.get("settle") or {}).get("steps", 0)) + int(bb.get("warmup", 0))
    bsl = slice(b0, b0 + int(bb.get("steps", 0))) if bb.get("steps") else slice(None)
    bflops = 2.5 * flops
    with open(os.path.join(outdir, "bwd_mha_causal_b2_h32_s4096_d128.md"), "w") as f:
        f.write("# Backward of the MHA causal prefill (B2 H32 S4096 d128, bf16), MI355X\n\n"
                "Written by `python rocprof_report.py report <dir>`.  Kernel trace (repo root; the "
                "backward alone after an untimed clock-settle phase, durations of the timed calls):\n\n"
                f"    {passes['bwd_trace']['cmd']}\n\n"
                "| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|\n")
        tot = 0.0
        for (k, g), durs in sorted(btrace.items(), key=lambda kv: -sum(kv[1])):
            if not k.startswith("bwd_"):
                continue
            d = durs[bsl] or durs
            tot += statistics.mean(d)
            f.write(f"| `{k}` | {len(d)} | {statistics.mean(d):.1f} | {min(d):.1f} | {max(d):.1f} |\n")
        f.write(f"\nSum of the kernels' averages: {tot:.1f} us per backward, {bflops / (tot * 1e-6) / 1e12:.1f} "
                f"TFLOP/s at 2.5x the forward's algorithmic FLOPs ({bflops / (tot * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1%} "
                "of 2.5 PFLOP/s).")
        if bb.get("avg_us"):
            f.write(f"  The bench line of the same run (HIP events around the timed calls): {bb['avg_us']} us "
                    f"per call, {bb.get('TFLOP/s')} TFLOP/s.")
        f.write("\n\nCounters (repo root, one pass each):\n\n")
        for name in ("bwd_mfma", "lds_bwd", "inst_bwd", "fetch_bwd", "write_bwd"):
            f.write(f"    {passes[name]['cmd']}\n")
        f.write("\nRatios as in `fwd_bf16_counters_mha_causal_b2_h32_s4096_d128.md`:\n\n")
        f.write("\n".join(stall_table(brows)) + "\n\n")
        f.write("HBM traffic per dispatch (copy-scaled FETCH_SIZE and WRITE_SIZE):\n\n"
                "| kernel | read MB | written MB |\n|---|---|---|\n")
        for key in sorted(set(bfe) | set(bwr)):
            if not key[0].startswith("bwd_"):
                continue
            rd = statistics.median(bfe[key]["FETCH_SIZE"]) * 1024 * fetch_scale / 1e6 if key in bfe else float("nan")
            wr = statistics.median(bwr[key]["WRITE_SIZE"]) * 1024 * write_scale / 1e6 if key in bwr else float("nan")
            f.write(f"| `{key[0]}` | {rd:.1f} | {wr:.1f} |\n")
        qkvo = prefill_alg_bytes
        f.write(f"\nAlgorithmic bytes of the backward: q, k, v, o, dO read and dq, dk, dv written, "
                f"{2 * qkvo / 1e6:.1f} MB (plus the fp32 row statistics).\n")

    log(f"wrote profiles: prefill {pavg:.1f} us ({ptf:.0f} TFLOP/s), decode {davg:.1f} us ({dgbs:.0f} GB/s), "
        f"traffic {traffic['prefill'][2] / 1e6:.1f} / {traffic['decode'][2] / 1e6:.1f} MB")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect", help="run the rocprofv3 passes (GPU machine)")
    c.add_argument("dir")
    c.add_argument("--timeout", type=int, default=300, help="seconds per pass")
    r = sub.add_parser("report", help="reduce collected CSVs into profiles/")
    r.add_argument("dir")
    r.add_argument("--out", default=PROFILES)
    a = ap.parse_args()
    if a.cmd == "collect":
        collect(a.dir, a.timeout)
    else:
        report(a.dir, a.out)


if __name__ == "__main__":
    main()
