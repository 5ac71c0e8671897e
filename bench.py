"""Benchmark of the tiled exact attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * fattn_fwd on the MHA causal prefill workload (B=2, H=32, S=4096, d=128,
    bf16), the workload the headline metric is quoted on, and
  * fattn_decode_int8 on the GQA int8-KV-cache decode workload (B=32, Hq=32,
    Hkv=8, Skv=32768, d=128).
Inputs are resident in HBM before timing starts (two copies of the 2.2 GB
decode cache, alternated from step to step, so no call finds the previous
call's cache lines in the last-level cache).  `value` is the prefill
attention throughput in TFLOP/s (4*d FLOPs per visible (query, key) pair per
query head, counted exactly); the decode leg reports HBM GB/s over its
algorithmic bytes (int8 K and V, their fp32 scales, the bf16 query and output).
Before the W warmup steps the step runs untimed for --settle-ms of wall time
(default 200 ms): the chip raises its clocks over the first tens of
milliseconds of load.  Each timed step runs the prefill launch, then the
decode call; HIP events
recorded on the launch stream (torch's current stream, which the binding
passes to libfattn) at the step and leg boundaries time each call.  The
sustained rate of K prefill launches in a row is reported beside it
(informational): with no decode between them the chip holds its matrix load
and lowers its clock.

After the timed steps, the other prefill workloads and the next rows of the
path are timed (informational), each as back-to-back calls after untimed
calls for half the settle time; under "next": the backward pass of the prefill workload,
decode over an int4 cache of the decode workload's shape, a packed
variable-length prefill, decode with per-sequence cache lengths, and the
int8 / int4 cache append of one 32K-token tensor.

The CPU baseline times the fp64 oracle on the host on a bounded sample of the
prefill workload (whole query rows of a few (batch, head) pairs).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s & % bf16 MFMA peak (prefill); HBM GB/s & % peak (decode)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)
PREFILL_KERNEL_SRC = os.path.join(ROOT, "tiled_exact_attention_amd", "csrc", "fwd_bf16.hip")
DECODE_KERNEL_SRC = os.path.join(ROOT, "tiled_exact_attention_amd", "csrc", "decode_kv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(Sq, Skv, causal, window):
    """Number of visible (query, key) pairs of one head (exact count)."""
    off = Skv - Sq
    if not causal:
        return Sq * Skv
    total = 0
    for i in range(Sq):
        hi = min(Skv, i + off + 1)
        lo = max(0, i + off - window + 1) if window else 0
        total += max(0, hi - lo)
    return total


def prefill_flops(w):
    return 4 * w.d * visible_pairs(w.Sq, w.Skv, w.causal, w.window) * w.B * w.Hq


def decode_bytes(w):
    kv = 2 * w.B * w.Hkv * w.Skv * w.d * w.bits // 8   # codes of K and V (int8 or packed int4)
    scales = 2 * w.B * w.Hkv * w.Skv * 4         # fp32 scales
    qo = 2 * w.B * w.Hq * w.d * 2                # bf16 query and output
    return kv + scales + qo


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel_src, key):
    """HBM bytes per launch measured with rocprofv3 counters, if they are current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get(f"{key}_source_sha256") != source_hash(kernel_src):
        return None  # the kernel changed since the counters were taken
    try:
        return float(vals[f"{key}_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def peak_clocks_mhz(device_index):
    """Peak shader and memory clocks from hipDeviceGetAttribute, through the HIP
    runtime this process already has loaded (attribute numbers from
    hip_runtime_api.h: hipDeviceAttributeClockRate = 5, MemoryClockRate = 60,
    both in kHz).  Empty if the runtime cannot be found."""
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    if path is None:
        return {}
    hip = ctypes.CDLL(path)
    out = {}
    for name, attr in (("peak_shader_clock_MHz", 5), ("peak_memory_clock_MHz", 60)):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(attr), ctypes.c_int(device_index)) == 0:
            out[name] = v.value / 1000
    return out


def time_cpu_baseline(w, q, k, v, budget_s):
    """Times the fp64 oracle on whole query rows of (b, h) pairs, growing the
    sample until about budget_s seconds of CPU work have been measured."""
    import numpy as np

    import oracle
    threads = oracle.max_threads(0)
    qd = q.double().numpy()
    kd = k.double().numpy()
    vd = v.double().numpy()
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    rng = np.random.default_rng(0)
    rng.shuffle(pairs)
    done_flops, elapsed, used = 0, 0.0, 0
    per_head = 4 * w.d * visible_pairs(w.Sq, w.Skv, w.causal, w.window)
    while used < len(pairs) and elapsed < budget_s:
        n = 1 if used == 0 else max(1, min(len(pairs) - used,
                                           int((budget_s - elapsed) / max(elapsed / used, 1e-9))))
        chunk = pairs[used:used + n]
        rows = np.array([(b, h, i) for b, h in chunk for i in range(w.Sq)], dtype=np.int64)
        t0 = time.perf_counter()
        oracle.fwd(qd, kd, vd, causal=w.causal, window=w.window, scale=w.scale, rows=rows,
                   threads=threads)
        elapsed += time.perf_counter() - t0
        done_flops += per_head * len(chunk)
        used += len(chunk)
    return {
        "value": round(done_flops / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{used} of {len(pairs)} (batch, head) pairs of the {w.name} workload, every "
                  f"query row, fp64 three-pass oracle; {done_flops / 1e9:.1f} GFLOP in {elapsed:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=("all", "prefill", "decode", "copy", "bwd"), default="all",
                    help="time one leg only (for profiler runs); the JSON line is then partial. "
                         "'copy' times a plain 1 GiB device-to-device copy, the known-size "
                         "reference that scales the HBM byte counters; 'bwd' times the backward "
                         "of the prefill workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--num-splits", type=int, default=0, help="decode key splits (0 = library default)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="wall time of untimed steps before the warmup steps, while the chip's clocks rise")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_exact_attention_amd as fa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / max(args.steps, 1)
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "avg_us": round(us, 2),
                          "GB/s": round(2 * n / (us * 1e-6) / 1e9, 1)}), flush=True)
        return

    wp, wd = W.MHA_CAUSAL, W.INT8_DECODE
    if args.only == "bwd":
        # the backward alone (forward once for o and lse, then K timed calls)
        q, k, v = (t.to(dev) for t in W.workload_inputs(wp))
        bdo = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(wp.seed + 100),
                          device=dev).to(torch.bfloat16)
        o, lse = fa.fwd(q, k, v, causal=wp.causal, scale=wp.scale, return_lse=True)
        bws = torch.empty((fa.fattn_bwd_workspace_size(wp.B, wp.Hq, wp.Hkv, wp.Sq, wp.Skv, wp.d),),
                          dtype=torch.uint8, device=dev)
        bout = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        call = lambda: fa.bwd(q, k, v, o, lse, bdo, causal=wp.causal, scale=wp.scale, workspace=bws, out=bout)
        settle_calls = 0
        t_end = time.perf_counter() + args.settle_ms / 1e3  # untimed, while the clocks rise
        while time.perf_counter() < t_end:
            call()
            torch.cuda.synchronize()
            settle_calls += 1
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / max(args.steps, 1)
        bflops = 2.5 * prefill_flops(wp)
        print(json.dumps({"workload": f"backward of {wp.name}", "avg_us": round(us, 2),
                          "TFLOP/s": round(bflops / (us * 1e-6) / 1e12, 2), "steps": args.steps,
                          "warmup": args.warmup, "settle": {"ms": args.settle_ms, "steps": settle_calls}}),
              flush=True)
        return
    do_prefill = args.only in ("all", "prefill")
    do_decode = args.only in ("all", "decode")

    if do_prefill:
        log(f"generating {wp.name}")
        q_cpu, k_cpu, v_cpu = W.workload_inputs(wp)
        q, k, v = q_cpu.to(dev), k_cpu.to(dev), v_cpu.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((wp.B, wp.Hq, wp.Sq), dtype=torch.float32, device=dev)
    if do_decode:
        log(f"generating {wd.name}")
        dq, dkq, dks, dvq, dvs = W.decode_workload_inputs(wd, device=dev)
        # a second copy of the cache: timed calls alternate between the two, so
        # no part of one call's cache can still sit in the last-level cache when
        # the next call reads it
        dcache = [(dkq, dks, dvq, dvs), tuple(t.clone() for t in (dkq, dks, dvq, dvs))]
        d_o = torch.empty_like(dq)
        d_lse = torch.empty((wd.B, wd.Hq), dtype=torch.float32, device=dev)
        ws = torch.empty((fa.decode_workspace_size(wd.B, wd.Hq, wd.Hkv, wd.Skv, wd.d, args.num_splits),),
                         dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def run_prefill():
        st = fa.fattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          wp.B, wp.Hq, wp.Hkv, wp.Sq, wp.Skv, wp.d, wp.scale, int(wp.causal),
                          wp.window, fa.FATTN_BF16, stream.cuda_stream)
        if st != 0:
            raise fa.FattnError(st, "fattn_fwd")

    def run_decode(step):
        ckq, cks, cvq, cvs = dcache[step % 2]
        st = fa.fattn_decode_int8(dq.data_ptr(), ckq.data_ptr(), cks.data_ptr(), cvq.data_ptr(),
                                  cvs.data_ptr(), d_o.data_ptr(), d_lse.data_ptr(), wd.B, wd.Hq,
                                  wd.Hkv, wd.Skv, wd.d, wd.scale, args.num_splits, ws.data_ptr(),
                                  ws.numel(), stream.cuda_stream)
        if st != 0:
            raise fa.FattnError(st, "fattn_decode_int8")

    # Clock settle: the chip raises its clocks over the first tens of
    # milliseconds of load (measured on MI355X: prefill launches of the step
    # take 401, 334, 304, 292 and then about 286 us per group of 10 steps
    # after process start, idle before or not), so the step runs untimed for
    # a fixed wall time before the warmup steps; the timed region is unchanged.
    settle_steps = 0
    if args.settle_ms > 0:
        log(f"settle: steps for {args.settle_ms:.0f} ms (untimed)")
        t_end = time.perf_counter() + args.settle_ms / 1e3
        while time.perf_counter() < t_end:
            for _ in range(5):
                if do_prefill:
                    run_prefill()
                if do_decode:
                    run_decode(settle_steps)
                settle_steps += 1
            torch.cuda.synchronize()

    log(f"warmup {args.warmup} steps")
    for s in range(args.warmup):
        if do_prefill:
            run_prefill()
        if do_decode:
            run_decode(s)
    torch.cuda.synchronize()

    # Timed region: K steps, each one pass of the path (the prefill launch,
    # then the decode call), with HIP events on the launch stream at the step
    # and leg boundaries (an event adds no gap between kernels on the GPU).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        if do_prefill:
            run_prefill()
        ev[s][1].record(stream)
        if do_decode:
            run_decode(s)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)]
    dec_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    pre_med, dec_med = statistics.median(pre_ms), statistics.median(dec_ms)
    log(f"prefill avg {pre_avg * 1e3:.1f} us, decode avg {dec_avg * 1e3:.1f} us, wall {wall * 1e3 / args.steps:.3f} ms/step")

    sustained_us = None
    if do_prefill and args.only == "all":
        # informational: K prefill launches back to back (no decode between
        # them): the chip then holds its matrix-core load and lowers its clock
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.steps):
            run_prefill()
        e1.record(stream)
        torch.cuda.synchronize()
        sustained_us = e0.elapsed_time(e1) * 1e3 / args.steps

    result = {
        "metric": METRIC,
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "settle": {"ms": args.settle_ms, "steps": settle_steps,
                   "note": "untimed steps before the warmup steps while the chip's clocks rise under load"},
        "config": {"workload": f"{wp.name} + {wd.name}", "prefill": {
            "B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "S": wp.Sq, "d": wp.d, "causal": wp.causal,
            "layout": "BSHD", "seed": wp.seed}, "decode": {
            "B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "Skv": wd.Skv, "d": wd.d, "kv": "int8 + fp32 scale per token/head",
            "num_splits": fa.decode_num_splits(wd.B, wd.Hq, wd.Hkv, wd.Skv, wd.d, args.num_splits),
            "seed": wd.seed}},
    }
    if do_prefill:
        flops = prefill_flops(wp)
        tflops = flops / (pre_avg * 1e-3) / 1e12
        traffic = read_traffic(PREFILL_KERNEL_SRC, "prefill")
        result["value"] = round(tflops, 2)
        result["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                              "traffic": traffic, "kernel": "fwd_bf16_kernel<128>",
                              "algorithmic_flop_per_launch": flops,
                              "avg_launch_us": round(pre_avg * 1e3, 2),
                              "median_launch_us": round(pre_med * 1e3, 2),
                              "min_launch_us": round(min(pre_ms) * 1e3, 2),
                              "timing": "HIP events on the launch stream around the prefill launch of each of "
                                        "the K steps (prefill, then decode)"}
        if sustained_us:
            result["prefill_back_to_back"] = {
                "note": "K prefill launches in a row with no decode between them (sustained matrix load; "
                        "the clock drops); informational",
                "avg_launch_us": round(sustained_us, 2),
                "TFLOP/s": round(flops / (sustained_us * 1e-6) / 1e12, 2)}
    if do_decode:
        nbytes = decode_bytes(wd)
        gbs = nbytes / (dec_avg * 1e-3) / 1e9
        result["decode"] = {"value": round(gbs, 1), "unit": "GB/s", "avg_call_us": round(dec_avg * 1e3, 2),
                            "median_call_us": round(dec_med * 1e3, 2),
                            "min_call_us": round(min(dec_ms) * 1e3, 2),
                            "timing": "HIP events around the decode call of each of the K steps (right after "
                                      "that step's prefill launch; the steps alternate two cache copies)",
                            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                         "traffic": read_traffic(DECODE_KERNEL_SRC, "decode"),
                                         "kernel": "decode_split_kernel<128, 8, true, true> (8 splits per "
                                                   "stream merged in the workgroup: one launch; "
                                                   "non-temporal cache loads)",
                                         "algorithmic_bytes_per_call": nbytes}}
        if not do_prefill:
            result["value"], result["unit"] = round(gbs, 1), "GB/s"

    if args.only == "all":
        # side context: the device and the bandwidth a plain 1 GiB device copy reaches
        props = torch.cuda.get_device_properties(dev)
        csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        for _ in range(2):
            cdst.copy_(csrc)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            cdst.copy_(csrc)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_us = c0.elapsed_time(c1) * 1e3 / 5
        result["context"] = {"device": props.name, "arch": props.gcnArchName,
                             "compute_units": props.multi_processor_count,
                             **peak_clocks_mhz(dev.index or 0),
                             "copy_1GiB_GBps_read_plus_write": round(2 * (1 << 30) / (copy_us * 1e-6) / 1e9, 1),
                             "cache_note": "prefill inputs (192 MiB) fit the 256 MB last-level cache and are "
                                           "not flushed between calls; the decode cache (2.2 GB) does not fit, "
                                           "and the timed decode calls alternate between two copies of it"}
        del csrc, cdst
        torch.cuda.empty_cache()

    def time_calls(fn, reps=10):
        """Average µs per call of fn over reps back-to-back calls, after calls
        for half the settle time (the clocks drop while the host prepares the
        inputs) and three warmup calls."""
        t_end = time.perf_counter() + args.settle_ms / 2e3
        while time.perf_counter() < t_end:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    if do_prefill and args.only == "all":
        # the other prefill workloads, informational (same kernel, same timing method)
        others = {}
        for w in (W.GQA_CAUSAL, W.MQA_CAUSAL, W.MQA_WINDOW):
            qq, kk, vv = (t.to(dev) for t in W.workload_inputs(w))
            oo = torch.empty_like(qq)
            us = time_calls(lambda: fa.fwd(qq, kk, vv, causal=w.causal, window=w.window, scale=w.scale, out=oo),
                            reps=20)
            tf = prefill_flops(w) / (us * 1e-6) / 1e12
            others[w.name] = {"us": round(us, 2), "TFLOP/s": round(tf, 2),
                              "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
            del qq, kk, vv, oo
        # long dense rows: the loop rate without the causal launch's short
        # blocks and masked tiles (informational)
        wl = W.MHA_DENSE_LONG
        qq, kk, vv = W.workload_inputs(wl, device=dev)
        oo = torch.empty_like(qq)
        us = time_calls(lambda: fa.fwd(qq, kk, vv, causal=False, scale=wl.scale, out=oo), reps=5)
        tf = prefill_flops(wl) / (us * 1e-6) / 1e12
        others[wl.name] = {"us": round(us, 2), "TFLOP/s": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                           "note": "loop rate on long unmasked rows; not a parity configuration"}
        del qq, kk, vv, oo
        result["prefill_other_workloads"] = others

    if args.only == "all":
        # next rows of the path, each timed the same way (informational)
        result["next"] = {}
        del dq, dkq, dks, dvq, dvs, dcache
        torch.cuda.empty_cache()

        def hbm_entry(workload, us, nbytes):
            return {"workload": workload, "us": round(us, 2),
                    "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                    "algorithmic_bytes": nbytes}

        # decode over the int4 cache of the same shape (two codes per byte)
        w4 = W.INT4_DECODE
        log(f"generating {w4.name}")
        q4, k4, ks4, v4, vs4 = W.decode_workload_inputs(w4, device=dev)
        o4 = torch.empty_like(q4)
        ws4 = torch.empty((fa.decode_workspace_size(w4.B, w4.Hq, w4.Hkv, w4.Skv, w4.d, 0),),
                          dtype=torch.uint8, device=dev)
        us = time_calls(lambda: fa.decode_int4(q4, k4, ks4, v4, vs4, scale=w4.scale, workspace=ws4,
                                               out=o4), reps=20)
        result["next"]["decode_int4"] = hbm_entry(w4.name, us, decode_bytes(w4))
        del q4, k4, ks4, v4, vs4, o4, ws4
        torch.cuda.empty_cache()

        # backward pass on the prefill workload (FLOPs: 2.5x the forward's, the five
        # products dV, dP, dS-recompute, dQ, dK counted once each)
        log("backward on the prefill workload")
        bdo = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(wp.seed + 100),
                          device=dev).to(torch.bfloat16)
        bws = torch.empty((fa.fattn_bwd_workspace_size(wp.B, wp.Hq, wp.Hkv, wp.Sq, wp.Skv, wp.d),),
                          dtype=torch.uint8, device=dev)
        bout = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        fa.fattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), wp.B, wp.Hq,
                     wp.Hkv, wp.Sq, wp.Skv, wp.d, wp.scale, int(wp.causal), wp.window, fa.FATTN_BF16,
                     stream.cuda_stream)
        us = time_calls(lambda: fa.bwd(q, k, v, o, lse, bdo, causal=wp.causal, scale=wp.scale,
                                       workspace=bws, out=bout), reps=10)
        bflops = 2.5 * prefill_flops(wp)
        result["next"]["bwd"] = {
            "workload": f"backward of {wp.name}", "us": round(us, 2),
            "TFLOP/s": round(bflops / (us * 1e-6) / 1e12, 2),
            "frac_bf16_peak": round(bflops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flop": bflops}
        del bdo, bws, bout

        # packed variable-length prefill (FLOPs counted per sequence, exactly)
        wv = W.VARLEN_PREFILL
        log(f"generating {wv.name}")
        vq_, vk_, vv_, vcq, vck = (t.to(dev) for t in W.varlen_workload_inputs(wv))
        vo = torch.empty_like(vq_)
        us = time_calls(lambda: fa.fwd_varlen(vq_, vk_, vv_, vcq, vck, max_seqlen_q=max(wv.lens),
                                              causal=wv.causal, scale=wv.scale, out=vo), reps=20)
        vflops = sum(4 * wv.d * visible_pairs(n, n, wv.causal, 0) * wv.Hq for n in wv.lens)
        result["next"]["prefill_varlen"] = {
            "workload": wv.name, "us": round(us, 2),
            "TFLOP/s": round(vflops / (us * 1e-6) / 1e12, 2),
            "frac_bf16_peak": round(vflops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flop": vflops}
        del vq_, vk_, vv_, vcq, vck, vo

        # decode with per-sequence lengths (bytes: only the tokens each sequence reads)
        wl = W.VARLEN_DECODE
        log(f"generating {wl.name}")
        lq, lkq, lks, lvq, lvs = W.decode_workload_inputs(wl, device=dev)
        lens = W.decode_seqlens(wl)
        lsl = lens.to(dev)
        lo = torch.empty_like(lq)
        lws = torch.empty((fa.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.Skv, wl.d, 0),),
                          dtype=torch.uint8, device=dev)
        us = time_calls(lambda: fa.decode_int8(lq, lkq, lks, lvq, lvs, scale=wl.scale, workspace=lws,
                                               out=lo, seqlens=lsl), reps=20)
        lbytes = int(lens.sum()) * wl.Hkv * (2 * wl.d + 8) + 2 * wl.B * wl.Hq * wl.d * 2
        result["next"]["decode_int8_varlen"] = hbm_entry(wl.name, us, lbytes)
        del lq, lkq, lks, lvq, lvs, lo, lws
        torch.cuda.empty_cache()

        # KV-cache append: quantise one tensor (K) of the decode workload's 32K-token cache
        g = torch.Generator(device=dev)
        g.manual_seed(wd.seed)
        xk = torch.randn(wd.B, wd.Skv, wd.Hkv, wd.d, generator=g, device=dev).to(torch.bfloat16)
        scs = torch.empty(wd.B, wd.Hkv, wd.Skv, dtype=torch.float32, device=dev)
        for bits in (8, 4):
            codes = torch.empty(wd.B, wd.Hkv, wd.Skv, wd.d * bits // 8,
                                dtype=torch.int8 if bits == 8 else torch.uint8, device=dev)
            append = fa.kv_append_int8 if bits == 8 else fa.kv_append_int4
            us = time_calls(lambda: append(xk, codes, scs, pos=0))
            nbytes = xk.numel() * 2 + codes.numel() + scs.numel() * 4
            result["next"][f"kv_append_int{bits}"] = hbm_entry(
                f"append B{wd.B} T{wd.Skv} Hkv{wd.Hkv} d{wd.d} bf16 -> int{bits} cache", us, nbytes)
            del codes
        del xk, scs

    if do_prefill and not args.no_cpu_baseline:
        log(f"cpu baseline: fp64 oracle, about {args.cpu_budget:.0f} s")
        result["cpu_baseline"] = time_cpu_baseline(wp, q_cpu, k_cpu, v_cpu, args.cpu_budget)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
