"""The library keeps no state between calls: work from several streams and
several host threads at once gives bit for bit the results of the same calls
made one after another.

* Forward, decode and backward are enqueued on three non-default streams with
  no synchronisation between them, repeatedly, so their kernels overlap on the
  GPU; every output must equal the sequential run's.
* Four host threads each call the forward on their own stream with their own
  inputs (the ctypes binding releases the interpreter lock during a call), and
  each result must equal the sequential run's.
"""
from __future__ import annotations

import sys
import threading

import pytest
import torch

import tiled_exact_attention_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_overlapping_streams_give_sequential_results(cuda_device):
    _say("case concurrency: fwd, decode and bwd on three streams")
    dev = cuda_device
    q, k, v = (t.to(dev) for t in W.prefill_inputs(2, 16, 4, 1024, 1024, 128, "bf16", seed=51))
    dq_, kq, ks, vq, vs = (t.to(dev) for t in W.decode_inputs(8, 32, 8, 8192, 128, seed=52))
    bq, bk, bv = (t.to(dev) for t in W.prefill_inputs(1, 8, 2, 700, 700, 64, "bf16", seed=53))
    g = torch.Generator(device=dev).manual_seed(54)
    bdo = torch.randn(bq.shape, generator=g, device=dev).to(torch.bfloat16)
    bo, blse = fa.fwd(bq, bk, bv, causal=True, return_lse=True)

    def run_fwd():
        return fa.fwd(q, k, v, causal=True, return_lse=True)

    def run_dec():
        return fa.decode_int8(dq_, kq, ks, vq, vs, return_lse=True)

    def run_bwd():
        return fa.bwd(bq, bk, bv, bo, blse, bdo, causal=True)

    ref = [run_fwd(), run_dec(), run_bwd()]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        outs = [None, None, None]
        torch.cuda.synchronize()
        for _ in range(2):  # two rounds so later launches overlap earlier ones
            for i, (s, fn) in enumerate(zip(streams, (run_fwd, run_dec, run_bwd))):
                with torch.cuda.stream(s):
                    outs[i] = fn()
        torch.cuda.synchronize()
        for name, a, b in zip(("fwd", "decode", "bwd"), outs, ref):
            assert all(torch.equal(x, y) for x, y in zip(a, b)), f"rep {rep}: {name} differs"


def test_host_threads_give_sequential_results(cuda_device):
    _say("case concurrency: four host threads")
    dev = cuda_device
    shapes = [(1, 8, 2, 777, 777, 128, True), (2, 4, 4, 300, 500, 64, True),
              (1, 32, 8, 1024, 1024, 128, True), (3, 2, 1, 129, 129, 64, False)]
    inputs = [tuple(t.to(dev) for t in W.prefill_inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", seed=60 + i))
              for i, (B, Hq, Hkv, Sq, Skv, d, _) in enumerate(shapes)]
    ref = [fa.fwd(*x, causal=c, return_lse=True) for x, (*_, c) in zip(inputs, shapes)]
    torch.cuda.synchronize()
    results = [[] for _ in shapes]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                for _ in range(5):
                    results[i].append(fa.fwd(*inputs[i], causal=shapes[i][-1], return_lse=True))
            s.synchronize()
        except Exception as e:  # reported below with the thread's index
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, runs in enumerate(results):
        assert len(runs) == 5
        for o, lse in runs:
            assert torch.equal(o, ref[i][0]) and torch.equal(lse, ref[i][1]), f"thread {i} differs"
