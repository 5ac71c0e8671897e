"""Every entry point runs on the caller's stream, in order with the work
queued before it there.

Each call is made on a fresh non-default stream whose inputs only become
valid late: the stream first runs a short GPU spin (torch's sleep kernel,
a bounded wait), then copies the real inputs over buffers filled with
poison (NaN, zero codes, zero lengths), then calls the library.  A launch
on any other stream (the null stream, a stream of the library's own) would
run before the copies and read poison; the results are compared bit for bit
with the same call made on the default stream.
"""
from __future__ import annotations

import sys

import pytest
import torch

import tiled_exact_attention_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 50_000_000  # well above launch latency; ends on its own


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _poison_like(t):
    if t.dtype.is_floating_point:
        return torch.full_like(t, float("nan"))
    return torch.zeros_like(t)


def _late(fn, inputs):
    """fn(*inputs) on a side stream whose input buffers are filled only after a spin."""
    bufs = [_poison_like(t) for t in inputs]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
        for b, t in zip(bufs, inputs):
            b.copy_(t)
        out = fn(*bufs)
    s.synchronize()
    torch.cuda.synchronize()
    return out


def _same(a, b, what):
    a = a if isinstance(a, (tuple, list)) else (a,)
    b = b if isinstance(b, (tuple, list)) else (b,)
    for x, y in zip(a, b):
        assert torch.equal(x, y), f"{what}: result differs from the default-stream call"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_on_caller_stream(dtype, cuda_device):
    _say(f"case stream fwd {dtype}")
    B, Hq, Hkv, S, d = (1, 8, 2, 600, 128) if dtype == "bf16" else (1, 2, 2, 130, 64)
    q, k, v = (t.to(cuda_device) for t in W.prefill_inputs(B, Hq, Hkv, S, S, d, dtype, seed=31))
    fn = lambda q, k, v: fa.fwd(q, k, v, causal=True, return_lse=True)
    ref = fn(q, k, v)
    _same(_late(fn, [q, k, v]), ref, f"fwd {dtype}")


def test_fwd_varlen_on_caller_stream(cuda_device):
    _say("case stream fwd_varlen")
    lens = (100, 300, 1)
    q, k, v, cq, ck = W.varlen_inputs(lens, lens, 8, 2, 128, "bf16", seed=32)
    q, k, v, cq, ck = (t.to(cuda_device) for t in (q, k, v, cq, ck))
    fn = lambda q, k, v, cq, ck: fa.fwd_varlen(q, k, v, cq, ck, max_seqlen_q=max(lens), causal=True,
                                               return_lse=True)
    ref = fn(q, k, v, cq, ck)
    _same(_late(fn, [q, k, v, cq, ck]), ref, "fwd_varlen")


def test_bwd_on_caller_stream(cuda_device):
    _say("case stream bwd")
    B, Hq, Hkv, S, d = 1, 4, 2, 300, 128
    q, k, v = (t.to(cuda_device) for t in W.prefill_inputs(B, Hq, Hkv, S, S, d, "bf16", seed=33))
    g = torch.Generator(device=cuda_device).manual_seed(34)
    do = torch.randn(q.shape, generator=g, device=cuda_device).to(torch.bfloat16)
    o, lse = fa.fwd(q, k, v, causal=True, return_lse=True)
    fn = lambda q, k, v, o, lse, do: fa.bwd(q, k, v, o, lse, do, causal=True)
    ref = fn(q, k, v, o, lse, do)
    _same(_late(fn, [q, k, v, o, lse, do]), ref, "bwd")


@pytest.mark.parametrize("bits", [8, 4])
def test_decode_on_caller_stream(bits, cuda_device):
    _say(f"case stream decode int{bits}")
    B, Hq, Hkv, Skv, d = 3, 8, 2, 2000, 128
    ins = [t.to(cuda_device) for t in W.decode_inputs(B, Hq, Hkv, Skv, d, seed=35, bits=bits)]
    sl = torch.tensor([2000, 17, 1234], dtype=torch.int32, device=cuda_device)
    dec = fa.decode_int8 if bits == 8 else fa.decode_int4
    fn = lambda q, kq, ks, vq, vs: dec(q, kq, ks, vq, vs, return_lse=True)
    _same(_late(fn, ins), fn(*ins), f"decode int{bits}")
    fnv = lambda q, kq, ks, vq, vs, sl: dec(q, kq, ks, vq, vs, return_lse=True, seqlens=sl)
    _same(_late(fnv, ins + [sl]), fnv(*ins, sl), f"decode int{bits} varlen")


@pytest.mark.parametrize("bits", [8, 4])
def test_kv_append_on_caller_stream(bits, cuda_device):
    _say(f"case stream kv_append int{bits}")
    B, T, Hkv, d, cap, pos = 2, 100, 2, 128, 300, 37
    g = torch.Generator(device=cuda_device).manual_seed(36)
    x = torch.randn(B, T, Hkv, d, generator=g, device=cuda_device).to(torch.bfloat16)
    append = fa.kv_append_int8 if bits == 8 else fa.kv_append_int4

    def fn(x):
        codes = torch.zeros(B, Hkv, cap, d * bits // 8, dtype=torch.int8 if bits == 8 else torch.uint8,
                            device=x.device)
        scales = torch.zeros(B, Hkv, cap, dtype=torch.float32, device=x.device)
        append(x, codes, scales, pos=pos)
        return codes, scales

    _same(_late(fn, [x]), fn(x), f"kv_append int{bits}")
