"""Entry points captured in a HIP graph (torch.cuda.CUDAGraph) replay correctly.

The library only launches kernels on the caller's stream (no allocation, no
memset, no synchronisation), so its calls can be captured.  Two graphs:

* a decode step as a serving loop runs it: append the new token's K and V to
  the int8 (or int4) cache at a fixed position, then decode over the cache with
  per-sequence lengths read from a device tensor;
* a training step's attention: forward with lse, then the backward.

Each graph is replayed several times; before each replay new inputs are
written into its static buffers by ordinary eager work, and after it the
outputs (and the updated caches) must equal, bit for bit, the same calls made
eagerly on copies of the same state.
"""
from __future__ import annotations

import sys

import pytest
import torch

import tiled_exact_attention_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("bits", [8, 4])
def test_decode_step_graph(bits, cuda_device):
    _say(f"case graph decode step int{bits}")
    dev = cuda_device
    B, Hq, Hkv, cap, d, pos = 4, 16, 4, 3000, 128, 2500
    q0, kq, ks, vq, vs = (t.to(dev) for t in W.decode_inputs(B, Hq, Hkv, cap, d, seed=41, bits=bits))
    append = fa.kv_append_int8 if bits == 8 else fa.kv_append_int4
    decode = fa.decode_int8 if bits == 8 else fa.decode_int4
    g = torch.Generator(device=dev).manual_seed(42)

    q = q0.clone()
    xk = torch.empty(B, 1, Hkv, d, dtype=torch.bfloat16, device=dev)
    xv = torch.empty_like(xk)
    seqlens = torch.tensor([pos + 1, 1000, pos + 1, 7], dtype=torch.int32, device=dev)
    ws = torch.empty(fa.decode_workspace_size(B, Hq, Hkv, cap, d), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)

    def step(q, kq, ks, vq, vs, out, ws):
        append(xk, kq, ks, pos=pos)
        append(xv, vq, vs, pos=pos)
        decode(q, kq, ks, vq, vs, out=out, workspace=ws, seqlens=seqlens)

    xk.normal_(generator=g)
    xv.normal_(generator=g)
    step(q, kq, ks, vq, vs, out, ws)  # eager warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(q, kq, ks, vq, vs, out, ws)
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        # new token, new query, and a length that changes between replays
        xk.copy_(torch.randn(xk.shape, generator=g, device=dev).to(torch.bfloat16))
        xv.copy_(torch.randn(xv.shape, generator=g, device=dev).to(torch.bfloat16))
        q.copy_(torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16))
        seqlens[1] = 1000 + 300 * r
        state = [t.clone() for t in (kq, ks, vq, vs)]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_out = torch.empty_like(out)
        ref_ws = torch.empty_like(ws)
        step(q, *state, ref_out, ref_ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: decode output differs from the eager step"
        for a, b, n in zip((kq, ks, vq, vs), state, ("k codes", "k scales", "v codes", "v scales")):
            assert torch.equal(a, b), f"replay {r}: {n} differ from the eager step"
        assert bool(torch.isfinite(out.float()).all())


def test_fwd_bwd_graph(cuda_device):
    _say("case graph fwd + bwd")
    dev = cuda_device
    B, Hq, Hkv, S, d = 2, 8, 2, 700, 128
    q, k, v = (t.to(dev) for t in W.prefill_inputs(B, Hq, Hkv, S, S, d, "bf16", seed=43))
    g = torch.Generator(device=dev).manual_seed(44)
    do = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
    o = torch.empty_like(q)
    bws = torch.empty(fa.fattn_bwd_workspace_size(B, Hq, Hkv, S, S, d), dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))

    def step(q, k, v, do, o, grads):
        _, lse = fa.fwd(q, k, v, causal=True, window=300, return_lse=True, out=o)
        fa.bwd(q, k, v, o, lse, do, causal=True, window=300, workspace=bws, out=grads)

    step(q, k, v, do, o, grads)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(q, k, v, do, o, grads)
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        for t in (q, k, v, do):
            t.copy_(torch.randn(t.shape, generator=g, device=dev).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_o = torch.empty_like(o)
        ref_grads = tuple(torch.empty_like(t) for t in grads)
        step(q, k, v, do, ref_o, ref_grads)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), f"replay {r}: forward output differs from the eager step"
        for a, b, n in zip(grads, ref_grads, ("dq", "dk", "dv")):
            assert torch.equal(a, b), f"replay {r}: {n} differs from the eager step"
