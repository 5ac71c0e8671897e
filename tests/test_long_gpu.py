"""GPU parity at long context: sequence lengths far beyond the benchmark
workloads (64K to 256K keys for prefill, 2^20 cached tokens for decode).

These exercise what short cases cannot: thousands of key tiles per query
block (long online-softmax chains, many lazy rescales), the causal and
window tile ranges far from the origin, 64-bit element offsets, split plans
over a million-token cache and a single split that walks all of it.  Rows are
sampled (first/last positions, tile edges, random) and computed one by one by
the fp64 oracle, which visits only each row's visible keys; the backward
case compares one whole (batch, kv head) group under a sliding window.

Bounds as in the other parity tests: bf16 max-abs 2e-2 and mean-abs 2e-3 on
o, max-abs 1e-3 on lse; gradients relative to their own scale (2^-6 of the
max, 2^-7 of the rms).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 1e-3
GRAD_MAX_REL, GRAD_MEAN_REL = 2.0 ** -6, 2.0 ** -7
GRAD_MAX_ABS, GRAD_MEAN_ABS = 1e-4, 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.detach().float().cpu().double().numpy()


def _check(o, o_ref, lse, lse_ref, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    assert err.max() <= BF16_MAX, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean-abs {err.mean():.3e}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: lse finiteness differs"
    if fin.any():
        le = np.abs(lse[fin] - lse_ref[fin]).max()
        assert le <= BF16_LSE, f"{what}: lse max-abs {le:.3e}"
    return err.max(), err.mean()


def _rows(B, Hq, Sq, n, seed):
    """(b, h, i): first/last positions, tile edges near the start and the end, random rows."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, 63, 64, 127, 128, 4095, 4096, Sq // 3, Sq // 2, Sq - 129, Sq - 128, Sq - 65,
             Sq - 64, Sq - 2, Sq - 1]
    rows = [(rng.integers(B), rng.integers(Hq), i) for i in edges if 0 <= i < Sq]
    rows += [(rng.integers(B), h, rng.integers(Sq)) for h in range(Hq)]
    while len(rows) < n:
        rows.append((rng.integers(B), rng.integers(Hq), rng.integers(Sq)))
    return np.array(rows, dtype=np.int64)


LONG_PREFILL = [
    # B, Hq, Hkv, Sq, Skv, d, causal, window
    (1, 8, 2, 65536, 65536, 128, True, 0),         # GQA causal, 1024 key tiles on the last rows
    (1, 16, 1, 131072, 131072, 64, True, 4096),    # MQA, window far from the origin
    (1, 4, 4, 300, 262144, 128, True, 0),          # a chunk at the end of a 256K context
    (1, 2, 1, 2048, 131072, 64, False, 0),         # no mask, 2048 tiles per row
]


@pytest.mark.parametrize("case", LONG_PREFILL, ids=[str(c) for c in LONG_PREFILL])
def test_long_prefill_sampled(case, cuda_device):
    B, Hq, Hkv, Sq, Skv, d, causal, window = case
    _say(f"case long prefill {case}")
    seed = 900 + Sq % 97 + Hq
    q, k, v = W.prefill_inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", seed=seed)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = q.to(cuda_device), k.to(cuda_device), v.to(cuda_device)
    o = torch.full_like(qd, float("nan"))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, window=window, scale=scale, return_lse=True, out=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "non-finite (or unwritten) output"
    vmax = v.float().abs().amax().item()
    assert float(o.float().abs().amax()) <= vmax * (1 + 2 ** -7) + 1e-6
    rows = _rows(B, Hq, Sq, 192, seed)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal=causal, window=window, scale=scale, rows=rows)
    o_np, l_np = _np64(o), lse.cpu().double().numpy()
    o_got = np.stack([o_np[b, i, h] for b, h, i in rows])
    l_got = np.array([l_np[b, h, i] for b, h, i in rows])
    mx, mean = _check(o_got, o_ref, l_got, lse_ref, str(case))
    _say(f"  sampled {len(rows)} rows: max-abs {mx:.3e} mean-abs {mean:.3e}")


LONG_DECODE = [
    # B, Hq, Hkv, Skv, d, bits, num_splits
    (1, 16, 2, 1 << 20, 128, 8, 0),
    (1, 16, 2, 1 << 20, 128, 4, 0),
    (1, 8, 1, 1 << 20, 128, 8, 1),     # one split walks the whole million-token cache
    (2, 8, 8, (1 << 19) + 77, 64, 8, 0),
]


@pytest.mark.parametrize("case", LONG_DECODE, ids=[str(c) for c in LONG_DECODE])
def test_long_decode(case, cuda_device):
    B, Hq, Hkv, Skv, d, bits, ns = case
    _say(f"case long decode {case}")
    q, kq, ks, vq, vs = W.decode_inputs(B, Hq, Hkv, Skv, d, seed=950 + bits + ns, device=cuda_device,
                                        bits=bits)
    scale = 1 / math.sqrt(d)
    fn = fa.decode_int8 if bits == 8 else fa.decode_int4
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device=cuda_device)
    o, lse = fn(q, kq, ks, vq, vs, scale=scale, num_splits=ns, return_lse=True, out=out)
    torch.cuda.synchronize()
    ref = oracle.decode_int8 if bits == 8 else oracle.decode_int4
    o_ref, lse_ref = ref(*(t.cpu() for t in (q, kq, ks, vq, vs)), scale=scale)
    mx, mean = _check(_np64(o), o_ref, _np64(lse), lse_ref, str(case))
    _say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_long_decode_varlen(cuda_device):
    # capacity 2^20; lengths at capacity, one token, a tile boundary and a ragged length
    B, Hq, Hkv, Skv, d = 4, 8, 2, 1 << 20, 128
    lens = (Skv, 1, 1 << 16, 777_777)
    _say(f"case long decode varlen lens {lens}")
    q, kq, ks, vq, vs = W.decode_inputs(B, Hq, Hkv, Skv, d, seed=960, device=cuda_device)
    sl = torch.tensor(lens, dtype=torch.int32)
    scale = 1 / math.sqrt(d)
    o, lse = fa.decode_int8(q, kq, ks, vq, vs, scale=scale, return_lse=True, seqlens=sl.to(cuda_device))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_int8(*(t.cpu() for t in (q, kq, ks, vq, vs)), scale=scale,
                                        seqlens=sl.numpy())
    mx, mean = _check(_np64(o), o_ref, _np64(lse), lse_ref, "long decode varlen")
    _say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_long_varlen_prefill_sampled(cuda_device):
    # one 64K-token sequence packed between short ones, GQA causal
    lens = (3, 65536, 1, 3001)
    Hq, Hkv, d = 8, 2, 128
    _say(f"case long varlen prefill lens {lens}")
    q, k, v, cu_q, cu_k = W.varlen_inputs(lens, lens, Hq, Hkv, d, "bf16", seed=970)
    scale = 1 / math.sqrt(d)
    dev = cuda_device
    o, lse = fa.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev),
                           max_seqlen_q=max(lens), causal=True, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(970)
    total = int(cu_q[-1])
    big0 = int(cu_q[1])
    idx = ([int(c) for c in cu_q[:-1]] + [int(c) - 1 for c in cu_q[1:]] +
           [big0 + 64, big0 + 65535 - 64] + list(rng.integers(0, total, 40)))
    rows = np.array([(rng.integers(Hq), i) for i in idx], dtype=np.int64)
    o_ref, lse_ref = oracle.fwd_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), causal=True,
                                       scale=scale, rows=rows)
    o_np, l_np = _np64(o), lse.cpu().double().numpy()
    o_got = np.stack([o_np[i, h] for h, i in rows])
    l_got = np.array([l_np[h, i] for h, i in rows])
    mx, mean = _check(o_got, o_ref, l_got, lse_ref, "long varlen prefill")
    _say(f"  sampled {len(rows)} rows: max-abs {mx:.3e} mean-abs {mean:.3e}")


def _check_grad(g, ref, what):
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    err = np.abs(g - ref)
    mx_ref = np.abs(ref).max()
    rms = math.sqrt(float((ref ** 2).mean()))
    assert err.max() <= GRAD_MAX_REL * mx_ref + GRAD_MAX_ABS, f"{what}: max {err.max():.3e} (ref {mx_ref:.3e})"
    assert err.mean() <= GRAD_MEAN_REL * rms + GRAD_MEAN_ABS, f"{what}: mean {err.mean():.3e} (rms {rms:.3e})"
    return err.max() / max(mx_ref, 1e-30), err.mean() / max(rms, 1e-30)


def test_long_bwd_window(cuda_device):
    # 32K tokens, a 512-key window: every key tile range is far from the origin
    B, Hq, Hkv, S, d, window = 1, 2, 1, 32768, 128, 512
    _say(f"case long bwd S {S} window {window}")
    q, k, v = W.prefill_inputs(B, Hq, Hkv, S, S, d, "bf16", seed=980)
    g = torch.Generator().manual_seed(981)
    do = torch.randn(B, S, Hq, d, generator=g).to(torch.bfloat16)
    scale = 1 / math.sqrt(d)
    dev = cuda_device
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=True, window=window, scale=scale, return_lse=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=True, window=window, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(q, k, v, do, causal=True, window=window, scale=scale)
    res = [_check_grad(_np64(a), r, n) for n, a, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))]
    _say("  rel max/mean: " + " ".join(f"{m:.2e}/{e:.2e}" for m, e in res))
