"""GPU parity of the int8 KV-cache append (fattn_kv_append_int8) against the
fp32 quantiser of the oracle: codes and scales must be bit-identical (the
codes are integers decided in fp32 on both sides), positions outside the
appended range untouched, and append-then-decode equal to decoding the
oracle-quantised cache.
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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # B, T, Hkv, d, pos, cap, dtype
    (1, 1, 1, 64, 0, 1, torch.bfloat16),
    (2, 7, 3, 128, 5, 20, torch.bfloat16),
    (1, 33, 8, 128, 0, 33, torch.float32),
    (3, 100, 2, 64, 17, 200, torch.float32),
    (2, 513, 4, 128, 1000, 1600, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_kv_append_bit_exact(case, cuda_device):
    B, T, Hkv, d, pos, cap, dt = case
    _say(f"case kv append {case}")
    g = torch.Generator().manual_seed(400 + T)
    x = torch.randn(B, T, Hkv, d, generator=g) * torch.exp(torch.randn(B, T, Hkv, 1, generator=g) * 2)
    x[0, 0, 0] = 0.0                       # all-zero row
    if d > 8:
        x[-1, -1, -1, :3] = torch.tensor([1e-40, -3e-39, 2e-45])  # denormals next to ...
        x[-1, -1, -1, 3:] = 0.0                                     # ... a tiny absmax
    x = x.to(dt)
    codes0 = torch.full((B, Hkv, cap, d), 55, dtype=torch.int8)
    scales0 = torch.full((B, Hkv, cap), -2.0, dtype=torch.float32)
    c_ref, s_ref = oracle.kv_quantize_int8(x.float().numpy(), codes0.numpy().copy(), scales0.numpy().copy(),
                                           pos=pos, cap=cap)
    codes, scales = codes0.to(cuda_device), scales0.to(cuda_device)
    fa.kv_append_int8(x.to(cuda_device), codes, scales, pos=pos)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), c_ref), "codes differ from the oracle"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales differ"


def test_append_then_decode(cuda_device):
    _say("case append then decode")
    B, Hq, Hkv, Skv, d = 2, 8, 2, 700, 128
    g = torch.Generator().manual_seed(410)
    k = torch.randn(B, Skv, Hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Skv, Hkv, d, generator=g).to(torch.bfloat16)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    dev = cuda_device
    kq = torch.zeros(B, Hkv, Skv, d, dtype=torch.int8, device=dev)
    vq = torch.zeros_like(kq)
    ks = torch.zeros(B, Hkv, Skv, dtype=torch.float32, device=dev)
    vs = torch.zeros_like(ks)
    # append in three uneven pieces, as a serving loop would
    for lo, hi in ((0, 300), (300, 301), (301, Skv)):
        fa.kv_append_int8(k[:, lo:hi].contiguous().to(dev), kq, ks, pos=lo)
        fa.kv_append_int8(v[:, lo:hi].contiguous().to(dev), vq, vs, pos=lo)
    o = fa.decode_int8(q.to(dev), kq, ks, vq, vs)
    torch.cuda.synchronize()
    kq_ref, ks_ref = oracle.kv_quantize_int8(k.float().numpy())
    vq_ref, vs_ref = oracle.kv_quantize_int8(v.float().numpy())
    assert np.array_equal(kq.cpu().numpy(), kq_ref) and np.array_equal(vq.cpu().numpy(), vq_ref)
    o_ref, _ = oracle.decode_int8(q, kq_ref, ks_ref, vq_ref, vs_ref, scale=1 / math.sqrt(d))
    err = np.abs(o.float().cpu().double().numpy() - o_ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_full_size_append_sampled(cuda_device):
    # the append that fills the 32K-token cache of the decode workload, one tensor
    w = W.INT8_DECODE
    _say(f"case full-size append B{w.B} T{w.Skv} Hkv{w.Hkv} d{w.d}")
    g = torch.Generator(device=cuda_device)
    g.manual_seed(420)
    x = torch.randn(w.B, w.Skv, w.Hkv, w.d, generator=g, device=cuda_device).to(torch.bfloat16)
    codes = torch.empty(w.B, w.Hkv, w.Skv, w.d, dtype=torch.int8, device=cuda_device)
    scales = torch.empty(w.B, w.Hkv, w.Skv, dtype=torch.float32, device=cuda_device)
    fa.kv_append_int8(x, codes, scales, pos=0)
    torch.cuda.synchronize()
    # sampled sequences: every token of 3 (b, kv head) streams
    for b, h in ((0, 0), (w.B - 1, w.Hkv - 1), (7, 3)):
        xs = x[b:b + 1, :, h:h + 1].float().cpu().numpy()
        c_ref, s_ref = oracle.kv_quantize_int8(xs)
        assert np.array_equal(codes[b, h].cpu().numpy(), c_ref[0, 0])
        assert np.array_equal(scales[b, h].cpu().numpy(), s_ref[0, 0])


def test_kv_append_exact_ties_round_to_even(cuda_device):
    # rows whose absmax is 127 * 2^e make the scale exactly 2^e, so (k + 1/2) * 2^e
    # gives exact halfway quotients: each must round to the even neighbour, both signs
    _say("case kv append exact ties")
    d = 128
    rows = []
    for e in (-20, 0, 7, 60):
        k = np.arange(-63, 64, dtype=np.float64)
        ties = (k + 0.5) * 2.0 ** e
        rows.append(np.concatenate([[127.0 * 2.0 ** e], ties]))
        rows.append(np.concatenate([[-127.0 * 2.0 ** e], -ties[::-1]]))
    x = torch.tensor(np.stack(rows), dtype=torch.float32).reshape(1, len(rows), 1, d)
    c_ref, s_ref = oracle.kv_quantize_int8(x.numpy())
    ties_codes = c_ref[0, 0, 0, 1:].astype(int)
    assert np.all(ties_codes % 2 == 0)  # the oracle itself rounds every tie to even
    codes = torch.zeros(1, 1, len(rows), d, dtype=torch.int8, device=cuda_device)
    scales = torch.zeros(1, 1, len(rows), dtype=torch.float32, device=cuda_device)
    fa.kv_append_int8(x.to(cuda_device), codes, scales, pos=0)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
