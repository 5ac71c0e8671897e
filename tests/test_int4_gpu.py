"""GPU parity of the int4 KV cache: fattn_decode_int4 against the fp64 oracle
(bf16 bounds: max-abs 2e-2 and mean-abs 2e-3 on o, max-abs 1e-3 on lse) and
fattn_kv_append_int4 bit for bit against the oracle's fp32 quantiser.

The cache packs two signed 4-bit codes per byte, element 2i in the low nibble
of byte i, one fp32 scale per (token, kv head).
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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.detach().float().cpu().double().numpy()


def _check(o_gpu, o_ref, lse_gpu, lse_ref, what):
    err = np.abs(o_gpu - o_ref)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert err.max() <= BF16_MAX, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean-abs {err.mean():.3e}"
    le = np.abs(lse_gpu - lse_ref).max()
    assert le <= BF16_LSE, f"{what}: lse max-abs {le:.3e}"
    return err.max(), err.mean()


DECODE_CASES = [
    # B, Hq, Hkv, Skv, d, num_splits
    (1, 1, 1, 1, 64, 0),
    (2, 4, 1, 7, 128, 0),
    (1, 8, 2, 64, 128, 1),
    (1, 8, 2, 65, 64, 0),
    (2, 8, 8, 1000, 128, 3),
    (1, 32, 8, 4097, 128, 0),
    (1, 20, 1, 333, 64, 4),       # 20 heads per kv head: two head chunks
    (1, 40, 2, 129, 128, 2),
    (3, 6, 3, 2050, 64, 7),
    (1, 4, 4, 999, 128, 1000),     # more splits requested than tiles
]


def _decode_case(q, kq, ks, vq, vs, num_splits, dev, scale=None):
    d = q.shape[-1]
    s = 1 / math.sqrt(d) if scale is None else scale
    o_ref, lse_ref = oracle.decode_int4(q, kq, ks, vq, vs, scale=s)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.bfloat16, device=dev)
    o, lse = fa.decode_int4(q.to(dev), kq.to(dev), ks.to(dev), vq.to(dev), vs.to(dev), scale=s,
                            num_splits=num_splits, return_lse=True, out=out)
    torch.cuda.synchronize()
    return _np64(o), o_ref, _np64(lse), lse_ref  # the argument order of _check


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c) for c in DECODE_CASES])
def test_int4_decode_odd_shapes(case, cuda_device):
    _say(f"case int4 decode {case}")
    B, Hq, Hkv, Skv, d, ns = case
    inputs = W.decode_inputs(B, Hq, Hkv, Skv, d, seed=500 + sum(case), bits=4)
    mx, mean = _check(*_decode_case(*inputs, ns, cuda_device), str(case))
    _say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_int4_decode_every_nibble_value(cuda_device):
    # random bytes: all 16 codes including -8 (which the quantiser never writes)
    _say("case int4 decode random bytes")
    B, Hq, Hkv, Skv, d = 2, 8, 2, 777, 128
    g = torch.Generator().manual_seed(510)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    kq = torch.randint(0, 256, (B, Hkv, Skv, d // 2), generator=g, dtype=torch.uint8)
    vq = torch.randint(0, 256, (B, Hkv, Skv, d // 2), generator=g, dtype=torch.uint8)
    ks = torch.rand(B, Hkv, Skv, generator=g) * 0.5 + 0.01
    vs = torch.rand(B, Hkv, Skv, generator=g) * 0.5 + 0.01
    _check(*_decode_case(q, kq, ks, vq, vs, 0, cuda_device), "random bytes")


def test_int4_decode_negative_and_zero_scale(cuda_device):
    inputs = W.decode_inputs(2, 8, 2, 300, 128, seed=511, bits=4)
    for s in (-0.15, 0.0):
        _say(f"case int4 decode scale {s}")
        _check(*_decode_case(*inputs, 0, cuda_device, scale=s), f"scale {s}")


def test_int4_split_count_does_not_change_the_result(cuda_device):
    _say("case int4 decode split invariance")
    B, Hq, Hkv, Skv, d = 2, 8, 2, 3000, 128
    q, kq, ks, vq, vs = [t.to(cuda_device) for t in W.decode_inputs(B, Hq, Hkv, Skv, d, seed=512, bits=4)]
    outs = []
    for ns in (1, 2, 5, 47):
        o, lse = fa.decode_int4(q, kq, ks, vq, vs, num_splits=ns, return_lse=True)
        outs.append((o.float(), lse))
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert float((o - outs[0][0]).abs().max()) <= 2 ** -7
        assert float((lse - outs[0][1]).abs().max()) <= 1e-4


APPEND_CASES = [
    # B, T, Hkv, d, pos, cap, dtype
    (1, 1, 1, 64, 0, 1, torch.bfloat16),
    (2, 7, 3, 128, 5, 20, torch.bfloat16),
    (1, 33, 8, 128, 0, 33, torch.float32),
    (3, 100, 2, 64, 17, 200, torch.float32),
    (2, 513, 4, 128, 1000, 1600, torch.bfloat16),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[str(c) for c in APPEND_CASES])
def test_int4_append_bit_exact(case, cuda_device):
    B, T, Hkv, d, pos, cap, dt = case
    _say(f"case int4 append {case}")
    g = torch.Generator().manual_seed(520 + T)
    x = torch.randn(B, T, Hkv, d, generator=g) * torch.exp(torch.randn(B, T, Hkv, 1, generator=g) * 2)
    x[0, 0, 0] = 0.0
    if d > 8:
        x[-1, -1, -1, :3] = torch.tensor([1e-40, -3e-39, 2e-45])
        x[-1, -1, -1, 3:] = 0.0
    x = x.to(dt)
    codes0 = torch.full((B, Hkv, cap, d // 2), 0x5A, dtype=torch.uint8)
    scales0 = torch.full((B, Hkv, cap), -2.0, dtype=torch.float32)
    c_ref, s_ref = oracle.kv_quantize_int4(x.float().numpy(), codes0.numpy().copy(),
                                           scales0.numpy().copy(), pos=pos, cap=cap)
    codes, scales = codes0.to(cuda_device), scales0.to(cuda_device)
    fa.kv_append_int4(x.to(cuda_device), codes, scales, pos=pos)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), c_ref), "codes differ from the oracle"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales differ"


def test_int4_append_exact_ties_round_to_even(cuda_device):
    # absmax 7 * 2^e makes the scale exactly 2^e: (k + 1/2) * 2^e are exact ties
    _say("case int4 append exact ties")
    d = 64
    rows = []
    half = np.arange(-6.5, 7.0, 1.0)  # -6.5 .. 6.5: every tie inside the clamp
    for e in (-30, 0, 9, 90):
        rows.append(np.concatenate([[7.0 * 2.0 ** e], np.resize(half, d - 1) * 2.0 ** e]))
        rows.append(np.concatenate([[-7.0 * 2.0 ** e], -np.resize(half, d - 1) * 2.0 ** e]))
    x = torch.tensor(np.stack(rows), dtype=torch.float32).reshape(1, len(rows), 1, d)
    c_ref, s_ref = oracle.kv_quantize_int4(x.numpy())
    codes = torch.zeros(1, 1, len(rows), d // 2, dtype=torch.uint8, device=cuda_device)
    scales = torch.zeros(1, 1, len(rows), dtype=torch.float32, device=cuda_device)
    fa.kv_append_int4(x.to(cuda_device), codes, scales, pos=0)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_int4_append_then_decode(cuda_device):
    _say("case int4 append then decode")
    B, Hq, Hkv, Skv, d = 2, 8, 2, 700, 64
    g = torch.Generator().manual_seed(530)
    k = torch.randn(B, Skv, Hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Skv, Hkv, d, generator=g).to(torch.bfloat16)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    dev = cuda_device
    kq = torch.zeros(B, Hkv, Skv, d // 2, dtype=torch.uint8, device=dev)
    vq = torch.zeros_like(kq)
    ks = torch.zeros(B, Hkv, Skv, dtype=torch.float32, device=dev)
    vs = torch.zeros_like(ks)
    for lo, hi in ((0, 300), (300, 301), (301, Skv)):
        fa.kv_append_int4(k[:, lo:hi].contiguous().to(dev), kq, ks, pos=lo)
        fa.kv_append_int4(v[:, lo:hi].contiguous().to(dev), vq, vs, pos=lo)
    o, lse = fa.decode_int4(q.to(dev), kq, ks, vq, vs, return_lse=True)
    torch.cuda.synchronize()
    kq_ref, ks_ref = oracle.kv_quantize_int4(k.float().numpy())
    vq_ref, vs_ref = oracle.kv_quantize_int4(v.float().numpy())
    assert np.array_equal(kq.cpu().numpy(), kq_ref) and np.array_equal(vq.cpu().numpy(), vq_ref)
    o_ref, lse_ref = oracle.decode_int4(q, kq_ref, ks_ref, vq_ref, vs_ref, scale=1 / math.sqrt(d))
    _check(_np64(o), o_ref, _np64(lse), lse_ref, "append then decode")
