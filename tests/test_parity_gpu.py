"""GPU parity: libfattn (through its C ABI) against the fp64 oracle.

Small and odd shapes are compared element by element over every output
(outputs NaN-poisoned, so every element must be written); the full-size
workloads are compared over every element in test_full_size_gpu.py.

Tolerances (fixed for this build): fp32 inputs max-abs 1e-5 on o and lse;
bf16 inputs max-abs 2e-2 and mean-abs 2e-3 on o, max-abs 1e-3 on lse.  The
decode output is bf16 and uses the bf16 bounds.
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

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.detach().float().cpu().double().numpy()


def _check_bf16(o_gpu, o_ref, lse_gpu, lse_ref, what):
    err = np.abs(o_gpu - o_ref)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert err.max() <= BF16_MAX, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean-abs {err.mean():.3e}"
    if lse_ref is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse_gpu)), f"{what}: lse finiteness differs"
        if fin.any():
            le = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
            assert le <= BF16_LSE, f"{what}: lse max-abs {le:.3e}"
    return err.max(), err.mean()


def _run_fwd(q, k, v, causal, window, scale, dev):
    o = torch.full_like(q, float("nan"), device=dev)  # poison: every element must be written
    o, lse = fa.fwd(q, k, v, causal=causal, window=window, scale=scale, return_lse=True, out=o)
    torch.cuda.synchronize()
    return o, lse


# ----------------------------------------------------------------- fp32 path

F32_CASES = [
    # B, Hq, Hkv, Sq, Skv, d, causal, window, scale
    (1, 2, 2, 1, 1, 64, False, 0, None),
    (2, 4, 2, 17, 17, 64, True, 0, None),
    (1, 3, 1, 129, 129, 128, True, 0, None),
    (1, 2, 1, 65, 200, 64, True, 0, None),
    (1, 2, 2, 200, 65, 128, True, 0, None),
    (1, 4, 4, 127, 127, 64, True, 5, None),
    (1, 2, 1, 100, 100, 128, False, 0, -0.3),
    (1, 2, 2, 70, 70, 64, True, 1000, 0.0),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[str(c) for c in F32_CASES])
def test_fp32_odd_shapes(case, cuda_device):
    B, Hq, Hkv, Sq, Skv, d, causal, window, scale = case
    _say(f"case fp32 {case}")
    g = torch.Generator().manual_seed(100 + sum(case[:6]))
    q = torch.randn(B, Sq, Hq, d, generator=g)
    k = torch.randn(B, Skv, Hkv, d, generator=g)
    v = torch.randn(B, Skv, Hkv, d, generator=g)
    s = 1 / math.sqrt(d) if scale is None else scale
    o_ref, lse_ref = oracle.fwd(q, k, v, causal=causal, window=window, scale=s)
    o, lse = _run_fwd(q.to(cuda_device), k.to(cuda_device), v.to(cuda_device), causal, window, s,
                      cuda_device)
    o, lse = _np64(o), _np64(lse)
    assert np.all(np.isfinite(o))
    assert np.abs(o - o_ref).max() <= F32_TOL
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= F32_TOL if fin.any() else True


# ----------------------------------------------------------------- bf16 path

BF16_CASES = [
    # B, Hq, Hkv, Sq, Skv, d, causal, window, scale
    (1, 1, 1, 1, 1, 64, False, 0, None),
    (1, 2, 2, 17, 17, 128, True, 0, None),
    (2, 4, 4, 128, 128, 128, True, 0, None),
    (1, 2, 2, 129, 129, 64, True, 0, None),
    (1, 2, 2, 300, 300, 128, False, 0, None),
    (1, 8, 2, 257, 257, 128, True, 0, None),      # GQA G=4
    (1, 16, 2, 100, 100, 64, True, 0, None),      # GQA G=8
    (1, 29, 1, 70, 70, 64, True, 0, None),        # odd group (G=29 -> 1 head per chunk)
    (1, 232, 1, 40, 40, 64, True, 0, None),       # MQA, 232 heads
    (1, 64, 1, 20, 20, 128, True, 0, None),       # 32-head chunks
    (1, 6, 3, 97, 250, 128, True, 0, None),       # Sq < Skv (continuation)
    (1, 2, 1, 250, 97, 64, True, 0, None),        # Sq > Skv: leading rows see nothing
    (1, 4, 2, 333, 333, 128, True, 63, None),     # window
    (1, 8, 1, 300, 300, 64, True, 1, None),       # window of one key
    (1, 2, 2, 200, 200, 128, True, 512, None),    # window >= S
    (1, 4, 2, 150, 150, 64, True, 0, -0.2),       # negative scale
    (1, 2, 2, 90, 90, 128, True, 0, 0.0),         # zero scale: uniform rows
    (2, 8, 8, 64, 1000, 64, False, 0, None),      # non-causal, long keys
    (1, 8, 2, 300, 900, 128, True, 200, None),    # window + continuation + GQA
    (1, 4, 1, 513, 513, 64, True, 130, None),     # window over several tiles, G = 4
    (2, 2, 2, 1030, 1030, 128, True, 257, None),  # long band: masked edges, unmasked pairs between
]


@pytest.mark.parametrize("case", BF16_CASES, ids=[str(c) for c in BF16_CASES])
def test_bf16_odd_shapes(case, cuda_device):
    B, Hq, Hkv, Sq, Skv, d, causal, window, scale = case
    _say(f"case bf16 {case}")
    q, k, v = W.prefill_inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", seed=200 + sum(case[:6]))
    s = 1 / math.sqrt(d) if scale is None else scale
    o_ref, lse_ref = oracle.fwd(q, k, v, causal=causal, window=window, scale=s)
    o, lse = _run_fwd(q.to(cuda_device), k.to(cuda_device), v.to(cuda_device), causal, window, s,
                      cuda_device)
    mx, mean = _check_bf16(_np64(o), o_ref, _np64(lse), lse_ref, str(case))
    _say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


# -------------------------------------------------------------------- decode

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


def _decode_case(B, Hq, Hkv, Skv, d, num_splits, seed, dev, scale=None):
    q, kq, ks, vq, vs = W.decode_inputs(B, Hq, Hkv, Skv, d, seed=seed)
    s = 1 / math.sqrt(d) if scale is None else scale
    o_ref, lse_ref = oracle.decode_int8(q, kq, ks, vq, vs, scale=s)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    o, lse = fa.decode_int8(q.to(dev), kq.to(dev), ks.to(dev), vq.to(dev), vs.to(dev), scale=s,
                            num_splits=num_splits, return_lse=True, out=out)
    torch.cuda.synchronize()
    return _np64(o), _np64(lse), o_ref, lse_ref


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c) for c in DECODE_CASES])
def test_decode_odd_shapes(case, cuda_device):
    _say(f"case decode {case}")
    o, lse, o_ref, lse_ref = _decode_case(*case, seed=300 + sum(case), dev=cuda_device)
    mx, mean = _check_bf16(o, o_ref, lse, lse_ref, str(case))
    _say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_decode_negative_and_zero_scale(cuda_device):
    for s in (-0.15, 0.0):
        _say(f"case decode scale {s}")
        o, lse, o_ref, lse_ref = _decode_case(2, 8, 2, 300, 128, 0, seed=7, dev=cuda_device, scale=s)
        _check_bf16(o, o_ref, lse, lse_ref, f"scale {s}")


def test_decode_split_count_does_not_change_the_result(cuda_device):
    _say("case decode split invariance")
    B, Hq, Hkv, Skv, d = 2, 8, 2, 3000, 128
    q, kq, ks, vq, vs = [t.to(cuda_device) for t in W.decode_inputs(B, Hq, Hkv, Skv, d, seed=9)]
    outs = []
    for ns in (1, 2, 5, 47):
        o, lse = fa.decode_int8(q, kq, ks, vq, vs, num_splits=ns, return_lse=True)
        outs.append((o.float(), lse))
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert float((o - outs[0][0]).abs().max()) <= 2 ** -7
        assert float((lse - outs[0][1]).abs().max()) <= 1e-4
