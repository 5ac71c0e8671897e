"""GPU parity of variable-length batches against the fp64 oracle:
fattn_fwd_varlen (packed sequences, cumulative offsets) for bf16 and fp32,
and fattn_decode_int8_varlen / fattn_decode_int4_varlen (per-sequence cache
lengths).  Bounds as for the dense paths: fp32 max-abs 1e-5; bf16 max-abs
2e-2 and mean-abs 2e-3 on o, max-abs 1e-3 on lse.
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


def _check(o, o_ref, lse, lse_ref, f32, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: lse finiteness differs"
    le = np.abs(lse[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    if f32:
        assert err.max() <= F32_TOL and le <= F32_TOL, f"{what}: max-abs {err.max():.3e} lse {le:.3e}"
    else:
        assert err.max() <= BF16_MAX, f"{what}: max-abs {err.max():.3e}"
        assert err.mean() <= BF16_MEAN, f"{what}: mean-abs {err.mean():.3e}"
        assert le <= BF16_LSE, f"{what}: lse max-abs {le:.3e}"
    return err.max(), err.mean()


VARLEN_CASES = [
    # lens_q, lens_k, Hq, Hkv, d, causal, window, dtype
    ((7,), (7,), 2, 2, 64, False, 0, "f32"),
    ((5, 0, 3, 70, 4, 1), (5, 2, 9, 66, 0, 1), 4, 2, 64, True, 0, "f32"),
    ((100, 33, 257), (100, 33, 257), 8, 2, 128, True, 0, "bf16"),
    ((300, 1, 129, 64), (300, 1, 129, 64), 4, 1, 64, False, 0, "bf16"),
    ((513, 77, 200), (600, 77, 150), 8, 8, 128, True, 0, "bf16"),     # Sq != Skv per sequence
    ((400, 0, 250, 31), (400, 12, 250, 31), 16, 2, 128, True, 64, "bf16"),  # window
    ((129, 5), (0, 5), 4, 4, 64, True, 0, "bf16"),                        # a key-less sequence
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[str(c) for c in VARLEN_CASES])
def test_fwd_varlen_matches_oracle(case, cuda_device):
    lens_q, lens_k, Hq, Hkv, d, causal, window, dtype = case
    _say(f"case fwd varlen {case}")
    q, k, v, cu_q, cu_k = W.varlen_inputs(lens_q, lens_k, Hq, Hkv, d, dtype, seed=700 + sum(lens_q))
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = oracle.fwd_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), causal=causal,
                                       window=window, scale=scale)
    dev = cuda_device
    out = torch.full_like(q, float("nan"), device=dev)
    o, lse = fa.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev), causal=causal,
                           window=window, scale=scale, return_lse=True, out=out)
    torch.cuda.synchronize()
    mx, mean = _check(_np64(o), o_ref, _np64(lse), lse_ref, dtype == "f32", str(case))
    _say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_varlen_equal_lengths_is_the_dense_batch(dtype, cuda_device):
    # identical kernels, identical arithmetic: bit-equal outputs
    _say(f"case fwd varlen equal lengths {dtype}")
    B, S, Hq, Hkv, d = 3, 200, 8, 2, 128
    q, k, v = (t.to(cuda_device) for t in W.prefill_inputs(B, Hq, Hkv, S, S, d, dtype, seed=710))
    o, lse = fa.fwd(q, k, v, causal=True, return_lse=True)
    cu = (torch.arange(B + 1, dtype=torch.int32) * S).to(cuda_device)
    ov, lv = fa.fwd_varlen(q.reshape(B * S, Hq, d), k.reshape(B * S, Hkv, d), v.reshape(B * S, Hkv, d),
                           cu, cu, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(ov.reshape(B, S, Hq, d), o)
    assert torch.equal(lv, lse.permute(1, 0, 2).reshape(Hq, B * S))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_varlen_sequence_longer_than_max_seqlen_q(dtype, cuda_device):
    # max_seqlen_q only sizes the grid: a longer sequence keeps its own causal
    # diagonal (offset Skv_b - Sq_b), so every row that is written is exact;
    # rows below max_seqlen_q must all be written, rows past it may stay unwritten
    lens_q, lens_k, Hq, Hkv, d, bound = (100, 300), (120, 330), 4, 2, 128, 200
    _say(f"case fwd varlen max_seqlen_q {bound} < {max(lens_q)} ({dtype})")
    q, k, v, cu_q, cu_k = W.varlen_inputs(lens_q, lens_k, Hq, Hkv, d, dtype, seed=720)
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = oracle.fwd_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), causal=True, scale=scale)
    dev = cuda_device
    out = torch.full_like(q, float("nan"), device=dev)
    o, lse = fa.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev),
                           max_seqlen_q=bound, causal=True, scale=scale, return_lse=True, out=out)
    torch.cuda.synchronize()
    o, lse = _np64(o), _np64(lse)
    pos = np.concatenate([np.arange(n) for n in lens_q])  # position of each packed row in its sequence
    written = np.isfinite(o).all(axis=(1, 2))
    assert written[pos < bound].all(), "rows below max_seqlen_q left unwritten"
    mx, mean = _check(o[written], o_ref[written], lse[:, written], lse_ref[:, written], dtype == "f32",
                      "written rows")
    _say(f"  {int(written.sum())} of {len(pos)} rows written; max-abs {mx:.3e} mean-abs {mean:.3e}")


def test_fwd_varlen_empty_batch(cuda_device):
    q = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device=cuda_device)
    k = torch.zeros(5, 4, 64, dtype=torch.bfloat16, device=cuda_device)
    cu_q = torch.zeros(3, dtype=torch.int32, device=cuda_device)
    cu_k = torch.tensor([0, 2, 5], dtype=torch.int32, device=cuda_device)
    o = fa.fwd_varlen(q, k, k, cu_q, cu_k, causal=True)
    assert o.shape == q.shape


DECODE_VARLEN_CASES = [
    # B, Hq, Hkv, Skv, d, lens, bits, num_splits
    (4, 8, 2, 1000, 128, (1000, 0, 1, 517), 8, 0),
    (3, 4, 4, 2050, 64, (64, 2050, 33), 8, 7),
    (4, 8, 2, 1000, 128, (999, 0, 2, 640), 4, 0),
    (2, 20, 1, 333, 64, (333, 100), 4, 3),
    # many splits, per-sequence chunks that do not divide the lengths evenly
    (2, 8, 2, 4096, 128, (1500, 4000), 8, 0),
    (3, 4, 1, 3000, 64, (3000, 129, 2999), 4, 5),
]


@pytest.mark.parametrize("case", DECODE_VARLEN_CASES, ids=[str(c) for c in DECODE_VARLEN_CASES])
def test_decode_varlen_matches_oracle(case, cuda_device):
    B, Hq, Hkv, Skv, d, lens, bits, ns = case
    _say(f"case decode varlen {case}")
    q, kq, ks, vq, vs = W.decode_inputs(B, Hq, Hkv, Skv, d, seed=720 + Skv, bits=bits)
    sl = torch.tensor(lens, dtype=torch.int32)
    scale = 1 / math.sqrt(d)
    ref = oracle.decode_int8 if bits == 8 else oracle.decode_int4
    o_ref, lse_ref = ref(q, kq, ks, vq, vs, scale=scale, seqlens=sl.numpy())
    fn = fa.decode_int8 if bits == 8 else fa.decode_int4
    dev = cuda_device
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    o, lse = fn(q.to(dev), kq.to(dev), ks.to(dev), vq.to(dev), vs.to(dev), scale=scale,
                num_splits=ns, return_lse=True, out=out, seqlens=sl.to(dev))
    torch.cuda.synchronize()
    mx, mean = _check(_np64(o), o_ref, _np64(lse), lse_ref, False, str(case))
    _say(f"  max-abs {mx:.3e} mean-abs {mean:.3e}")
