"""GPU parity of the backward pass (fattn_bwd, bf16) against the fp64 oracle.

The GPU runs its own forward first (fattn_fwd with lse), then the backward by
recomputation from that lse; the oracle computes the gradients from the
definition.  Bars, relative to each gradient tensor's own scale (gradients are
not bounded like attention outputs, so absolute output bounds do not apply):
  max |err| <= 2^-6 * max |ref| + 1e-4  and  mean |err| <= 2^-7 * rms(ref) + 1e-5
(bf16 rounding of dq/dk/dv and of the P and dS operands gives about 2^-9 of
the value per element; the bars leave a factor 4 over what was measured).  The
absolute terms cover gradients that are exactly zero in real arithmetic, such
as dS = dP - D with a single visible key, where the kernel's fp32 difference
of two differently ordered sums leaves about 1e-6.
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

MAX_REL, MEAN_REL = 2.0 ** -6, 2.0 ** -7
MAX_ABS, MEAN_ABS = 1e-4, 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.detach().float().cpu().double().numpy()


def _check_grad(g, ref, what):
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    err = np.abs(g - ref)
    mx_ref = np.abs(ref).max() if ref.size else 0.0
    rms = math.sqrt(float((ref ** 2).mean())) if ref.size else 0.0
    assert err.max() <= MAX_REL * mx_ref + MAX_ABS, f"{what}: max {err.max():.3e} (ref max {mx_ref:.3e})"
    assert err.mean() <= MEAN_REL * rms + MEAN_ABS, f"{what}: mean {err.mean():.3e} (ref rms {rms:.3e})"
    return err.max() / max(mx_ref, 1e-30), err.mean() / max(rms, 1e-30)


def _run(q, k, v, do, causal, window, scale, dev):
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, window=window, scale=scale, return_lse=True)
    poison = lambda t: torch.full_like(t, float("nan"))
    out = (poison(qd), poison(kd), poison(vd))
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, window=window, scale=scale, out=out)
    torch.cuda.synchronize()
    return _np64(dq), _np64(dk), _np64(dv)


BWD_CASES = [
    # B, Hq, Hkv, Sq, Skv, d, causal, window, scale
    (1, 2, 2, 64, 64, 64, False, 0, None),
    (1, 2, 2, 128, 128, 128, True, 0, None),
    (2, 8, 2, 200, 200, 128, True, 0, None),        # GQA, ragged tiles
    (1, 4, 1, 333, 333, 64, True, 0, None),         # MQA
    (1, 4, 4, 100, 260, 128, True, 0, None),        # Sq < Skv (bottom-right causal)
    (1, 4, 4, 260, 100, 128, True, 0, None),        # Sq > Skv: rows with no key
    (1, 8, 2, 300, 300, 128, True, 64, None),       # window
    (1, 2, 2, 130, 70, 64, False, 0, -0.2),         # negative scale
    (1, 16, 2, 65, 65, 64, True, 1, None),          # window of one key
    (1, 232, 1, 40, 40, 64, True, 0, None),         # 232 query heads on one kv head
    (3, 2, 1, 1, 1, 128, True, 0, None),            # one query, one key
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_bwd_matches_oracle(case, cuda_device):
    B, Hq, Hkv, Sq, Skv, d, causal, window, scale = case
    _say(f"case bwd {case}")
    s = 1 / math.sqrt(d) if scale is None else scale
    q, k, v = W.prefill_inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", seed=800 + Sq + Hq)
    g = torch.Generator().manual_seed(900 + Sq + Hq)
    do = torch.randn(B, Sq, Hq, d, generator=g).to(torch.bfloat16)
    dq, dk, dv = _run(q, k, v, do, causal, window, s, cuda_device)
    rq, rk, rv = oracle.bwd(q, k, v, do, causal=causal, window=window, scale=s)
    res = [_check_grad(a, r, f"{n} {case}") for n, a, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))]
    _say("  rel max/mean: " + " ".join(f"{m:.2e}/{e:.2e}" for m, e in res))


def test_bwd_zero_scale_gives_zero_dq_dk(cuda_device):
    # scale 0: uniform weights, so dS = 0 exactly; dv is the mean of dO over visible rows
    _say("case bwd scale 0")
    q, k, v = W.prefill_inputs(1, 4, 2, 257, 257, 128, "bf16", seed=810)
    do = torch.randn(1, 257, 4, 128, generator=torch.Generator().manual_seed(811)).to(torch.bfloat16)
    dq, dk, dv = _run(q, k, v, do, True, 0, 0.0, cuda_device)
    assert np.abs(dq).max() <= MAX_ABS and np.abs(dk).max() <= MAX_ABS
    _, _, rv = oracle.bwd(q, k, v, do, causal=True, scale=0.0)
    _check_grad(dv, rv, "dv scale 0")


def test_bwd_is_bitwise_repeatable(cuda_device):
    _say("case bwd repeatability")
    q, k, v = (t.to(cuda_device) for t in W.prefill_inputs(2, 8, 2, 500, 500, 128, "bf16", seed=812))
    do = torch.randn(2, 500, 8, 128, device=cuda_device).to(torch.bfloat16)
    o, lse = fa.fwd(q, k, v, causal=True, return_lse=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
