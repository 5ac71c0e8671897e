"""GPU parity at the workloads' full sizes, over every output element.

Each headline workload (tiny fp32; MHA, GQA, MQA and windowed-MQA causal
prefill; int8-cache decode) and the full-size next rows (int4 decode,
packed varlen prefill, varlen decode, the backward of the MHA and GQA
prefills) run through the C ABI exactly as the benchmark launches them, and
every element of o and lse (of dq, dk, dv for the backward) is compared with
the fp64 oracle computed over the whole workload.  Outputs and workspaces
are guarded: the tensors are NaN-poisoned (every element must be written)
and fenced by sentinel bytes on both sides (no byte outside them may change).
Each workload also runs twice and must give the same bits.

Bars: fp32 max-abs 1e-5 on o and lse; bf16 max-abs 2e-2 and mean-abs 2e-3
on o, max-abs 1e-3 on lse; gradients max-abs <= 2^-6 max|ref| + 1e-4 and
mean-abs <= 2^-7 rms(ref) + 1e-5 per tensor.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_amd as fa
import workloads as W
from guard import Guarded

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 1e-3
GRAD_MAX_REL, GRAD_MEAN_REL, GRAD_MAX_ABS, GRAD_MEAN_ABS = 2.0 ** -6, 2.0 ** -7, 1e-4, 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.detach().float().cpu().double().numpy()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _compare(o, o_ref, lse, lse_ref, what, fp32=False):
    """Every element of o and lse against the oracle; returns (max, mean, lse max)."""
    assert o.shape == o_ref.shape and lse.shape == lse_ref.shape
    assert np.all(np.isfinite(o)), f"{what}: non-finite (or unwritten) output"
    err = np.abs(o - o_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: lse finiteness differs"
    lerr = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    mx, mean = float(err.max()), float(err.mean())
    _say(f"  {what}: {o.size} output elements, max-abs {mx:.3e} mean-abs {mean:.3e}; "
         f"{lse.size} lse values, max-abs {lerr:.3e}")
    if fp32:
        assert mx <= F32_TOL and lerr <= F32_TOL, what
    else:
        assert mx <= BF16_MAX, f"{what}: max-abs {mx:.3e}"
        assert mean <= BF16_MEAN, f"{what}: mean-abs {mean:.3e}"
        assert lerr <= BF16_LSE, f"{what}: lse max-abs {lerr:.3e}"
    return mx, mean, lerr


def _fwd(w, qd, kd, vd, dev):
    """One fattn_fwd call into guarded, NaN-poisoned o and lse."""
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    o = Guarded(qd.shape, dt, dev, fill=float("nan"))
    lse = Guarded((w.B, w.Hq, w.Sq), torch.float32, dev, fill=float("nan"))
    st = fa.fattn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.ptr, lse.ptr, w.B, w.Hq, w.Hkv,
                      w.Sq, w.Skv, w.d, w.scale, int(w.causal), w.window,
                      fa.FATTN_F32 if w.dtype == "f32" else fa.FATTN_BF16, _stream(dev))
    assert st == 0, fa.fattn_status_string(st)
    torch.cuda.synchronize()
    o.assert_intact("o")
    lse.assert_intact("lse")
    return o.t, lse.t


PREFILL = [W.TINY_F32, W.MHA_CAUSAL, W.GQA_CAUSAL, W.MQA_CAUSAL, W.MQA_WINDOW]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", PREFILL, ids=[w.name for w in PREFILL])
def test_prefill_every_element(w, cuda_device):
    _say(f"case: {w.name}")
    q, k, v = W.workload_inputs(w)
    qd, kd, vd = q.to(cuda_device), k.to(cuda_device), v.to(cuda_device)
    o, lse = _fwd(w, qd, kd, vd, cuda_device)
    o2, lse2 = _fwd(w, qd, kd, vd, cuda_device)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "not bitwise repeatable"
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.fwd(q, k, v, causal=w.causal, window=w.window, scale=w.scale)
    _say(f"  oracle over the whole workload: {time.perf_counter() - t0:.1f} s")
    _compare(_np64(o), o_ref, _np64(lse), lse_ref, w.name, fp32=w.dtype == "f32")


def _decode(w, tensors, dev, seqlens=None, num_splits=0):
    """One decode call (int8 or int4, optional lengths) into guarded buffers;
    the workspace starts full of garbage bytes."""
    q, kq, ks, vq, vs = tensors
    o = Guarded(q.shape, torch.bfloat16, dev, fill=float("nan"))
    lse = Guarded((w.B, w.Hq), torch.float32, dev, fill=float("nan"))
    need = fa.decode_workspace_size(w.B, w.Hq, w.Hkv, w.Skv, w.d, num_splits)
    ws = Guarded((need,), torch.uint8, dev, fill=0x7F)
    args = (w.B, w.Hq, w.Hkv, w.Skv, w.d, w.scale, num_splits, ws.ptr, need, _stream(dev))
    ptrs = [t.data_ptr() for t in (q, kq, ks, vq, vs)]
    if seqlens is None:
        fn = fa.fattn_decode_int8 if w.bits == 8 else fa.fattn_decode_int4
        st = fn(*ptrs, o.ptr, lse.ptr, *args)
    else:
        fn = fa.fattn_decode_int8_varlen if w.bits == 8 else fa.fattn_decode_int4_varlen
        st = fn(*ptrs, seqlens.data_ptr(), o.ptr, lse.ptr, *args)
    assert st == 0, fa.fattn_status_string(st)
    torch.cuda.synchronize()
    for g, name in ((o, "o"), (lse, "lse"), (ws, "workspace")):
        g.assert_intact(name)
    return o.t, lse.t


DECODE = [W.INT8_DECODE, W.INT4_DECODE]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", DECODE, ids=[w.name for w in DECODE])
def test_decode_every_element(w, cuda_device):
    _say(f"case: {w.name}")
    tensors = W.decode_workload_inputs(w, device=cuda_device)
    o, lse = _decode(w, tensors, cuda_device)
    o2, lse2 = _decode(w, tensors, cuda_device)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "not bitwise repeatable"
    qc, kqc, ksc, vqc, vsc = (t.cpu() for t in tensors)
    del tensors
    t0 = time.perf_counter()
    ref = oracle.decode_int8 if w.bits == 8 else oracle.decode_int4
    o_ref, lse_ref = ref(qc, kqc, ksc, vqc, vsc, scale=w.scale)
    _say(f"  oracle over the whole workload: {time.perf_counter() - t0:.1f} s")
    _compare(_np64(o), o_ref, _np64(lse), lse_ref, w.name)


@pytest.mark.timeout(600)
def test_varlen_decode_every_element(cuda_device):
    w = W.VARLEN_DECODE
    _say(f"case: {w.name}")
    tensors = W.decode_workload_inputs(w, device=cuda_device)
    sl = W.decode_seqlens(w)
    o, lse = _decode(w, tensors, cuda_device, seqlens=sl.to(cuda_device))
    qc, kqc, ksc, vqc, vsc = (t.cpu() for t in tensors)
    del tensors
    o_ref, lse_ref = oracle.decode_int8(qc, kqc, ksc, vqc, vsc, scale=w.scale, seqlens=sl.numpy())
    _compare(_np64(o), o_ref, _np64(lse), lse_ref, w.name)


@pytest.mark.timeout(600)
def test_varlen_prefill_every_element(cuda_device):
    w = W.VARLEN_PREFILL
    _say(f"case: {w.name}")
    q, k, v, cu_q, cu_k = W.varlen_workload_inputs(w)
    dev = cuda_device
    qd, kd, vd, cqd, ckd = (t.to(dev) for t in (q, k, v, cu_q, cu_k))
    total_q, total_k = q.shape[0], k.shape[0]
    outs = []
    for _ in range(2):
        o = Guarded(qd.shape, torch.bfloat16, dev, fill=float("nan"))
        lse = Guarded((w.Hq, total_q), torch.float32, dev, fill=float("nan"))
        st = fa.fattn_fwd_varlen(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.ptr, lse.ptr,
                                 cqd.data_ptr(), ckd.data_ptr(), len(w.lens), w.Hq, w.Hkv, total_q,
                                 total_k, max(w.lens), w.d, w.scale, int(w.causal), 0, fa.FATTN_BF16,
                                 _stream(dev))
        assert st == 0, fa.fattn_status_string(st)
        torch.cuda.synchronize()
        o.assert_intact("o")
        lse.assert_intact("lse")
        outs.append((o.t, lse.t))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    o_ref, lse_ref = oracle.fwd_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), causal=w.causal,
                                       scale=w.scale)
    _compare(_np64(outs[0][0]), o_ref, _np64(outs[0][1]), lse_ref, w.name)


def _check_grad(g, ref, what):
    assert np.all(np.isfinite(g)), f"{what}: non-finite (or unwritten) gradient"
    err = np.abs(g - ref)
    mx_ref = float(np.abs(ref).max())
    rms = math.sqrt(float((ref ** 2).mean()))
    mx, mean = float(err.max()), float(err.mean())
    _say(f"  {what}: {g.size} elements, max-abs {mx:.3e} (bound {GRAD_MAX_REL * mx_ref + GRAD_MAX_ABS:.3e}), "
         f"mean-abs {mean:.3e} (bound {GRAD_MEAN_REL * rms + GRAD_MEAN_ABS:.3e})")
    assert mx <= GRAD_MAX_REL * mx_ref + GRAD_MAX_ABS, what
    assert mean <= GRAD_MEAN_REL * rms + GRAD_MEAN_ABS, what


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", [W.MHA_CAUSAL, W.GQA_CAUSAL], ids=lambda w: w.name)
def test_bwd_every_element(w, cuda_device):
    _say(f"case bwd: {w.name}")
    dev = cuda_device
    q, k, v = W.workload_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 100)
    do = torch.randn(w.B, w.Sq, w.Hq, w.d, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = _fwd(w, qd, kd, vd, dev)
    need = fa.fattn_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d)
    ws = Guarded((need,), torch.uint8, dev, fill=0x7F)
    grads = [Guarded(t.shape, torch.bfloat16, dev, fill=float("nan")) for t in (qd, kd, vd)]
    st = fa.fattn_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      dod.data_ptr(), *(t.ptr for t in grads), w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d,
                      w.scale, int(w.causal), w.window, fa.FATTN_BF16, ws.ptr, need, _stream(dev))
    assert st == 0, fa.fattn_status_string(st)
    torch.cuda.synchronize()
    for t, name in ((ws, "workspace"), *zip(grads, ("dq", "dk", "dv"))):
        t.assert_intact(name)
    t0 = time.perf_counter()
    refs = oracle.bwd(q, k, v, do, causal=w.causal, window=w.window, scale=w.scale)
    _say(f"  oracle over the whole workload: {time.perf_counter() - t0:.1f} s")
    for t, ref, name in zip(grads, refs, ("dq", "dk", "dv")):
        _check_grad(_np64(t.t), ref, name)
