"""Seeded synthetic inputs for tiled exact attention (shared by tests, smoke and bench).

This module only draws random tensors and names the workloads; it holds none
of the attention arithmetic, imports neither the HIP library nor the oracle,
and is the one piece of code both sides of every parity check share.

Workloads are shaped like the pages' examples: Llama-2-7B style MHA (32/32
heads, d=128), Mistral-7B style GQA (32 query / 8 kv heads), Falcon-180B
style MQA (232 / 1, d=64), S=4096 with batch 2, a 512-token sliding window and
a 32K-token int8 KV cache.  Values are i.i.d. N(0, 1) from ``torch.randn`` on a
seeded generator, drawn in the order Q, K, V and cast to bf16 by
round-to-nearest-even where the workload is bf16.

The int8 cache recipe (a reading: the pages name an int8 cache with no
scheme): symmetric per (token, kv head), scale = absmax / 127 in fp32,
code = clamp(round_half_even(x / scale), -127, 127); an all-zero row gets
scale 0 and codes 0.  The int4 cache uses the same recipe with 7 in place
of 127 and packs two codes per byte, element 2i in the low nibble of byte i
(signed 4-bit two's complement).  The consumers only ever see the stored
codes and scales, so this rounding cannot influence parity.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    d: int
    causal: bool
    window: int
    dtype: str  # "f32" or "bf16"
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    B: int
    Hq: int
    Hkv: int
    Skv: int
    d: int
    seed: int
    bits: int = 8  # code width of the KV cache: 8 or 4

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads (plus the windowed variant of the MQA one).
TINY_F32 = Prefill("tiny fp32 exact attention B1 H2 S128 d64 non-causal", 1, 2, 2, 128, 128, 64, False, 0, "f32", 0)
MHA_CAUSAL = Prefill("MHA causal prefill bf16 B2 H32 S4096 d128", 2, 32, 32, 4096, 4096, 128, True, 0, "bf16", 1)
GQA_CAUSAL = Prefill("GQA causal prefill bf16 B1 Hq32 Hkv8 S4096 d128", 1, 32, 8, 4096, 4096, 128, True, 0, "bf16", 2)
MQA_CAUSAL = Prefill("MQA causal prefill bf16 B1 Hq232 Hkv1 S2048 d64", 1, 232, 1, 2048, 2048, 64, True, 0, "bf16", 3)
MQA_WINDOW = Prefill("MQA causal sliding-window-512 prefill bf16 B1 Hq232 Hkv1 S2048 d64", 1, 232, 1, 2048, 2048, 64, True, 512, "bf16", 3)
# long dense rows: the kernel's loop rate with few blocks' fixed costs and no
# masked tiles (informational, not one of the parity configurations)
MHA_DENSE_LONG = Prefill("MHA dense prefill bf16 B1 H32 S16384 d128", 1, 32, 32, 16384, 16384, 128, False, 0, "bf16", 5)
INT8_DECODE = Decode("GQA decode over int8 KV cache B32 Hq32 Hkv8 Skv32768 d128", 32, 32, 8, 32768, 128, 4)
INT4_DECODE = Decode("GQA decode over int4 KV cache B32 Hq32 Hkv8 Skv32768 d128", 32, 32, 8, 32768, 128, 5, bits=4)

PREFILL_WORKLOADS = (TINY_F32, MHA_CAUSAL, GQA_CAUSAL, MQA_CAUSAL, MQA_WINDOW)


@dataclasses.dataclass(frozen=True)
class VarlenPrefill:
    name: str
    lens: tuple      # per-sequence lengths (queries = keys: causal self-attention)
    Hq: int
    Hkv: int
    d: int
    causal: bool
    dtype: str
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# A packed batch of 8 GQA sequences of mixed lengths, 16K tokens in all.
VARLEN_PREFILL = VarlenPrefill("packed variable-length GQA causal prefill bf16 8 sequences 256..4096 "
                               "(16384 tokens) Hq32 Hkv8 d128",
                               (4096, 512, 2048, 1024, 3072, 256, 1792, 3584), 32, 8, 128, True, "bf16", 6)
# Decode over a 32K-token int8 cache whose 32 sequences hold 1 .. 32768 tokens
# (uniform, seeded; drawn after the cache).
VARLEN_DECODE = Decode("GQA decode over int8 KV cache with per-sequence lengths 1..32768 "
                       "B32 Hq32 Hkv8 capacity 32768 d128", 32, 32, 8, 32768, 128, 7)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    raise ValueError(dtype)


def prefill_inputs(B, Hq, Hkv, Sq, Skv, d, dtype="bf16", seed=0, device="cpu"):
    """q [B,Sq,Hq,d], k/v [B,Skv,Hkv,d], i.i.d. N(0,1), drawn Q then K then V."""
    g = _gen(seed, device)
    q = torch.randn((B, Sq, Hq, d), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((B, Skv, Hkv, d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((B, Skv, Hkv, d), generator=g, device=device, dtype=torch.float32)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)


def key_drift(Skv, profile, step):
    """Per-key amplitudes a_j [Skv] (fp32, CPU): "rise" a_j = step * j, "fall"
    step * (Skv - 1 - j), "spikes" n * step at key 150 n - 50 (n = 1, 2, ...: keys
    100, 250, 400, ...) and 0 elsewhere."""
    j = torch.arange(Skv, dtype=torch.float32)
    if profile == "rise":
        return step * j
    if profile == "fall":
        return step * (Skv - 1 - j)
    if profile == "spikes":
        return torch.where(j % 150 == 100, step * (torch.div(j, 150, rounding_mode="floor") + 1), torch.tensor(0.0))
    raise ValueError(profile)


def drifting_inputs(B, Hq, Hkv, Sq, Skv, d, profile, step, dtype="bf16", seed=0, device="cpu"):
    """prefill_inputs' draws with every Q row moved by 2 and key j by a_j (key_drift)
    along the all-ones direction, before the cast: a score then carries an extra
    2 * a_j * d * scale, so along the keys the scores climb, fall, or jump at
    isolated keys far above every earlier one."""
    g = _gen(seed, device)
    q = torch.randn((B, Sq, Hq, d), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((B, Skv, Hkv, d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((B, Skv, Hkv, d), generator=g, device=device, dtype=torch.float32)
    q += 2.0
    k += key_drift(Skv, profile, step).to(device).view(1, Skv, 1, 1)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)


def workload_inputs(w: Prefill, device="cpu"):
    return prefill_inputs(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d, w.dtype, w.seed, device)


def cu_seqlens(lens) -> torch.Tensor:
    """Cumulative offsets [B+1] (int32) of packed sequences of the given lengths."""
    out = torch.zeros(len(lens) + 1, dtype=torch.int32)
    out[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    return out


def varlen_inputs(lens_q, lens_k, Hq, Hkv, d, dtype="bf16", seed=0, device="cpu"):
    """Packed q [sum(lens_q), Hq, d], k/v [sum(lens_k), Hkv, d], i.i.d. N(0,1)
    drawn Q then K then V, and the int32 offsets cu_q, cu_k [B+1] (on the CPU)."""
    g = _gen(seed, device)
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    q = torch.randn((tq, Hq, d), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((tk, Hkv, d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((tk, Hkv, d), generator=g, device=device, dtype=torch.float32)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype), cu_seqlens(lens_q), cu_seqlens(lens_k)


def varlen_workload_inputs(w: VarlenPrefill, device="cpu"):
    return varlen_inputs(w.lens, w.lens, w.Hq, w.Hkv, w.d, w.dtype, w.seed, device)


def decode_seqlens(w: Decode) -> torch.Tensor:
    """Per-sequence lengths of a variable-length decode workload: uniform in
    1 .. Skv from a generator seeded with seed + 1 (int32, on the CPU)."""
    g = _gen(w.seed + 1, "cpu")
    return torch.randint(1, w.Skv + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)


def quantize_rows_int8(x: torch.Tensor):
    """Per-row symmetric int8 codes over the last axis (see the module docstring)."""
    x = x.float()
    absmax = x.abs().amax(dim=-1)
    scale = absmax / 127.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    codes = torch.round(x / safe.unsqueeze(-1)).clamp_(-127, 127)
    codes = torch.where(scale.unsqueeze(-1) > 0, codes, torch.zeros_like(codes))
    return codes.to(torch.int8), scale.to(torch.float32)


def quantize_rows_int4(x: torch.Tensor):
    """Per-row symmetric int4 codes over the last axis, packed two per byte."""
    x = x.float()
    absmax = x.abs().amax(dim=-1)
    scale = absmax / 7.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    codes = torch.round(x / safe.unsqueeze(-1)).clamp_(-7, 7)
    codes = torch.where(scale.unsqueeze(-1) > 0, codes, torch.zeros_like(codes)).to(torch.int32)
    nib = codes & 15
    packed = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return packed.to(torch.uint8), scale.to(torch.float32)


def decode_inputs(B, Hq, Hkv, Skv, d, seed=0, device="cpu", keep_float=False, bits=8, k_drift=None):
    """q [B,Hq,d] bf16; kq/vq [B,Hkv,Skv,d] int8 (bits=8) or [B,Hkv,Skv,d/2]
    uint8 holding two int4 codes per byte (bits=4); k_scale/v_scale [B,Hkv,Skv] fp32.

    Draw order: Q, then for each batch entry K_b [Hkv,Skv,d] and V_b, each
    quantised as soon as it is drawn (so host memory stays at one slice).
    With keep_float=True the unquantised fp32 K and V are returned as well.
    With k_drift (a [Skv] tensor from key_drift) Q is moved by 2 and key j by
    k_drift[j] along the all-ones direction before quantisation.
    """
    if bits not in (8, 4):
        raise ValueError(bits)
    quantize_rows = quantize_rows_int8 if bits == 8 else quantize_rows_int4
    g = _gen(seed, device)
    q = torch.randn((B, Hq, d), generator=g, device=device, dtype=torch.float32)
    if k_drift is not None:
        q += 2.0
        k_drift = k_drift.to(device=device, dtype=torch.float32).view(1, Skv, 1)
    q = q.to(torch.bfloat16)
    if bits == 8:
        kq = torch.empty((B, Hkv, Skv, d), dtype=torch.int8, device=device)
    else:
        kq = torch.empty((B, Hkv, Skv, d // 2), dtype=torch.uint8, device=device)
    vq = torch.empty_like(kq)
    ks = torch.empty((B, Hkv, Skv), dtype=torch.float32, device=device)
    vs = torch.empty_like(ks)
    kf = vf = None
    if keep_float:
        kf = torch.empty((B, Hkv, Skv, d), dtype=torch.float32, device=device)
        vf = torch.empty_like(kf)
    for b in range(B):
        kb = torch.randn((Hkv, Skv, d), generator=g, device=device, dtype=torch.float32)
        if k_drift is not None:
            kb += k_drift
        kq[b], ks[b] = quantize_rows(kb)
        if keep_float:
            kf[b] = kb
        del kb
        vb = torch.randn((Hkv, Skv, d), generator=g, device=device, dtype=torch.float32)
        vq[b], vs[b] = quantize_rows(vb)
        if keep_float:
            vf[b] = vb
        del vb
    if keep_float:
        return q, kq, ks, vq, vs, kf, vf
    return q, kq, ks, vq, vs


def decode_workload_inputs(w: Decode, device="cpu", keep_float=False):
    return decode_inputs(w.B, w.Hq, w.Hkv, w.Skv, w.d, w.seed, device, keep_float, w.bits)
