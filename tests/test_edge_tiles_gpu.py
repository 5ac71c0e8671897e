"""GPU parity of the prefill's edge-tile paths against the fp64 oracle.

Shapes picked so that the band of some blocks ends within the first 32 keys
of its last 64-key tile (the half-width last iteration), and so that the
causal and window edges cut one, both or neither 32-key block of a masked
tile for the waves of a block (rows enumerate (position, head) with the heads
of a chunk fastest: 1 head per position for MHA, 4 for G = 4, 8 for G = 8).
Every output element is compared (outputs NaN-poisoned), with the bf16
bounds of the other parity tests: max-abs 2e-2 and mean-abs 2e-3 on o,
max-abs 1e-3 on lse.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_amd as fa
import workloads as W

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_LSE = 2e-2, 2e-3, 1e-3

# (B, Hq, Hkv, Sq, Skv, d, causal, window)
CASES = [
    (1, 2, 2, 100, 80, 64, False, 0),     # unmasked band of 80 keys: last tile holds 16
    (1, 2, 1, 70, 96, 128, False, 0),     # 96 keys: last tile holds 32 (exactly half)
    (1, 2, 2, 97, 97, 128, False, 0),     # 97 keys: last tile holds 33 (full width)
    (1, 16, 2, 300, 300, 64, True, 80),   # G = 8: 16 positions per block, band W + 15 = 95 keys
    (1, 16, 2, 300, 300, 128, True, 80),
    (1, 16, 1, 257, 257, 64, True, 0),    # G = 16: 8 positions per block
    (2, 8, 2, 200, 200, 128, True, 0),    # G = 4: 32 positions per block, every other band half-width
    (1, 8, 2, 150, 230, 64, True, 0),     # Skv > Sq: the diagonal moves by 80 keys
    (1, 4, 4, 96, 96, 128, True, 0),      # MHA: one block, the diagonal cuts one 32-key block per wave
    (1, 4, 4, 200, 200, 64, True, 20),    # window narrower than a 32-key block: both edges in one block
    (1, 8, 1, 130, 130, 128, True, 1),    # window of one key (self only)
    (1, 8, 8, 64, 40, 64, True, 0),       # Skv < Sq: leading rows see no key (lse -inf)
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(t):
    return t.detach().float().cpu().double().numpy()


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_edge_tiles(case, cuda_device):
    B, Hq, Hkv, Sq, Skv, d, causal, window = case
    _say(f"case edge tiles {case}")
    seed = 7100 + CASES.index(case)
    q, k, v = W.prefill_inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", seed=seed)
    scale = 1.0 / d ** 0.5
    o_ref, lse_ref = oracle.fwd(q, k, v, causal=causal, window=window, scale=scale)
    dev = cuda_device
    out = torch.full_like(q, float("nan"), device=dev)
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, window=window, scale=scale,
                    return_lse=True, out=out)
    torch.cuda.synchronize()
    o64, lse64 = _np64(o), _np64(lse)
    # rows with no visible key: the output is 0 and lse is -inf on both sides
    assert np.all(np.isfinite(o64)), f"{case}: non-finite output"
    err = np.abs(o64 - o_ref)
    assert err.max() <= BF16_MAX, f"{case}: max-abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN, f"{case}: mean-abs {err.mean():.3e}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse64)), f"{case}: lse finiteness differs"
    if fin.any():
        le = np.abs(lse64[fin] - lse_ref[fin]).max()
        assert le <= BF16_LSE, f"{case}: lse max-abs {le:.3e}"
    _say(f"  max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
