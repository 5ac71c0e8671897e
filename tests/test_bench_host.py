"""Host-side logic of bench.py (no GPU): the one-GPU refusal and the
algorithmic FLOP and byte counts the reported rates are built on.

The counts are pinned to closed forms, not to bench.py's own loop:
  * causal, Sq = Skv = S: S(S+1)/2 visible pairs per head;
  * causal with a window of W keys (the query included): W(W+1)/2 + (S-W)W,
    which for the page's N = 4096, W = 512 is N*W - W(W-1)/2 (the golden
    fixture tests/golden/window_connections.json, [FA-VARIANTS] section on
    local window attention);
  * 4 d FLOP per visible pair per query head (two products of 2 d FLOP);
  * decode bytes: int8 K and V codes, one fp32 scale per (token, kv head) for
    each, the bf16 query and output.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


@pytest.mark.parametrize("S", [1, 2, 64, 777, 4096])
def test_causal_pairs_closed_form(S):
    assert bench.visible_pairs(S, S, True, 0) == S * (S + 1) // 2


@pytest.mark.parametrize("S,Wn", [(2048, 512), (4096, 512), (100, 1), (100, 100), (100, 250)])
def test_window_pairs_closed_form(S, Wn):
    w = min(Wn, S)
    assert bench.visible_pairs(S, S, True, Wn) == w * (w + 1) // 2 + (S - w) * w


def test_window_pairs_match_the_page_count():
    with open(os.path.join(ROOT, "tests", "golden", "window_connections.json")) as f:
        g = json.load(f)
    N, Wn = g["N"], g["W"]
    assert g["full_connections"] == N * N
    assert g["window_connections_per_token_count"] == N * Wn
    assert bench.visible_pairs(N, N, True, Wn) == N * Wn - Wn * (Wn - 1) // 2


def test_pairs_with_unequal_lengths():
    # bottom-right alignment: query i sees keys j <= i + Skv - Sq
    assert bench.visible_pairs(3, 5, True, 0) == 3 + 4 + 5
    assert bench.visible_pairs(5, 3, True, 0) == 0 + 0 + 1 + 2 + 3
    assert bench.visible_pairs(7, 9, False, 0) == 63


def test_workload_flops():
    # 4 d FLOP per pair per query head, per batch entry
    assert bench.prefill_flops(W.MHA_CAUSAL) == 4 * 128 * (4096 * 4097 // 2) * 2 * 32 == 274_945_015_808
    assert bench.prefill_flops(W.GQA_CAUSAL) == 4 * 128 * (4096 * 4097 // 2) * 1 * 32 == 137_472_507_904
    assert bench.prefill_flops(W.MQA_CAUSAL) == 4 * 64 * (2048 * 2049 // 2) * 232 == 124_614_868_992
    assert bench.prefill_flops(W.MQA_WINDOW) == 4 * 64 * (512 * 513 // 2 + 1536 * 512) * 232 == 54_507_601_920
    assert bench.prefill_flops(W.TINY_F32) == 4 * 64 * 128 * 128 * 2


def test_decode_bytes():
    w = W.INT8_DECODE
    codes = 2 * 32 * 8 * 32768 * 128          # int8 K and V
    scales = 2 * 32 * 8 * 32768 * 4           # fp32 per (token, kv head)
    qo = 2 * 32 * 32 * 128 * 2                # bf16 q and o
    assert bench.decode_bytes(w) == codes + scales + qo == 2_215_116_800
    assert bench.decode_bytes(W.INT4_DECODE) == codes // 2 + scales + qo
