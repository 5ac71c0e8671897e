"""Pins for the fp64 oracle: facts the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: a
closed form, an invariant, a value the pages print, an independent algorithm
(brute force over the full score matrix, the online one-pass softmax with a
split and log-sum-exp merge) or a library routine (torch's CPU attention in
float64).  ``test_planted_mistakes_are_caught`` builds mutated copies of the
oracle source, each with one plausible mistake, and requires that some pin
fails on each of them.

Sources, cited by page title and section:
 [FA-NPU]      "When Transformer meets the Ascend NPU: the memory-slimming
               secret of the FlashAttention operator"
 [FA-3MOVES]   the ai6s.net article on FlashAttention's three moves
 [FA-VARIANTS] "The FlashAttention variant family: GQA, MQA and sparse
               attention, how to choose"
"""
from __future__ import annotations

import json
import math
import os
import tempfile

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------
# independent algorithms written in this file (not the oracle's code)
# ----------------------------------------------------------------------------

def brute_force(q, k, v, causal, window, scale):
    """Two-pass softmax over the full [Sq, Skv] score matrix, per (b, h)."""
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    off = Skv - Sq
    i = np.arange(Sq)[:, None]
    j = np.arange(Skv)[None, :]
    vis = np.ones((Sq, Skv), dtype=bool)
    if causal:
        vis &= j <= i + off
        if window:
            vis &= j > i + off - window
    o = np.zeros((B, Sq, Hq, d))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, h // G, :].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            e = np.where(vis, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
            l = e.sum(axis=1, keepdims=True)
            p = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
            o[b, :, h, :] = p @ v[b, :, h // G, :]
            lse[b, h, ok] = (m[:, 0] + np.log(l[:, 0]))[ok]
    return o, lse


def online_row(qrow, K, V, scale, block):
    """Online softmax over key blocks: running max m, running sum l, rescaled acc.

    [FA-NPU] tiling section (each block's local max and sum, corrected at the
    end) and [FA-3MOVES] move 2 (only the current max and current exp-sum are
    kept).  Returns (o, lse) for one query row over the given visible keys.
    """
    m, l = -np.inf, 0.0
    acc = np.zeros(V.shape[1])
    for j0 in range(0, K.shape[0], block):
        s = scale * (K[j0:j0 + block] @ qrow)
        m_new = max(m, s.max())
        alpha = math.exp(m - m_new) if np.isfinite(m) else 0.0
        p = np.exp(s - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ V[j0:j0 + block]
        m = m_new
    return acc / l, m + math.log(l)


def lse_merge(parts):
    """Merge (o_s, lse_s) partials of disjoint key splits by log-sum-exp."""
    lses = np.array([p[1] for p in parts])
    M = lses.max()
    w = np.exp(lses - M)
    o = sum(wi * p[0] for wi, p in zip(w, parts)) / w.sum()
    return o, M + math.log(w.sum())


# ----------------------------------------------------------------------------
# the pins; each takes the path of an oracle build (None = the real one)
# ----------------------------------------------------------------------------

def pin_probabilities_sum_to_one(lib):
    # V = identity rows (Skv <= d): O[i] is the probability row of query i.
    B, S, H, d = 1, 12, 2, 16
    q = _rand((B, S, H, d), 1)
    k = _rand((B, S, H, d), 2)
    v = np.zeros((B, S, H, d))
    for j in range(S):
        v[0, j, :, j] = 1.0
    for causal, window in ((False, 0), (True, 0), (True, 5)):
        o, _ = oracle.fwd(q, k, v, causal=causal, window=window, lib=lib)
        p = o[..., :S]
        assert np.all(p >= 0)
        assert np.allclose(p.sum(-1), 1.0, atol=1e-12, rtol=0)
        assert np.all(o[..., S:] == 0)
        if causal:
            i = np.arange(S)[:, None]
            j = np.arange(S)[None, :]
            masked = j > i
            if window:
                masked |= j <= i - window
            assert np.all(p[0].transpose(1, 0, 2)[:, masked] == 0)


def pin_constant_values(lib):
    # V[b, j, hk, :] = c[b, hk] for all j  =>  O[b, i, h, :] = c[b, h // G].
    B, S, Hq, Hkv, d = 2, 9, 4, 2, 8
    q = _rand((B, S, Hq, d), 3)
    k = _rand((B, S, Hkv, d), 4)
    c = _rand((B, Hkv, d), 5)
    v = np.broadcast_to(c[:, None, :, :], (B, S, Hkv, d)).copy()
    for causal in (False, True):
        o, _ = oracle.fwd(q, k, v, causal=causal, lib=lib)
        want = np.repeat(c, Hq // Hkv, axis=1)[:, None, :, :]
        assert np.allclose(o, np.broadcast_to(want, o.shape), atol=1e-12, rtol=0)


def pin_identical_keys_average_values(lib):
    # all key rows equal => uniform weights => O[i] = mean of V over the visible keys.
    B, S, H, d = 1, 10, 1, 6
    q = _rand((B, S, H, d), 6)
    k = np.broadcast_to(_rand((1, 1, 1, d), 7), (B, S, H, d)).copy()
    v = _rand((B, S, H, d), 8)
    o, _ = oracle.fwd(q, k, v, causal=False, lib=lib)
    assert np.allclose(o[0, :, 0], v[0, :, 0].mean(0), atol=1e-12, rtol=0)
    o, _ = oracle.fwd(q, k, v, causal=True, lib=lib)
    for i in range(S):
        assert np.allclose(o[0, i, 0], v[0, :i + 1, 0].mean(0), atol=1e-12, rtol=0)
    o, _ = oracle.fwd(q, k, v, causal=True, window=3, lib=lib)
    for i in range(S):
        assert np.allclose(o[0, i, 0], v[0, max(0, i - 2):i + 1, 0].mean(0), atol=1e-12, rtol=0)


def pin_causal_first_row(lib):
    # causal row 0 sees only key 0: O = V[0], lse = scale * q0 . k0.
    B, S, H, d = 2, 7, 3, 8
    q, k, v = _rand((B, S, H, d), 9), _rand((B, S, H, d), 10), _rand((B, S, H, d), 11)
    scale = 0.37
    o, lse = oracle.fwd(q, k, v, causal=True, scale=scale, lib=lib)
    assert np.allclose(o[:, 0], v[:, 0], atol=1e-12, rtol=0)
    want = scale * np.einsum("bhc,bhc->bh", q[:, 0], k[:, 0])
    assert np.allclose(lse[:, :, 0], want, atol=1e-12, rtol=0)


def pin_two_key_closed_form(lib):
    # q = a e1, k0 = 0, k1 = b e1: p1 = sigmoid(scale a b), lse = log(1 + e^{scale a b}).
    d = 4
    for a, b, scale in ((1.5, 2.0, 0.5), (-3.0, 1.0, 0.25), (2.0, -2.5, 1.0)):
        q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = a
        k = np.zeros((1, 2, 1, d)); k[0, 1, 0, 0] = b
        v = _rand((1, 2, 1, d), 12)
        o, lse = oracle.fwd(q, k, v, causal=False, scale=scale, lib=lib)
        t = scale * a * b
        p1 = 1.0 / (1.0 + math.exp(-t))
        assert np.allclose(o[0, 0, 0], (1 - p1) * v[0, 0, 0] + p1 * v[0, 1, 0], atol=1e-12, rtol=0)
        assert abs(lse[0, 0, 0] - math.log1p(math.exp(t))) < 1e-12


def pin_zero_keys_count_visible(lib):
    # K = 0 => every visible score is 0 => lse = log |Vis(i)|.
    for (Sq, Skv, causal, window) in ((6, 6, False, 0), (6, 6, True, 0), (6, 6, True, 2),
                                      (3, 8, True, 0), (3, 8, True, 4), (1, 5, True, 0)):
        q = _rand((1, Sq, 1, 4), 13)
        k = np.zeros((1, Skv, 1, 4))
        v = _rand((1, Skv, 1, 4), 14)
        _, lse = oracle.fwd(q, k, v, causal=causal, window=window, lib=lib)
        off = Skv - Sq
        for i in range(Sq):
            n = Skv if not causal else min(i + off + 1, Skv)
            if window:
                n = min(n, window)
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-12, (Sq, Skv, causal, window, i)


def pin_online_and_brute_force_agree(lib):
    # the three-pass oracle == full-matrix two-pass == online one-pass, and any
    # split of the keys merged by log-sum-exp gives the same row.
    B, Sq, Skv, Hq, Hkv, d = 1, 9, 13, 4, 2, 8
    q, k, v = _rand((B, Sq, Hq, d), 15), _rand((B, Skv, Hkv, d), 16), _rand((B, Skv, Hkv, d), 17)
    scale = 0.3
    for causal, window in ((False, 0), (True, 0), (True, 4)):
        o, lse = oracle.fwd(q, k, v, causal=causal, window=window, scale=scale, lib=lib)
        ob, lb = brute_force(q, k, v, causal, window, scale)
        assert np.allclose(o, ob, atol=1e-12, rtol=0)
        assert np.allclose(lse, lb, atol=1e-12, rtol=0)
        off = Skv - Sq
        for h in range(Hq):
            for i in range(Sq):
                lo, hi = 0, Skv
                if causal:
                    hi = i + off + 1
                    if window:
                        lo = max(0, hi - window)
                K, V = k[0, lo:hi, h // 2], v[0, lo:hi, h // 2]
                for block in (1, 3, 64):
                    oo, ll = online_row(q[0, i, h], K, V, scale, block)
                    assert np.allclose(oo, o[0, i, h], atol=1e-12, rtol=0)
                    assert abs(ll - lse[0, h, i]) < 1e-12
                n = hi - lo
                if n >= 3:
                    cuts = [0, n // 3, n // 2 + 1, n]
                    parts = [online_row(q[0, i, h], K[a:b], V[a:b], scale, 2)
                             for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
                    om, lm = lse_merge(parts)
                    assert np.allclose(om, o[0, i, h], atol=1e-12, rtol=0)
                    assert abs(lm - lse[0, h, i]) < 1e-12


def pin_gqa_equals_mha_on_repeated_kv(lib):
    # [FA-VARIANTS] GQA section: GQA(q, k, v) == MHA(q, repeat_interleave(k), repeat_interleave(v)),
    # for the head ratios of the page's example models (scaled-down sequence).
    g = _golden("gqa_head_configs.json")
    for mdl in g["models"]:
        Hq, Hkv = mdl["num_q_heads"], mdl["num_kv_heads"]  # the page's head counts
        B, S, d = 1, 5, 8
        q = _rand((B, S, Hq, d), 18)
        k, v = _rand((B, S, Hkv, d), 19), _rand((B, S, Hkv, d), 20)
        ratio = Hq // Hkv
        kr = np.repeat(k, ratio, axis=2)  # repeat_interleave along heads
        vr = np.repeat(v, ratio, axis=2)
        for causal in (False, True):
            o1, l1 = oracle.fwd(q, k, v, causal=causal, lib=lib)
            o2, l2 = oracle.fwd(q, kr, vr, causal=causal, lib=lib)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2), mdl["model"]
    # distinct kv heads must actually be told apart (a h % Hkv mapping fails here)
    q = _rand((1, 4, 8, 8), 21)
    k, v = _rand((1, 4, 2, 8), 22), _rand((1, 4, 2, 8), 23)
    o, _ = oracle.fwd(q, k, v, causal=True, lib=lib)
    o_first, _ = oracle.fwd(q[:, :, :4], k[:, :, :1], v[:, :, :1], causal=True, lib=lib)
    assert np.array_equal(o[:, :, :4], o_first)


def pin_window_conventions(lib):
    B, S, H, d = 1, 11, 2, 8
    q, k, v = _rand((B, S, H, d), 24), _rand((B, S, H, d), 25), _rand((B, S, H, d), 26)
    o, lse = oracle.fwd(q, k, v, causal=True, window=1, lib=lib)  # W=1: only itself
    assert np.allclose(o, v, atol=1e-12, rtol=0)
    want = np.einsum("bshc,bshc->bhs", q, k) / math.sqrt(d)
    assert np.allclose(lse, want, atol=1e-12, rtol=0)
    oc, lc = oracle.fwd(q, k, v, causal=True, lib=lib)
    for W in (S, S + 5):  # W >= Skv is plain causal
        ow, lw = oracle.fwd(q, k, v, causal=True, window=W, lib=lib)
        assert np.array_equal(ow, oc) and np.array_equal(lw, lc)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, causal=False, window=3, lib=lib)


def pin_window_connection_count_from_page(lib):
    # [FA-VARIANTS] sliding window section: N=4096 gives N^2 = 16,777,216 full
    # connections; W=512 gives N*W = 2,097,152 (W per token; exact count with the
    # first W-1 rows short is N*W - W(W-1)/2).  K = 0 makes exp(lse) the count.
    g = _golden("window_connections.json")
    N, W = g["N"], g["W"]
    q = np.zeros((1, N, 1, 1)); k = np.zeros((1, N, 1, 1)); v = np.zeros((1, N, 1, 1))
    _, lse = oracle.fwd(q, k, v, causal=False, lib=lib)
    assert round(float(np.exp(lse).sum())) == g["full_connections"]
    _, lse = oracle.fwd(q, k, v, causal=True, window=W, lib=lib)
    counts = np.rint(np.exp(lse[0, 0])).astype(np.int64)
    assert np.all(counts[W - 1:] == W)  # every token past the start sees W keys
    assert counts.sum() == g["window_connections_per_token_count"] - W * (W - 1) // 2
    saving = 100.0 * (1 - g["window_connections_per_token_count"] / g["full_connections"])
    assert abs(saving - g["saving_percent"]) < 1e-9


def pin_shift_invariance(lib):
    # adding the same vector u to every key row shifts each query's scores by
    # scale * q.u: O unchanged, lse shifted by that constant.
    B, S, Hq, Hkv, d = 2, 8, 4, 2, 8
    q, k, v = _rand((B, S, Hq, d), 27), _rand((B, S, Hkv, d), 28), _rand((B, S, Hkv, d), 29)
    u = _rand((B, 1, Hkv, d), 30) * 3
    scale = 0.4
    for causal in (False, True):
        o1, l1 = oracle.fwd(q, k, v, causal=causal, scale=scale, lib=lib)
        o2, l2 = oracle.fwd(q, k + u, v, causal=causal, scale=scale, lib=lib)
        assert np.allclose(o1, o2, atol=1e-11, rtol=0)
        shift = scale * np.einsum("bshc,bhc->bhs", q, np.repeat(u[:, 0], Hq // Hkv, axis=1))
        assert np.allclose(l2 - l1, shift, atol=1e-11, rtol=0)


def pin_permutation_invariance(lib):
    # non-causal attention does not see key order: permuting K and V rows together changes nothing.
    B, S, H, d = 1, 10, 2, 8
    q, k, v = _rand((B, S, H, d), 31), _rand((B, S, H, d), 32), _rand((B, S, H, d), 33)
    perm = np.random.default_rng(34).permutation(S)
    o1, l1 = oracle.fwd(q, k, v, causal=False, lib=lib)
    o2, l2 = oracle.fwd(q, k[:, perm], v[:, perm], causal=False, lib=lib)
    assert np.allclose(o1, o2, atol=1e-12, rtol=0) and np.allclose(l1, l2, atol=1e-12, rtol=0)


def pin_large_logits_stay_finite(lib):
    B, S, H, d = 1, 16, 1, 8
    q, k, v = _rand((B, S, H, d), 35) * 30, _rand((B, S, H, d), 36) * 30, _rand((B, S, H, d), 37)
    o, lse = oracle.fwd(q, k, v, causal=True, scale=10.0, lib=lib)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.all(np.abs(o) <= np.abs(v).max() + 1e-12)


def pin_empty_rows(lib):
    # Sq > Skv with the bottom-right causal alignment: the first Sq-Skv rows see no key.
    q, k, v = _rand((1, 5, 1, 4), 38), _rand((1, 3, 1, 4), 39), _rand((1, 3, 1, 4), 40)
    o, lse = oracle.fwd(q, k, v, causal=True, lib=lib)
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.allclose(o[0, 2, 0], v[0, 0, 0], atol=1e-12, rtol=0)


def _quantise(x):
    s = np.abs(x).max(-1) / 127.0
    c = np.clip(np.rint(x / np.where(s > 0, s, 1)[..., None]), -127, 127).astype(np.int8)
    return c, s.astype(np.float32)


def pin_decode_equals_forward_on_dequantised(lib):
    # the decode oracle is attention of one query over code * scale values.
    B, Hq, Hkv, Skv, d = 2, 4, 2, 9, 8
    q = _rand((B, Hq, d), 41)
    kq, ks = _quantise(_rand((B, Hkv, Skv, d), 42))
    vq, vs = _quantise(_rand((B, Hkv, Skv, d), 43))
    ks[0, 1, 3] = 0.0  # a zero scale row
    kq[0, 1, 3] = 0
    o, lse = oracle.decode_int8(q, kq, ks, vq, vs, scale=0.3, lib=lib)
    kd = kq.astype(np.float64) * ks.astype(np.float64)[..., None]
    vd = vq.astype(np.float64) * vs.astype(np.float64)[..., None]
    # to the forward layout: q [B, 1, Hq, d], k/v [B, Skv, Hkv, d]
    of, lf = oracle.fwd(q[:, None], kd.transpose(0, 2, 1, 3), vd.transpose(0, 2, 1, 3),
                        causal=True, scale=0.3, lib=lib)
    assert np.array_equal(o, of[:, 0]) and np.array_equal(lse, lf[:, :, 0])
    # and against the brute-force definition
    ob, lb = brute_force(q[:, None], kd.transpose(0, 2, 1, 3), vd.transpose(0, 2, 1, 3), False, 0, 0.3)
    assert np.allclose(o, ob[:, 0], atol=1e-12, rtol=0) and np.allclose(lse, lb[:, :, 0], atol=1e-12, rtol=0)


def pin_rows_subset_matches_full(lib):
    B, S, Hq, Hkv, d = 2, 7, 4, 2, 8
    q, k, v = _rand((B, S, Hq, d), 44), _rand((B, S, Hkv, d), 45), _rand((B, S, Hkv, d), 46)
    o, lse = oracle.fwd(q, k, v, causal=True, lib=lib)
    rows = np.array([[1, 3, 6], [0, 0, 0], [1, 2, 4]])
    orow, lrow = oracle.fwd(q, k, v, causal=True, rows=rows, lib=lib)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(orow[r], o[b, i, h]) and lrow[r] == lse[b, h, i]


def pin_torch_sdpa_float64(lib):
    # independent library cross-check (torch's math attention, CPU float64; its
    # is_causal is top-left aligned, so only Sq == Skv is compared).
    B, S, H, d = 2, 11, 3, 16
    q, k, v = _rand((B, S, H, d), 47), _rand((B, S, H, d), 48), _rand((B, S, H, d), 49)
    for causal in (False, True):
        o, _ = oracle.fwd(q, k, v, causal=causal, lib=lib)
        t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
        assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)


def pin_quantizer_rounding_and_bounds(lib):
    # absmax 127 gives scale exactly 1: codes are round-half-even of the values
    x = np.zeros((1, 1, 1, 8), dtype=np.float32)
    x[0, 0, 0] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -126.5, 1.25]
    c, sc = oracle.kv_quantize_int8(x, lib=lib)
    assert sc[0, 0, 0] == np.float32(1.0)
    assert list(c[0, 0, 0]) == [127, 2, 4, -2, -4, 0, -126, 1]
    # general rows: the absmax element maps to +-127, the error is at most half a step
    rng = np.random.default_rng(50)
    x = rng.standard_normal((2, 5, 3, 16)).astype(np.float32) * rng.uniform(0.01, 100, (2, 5, 3, 1)).astype(np.float32)
    x[1, 2, 1] = 0.0  # an all-zero row
    codes = np.full((2, 3, 9, 16), 77, dtype=np.int8)
    scales = np.full((2, 3, 9), -1.0, dtype=np.float32)
    oracle.kv_quantize_int8(x, codes, scales, pos=3, cap=9, lib=lib)
    assert np.all(codes[:, :, :3] == 77) and np.all(codes[:, :, 8:] == 77)  # untouched
    assert np.all(scales[:, :, :3] == -1) and np.all(scales[:, :, 8:] == -1)
    got_c = codes[:, :, 3:8].transpose(0, 2, 1, 3)  # -> [B, T, Hkv, d]
    got_s = scales[:, :, 3:8].transpose(0, 2, 1)
    assert got_s[1, 2, 1] == 0 and np.all(got_c[1, 2, 1] == 0)
    amax = np.abs(x).max(-1)
    nz = amax > 0
    assert np.all(np.abs(got_c[nz].astype(int)).max(-1) == 127)
    assert np.all(np.abs(got_c.astype(int)) <= 127)
    deq = got_c.astype(np.float64) * got_s[..., None].astype(np.float64)
    assert np.all(np.abs(deq - x) <= 0.5 * got_s[..., None] * (1 + 1e-6) + 1e-30)
    assert np.allclose(got_s[nz], amax[nz] / 127.0, rtol=1e-7, atol=0)


def pin_quantizer_matches_torch(lib):
    # an independent implementation of the same fp32 recipe (torch ops, CPU)
    import workloads as W
    g = torch.Generator().manual_seed(51)
    x = torch.randn(3, 7, 4, 64, generator=g) * 3
    x[0, 1, 2] = 0
    c_ref, s_ref = W.quantize_rows_int8(x)  # over the last axis, rows (b, t, h)
    c, sc = oracle.kv_quantize_int8(x.numpy(), lib=lib)
    assert np.array_equal(c.transpose(0, 2, 1, 3), c_ref.numpy())
    assert np.array_equal(sc.transpose(0, 2, 1), s_ref.numpy())


def _pack_int4(codes):
    """Two signed 4-bit codes per byte: element 2i low nibble, 2i+1 high nibble."""
    c = np.asarray(codes, dtype=np.int64)
    return ((c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)).astype(np.uint8)


def _unpack_int4(packed):
    """Inverse of _pack_int4, written with the xor form of sign extension."""
    b = np.asarray(packed, dtype=np.int64)
    lo, hi = ((b & 15) ^ 8) - 8, ((b >> 4) ^ 8) - 8
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return out


def pin_int4_decode_single_key_closed_form(lib):
    # one cached token: every probability is 1, so O is that token's value row
    # (code * scale, all 16 nibble values present) and lse its scaled score.
    d = 16
    vcodes = np.arange(-8, 8)               # every 4-bit two's complement value
    kcodes = np.array([3, -1, 0, 7, -7, 2, -8, 5, 1, 1, -2, 4, 0, -3, 6, -5])
    kq, vq = _pack_int4(kcodes)[None, None, None], _pack_int4(vcodes)[None, None, None]
    assert list(vq[0, 0, 0]) == [0x98, 0xBA, 0xDC, 0xFE, 0x10, 0x32, 0x54, 0x76]
    ks = np.full((1, 1, 1), 0.25, dtype=np.float32)
    vs = np.full((1, 1, 1), 0.5, dtype=np.float32)
    q = _rand((1, 2, d), 52)                # two query heads share the kv head
    o, lse = oracle.decode_int4(q, kq, ks, vq, vs, scale=0.7, lib=lib)
    for h in range(2):
        assert np.array_equal(o[0, h], 0.5 * vcodes)
        assert abs(lse[0, h] - 0.7 * float(q[0, h] @ (0.25 * kcodes))) < 1e-12


def pin_int4_decode_equals_forward_on_dequantised(lib):
    B, Hq, Hkv, Skv, d = 2, 6, 3, 11, 16
    rng = np.random.default_rng(53)
    kq = rng.integers(0, 256, (B, Hkv, Skv, d // 2), dtype=np.uint8)
    vq = rng.integers(0, 256, (B, Hkv, Skv, d // 2), dtype=np.uint8)
    ks = rng.uniform(0.05, 2, (B, Hkv, Skv)).astype(np.float32)
    vs = rng.uniform(0.05, 2, (B, Hkv, Skv)).astype(np.float32)
    q = _rand((B, Hq, d), 54)
    o, lse = oracle.decode_int4(q, kq, ks, vq, vs, scale=0.2, lib=lib)
    kd = _unpack_int4(kq).astype(np.float64) * ks.astype(np.float64)[..., None]
    vd = _unpack_int4(vq).astype(np.float64) * vs.astype(np.float64)[..., None]
    ob, lb = brute_force(q[:, None], kd.transpose(0, 2, 1, 3), vd.transpose(0, 2, 1, 3), False, 0, 0.2)
    assert np.allclose(o, ob[:, 0], atol=1e-12, rtol=0) and np.allclose(lse, lb[:, :, 0], atol=1e-12, rtol=0)


def pin_int4_quantizer_rounding_packing_and_bounds(lib):
    # absmax 7 gives scale exactly 1: codes are round-half-even of the values
    x = np.zeros((1, 1, 1, 8), dtype=np.float32)
    x[0, 0, 0] = [7.0, 2.5, 3.5, -2.5, -3.5, 0.5, -6.5, 1.25]
    c, sc = oracle.kv_quantize_int4(x, lib=lib)
    assert sc[0, 0, 0] == np.float32(1.0)
    # codes 7, 2 | 4, -2 | -4, 0 | -6, 1 packed low nibble first
    assert list(c[0, 0, 0]) == [0x27, 0xE4, 0x0C, 0x1A]
    rng = np.random.default_rng(55)
    x = rng.standard_normal((2, 4, 3, 32)).astype(np.float32) * rng.uniform(0.01, 100, (2, 4, 3, 1)).astype(np.float32)
    x[0, 3, 2] = 0.0
    codes = np.full((2, 3, 7, 16), 0xAB, dtype=np.uint8)
    scales = np.full((2, 3, 7), -1.0, dtype=np.float32)
    oracle.kv_quantize_int4(x, codes, scales, pos=2, cap=7, lib=lib)
    assert np.all(codes[:, :, :2] == 0xAB) and np.all(codes[:, :, 6:] == 0xAB)
    assert np.all(scales[:, :, :2] == -1) and np.all(scales[:, :, 6:] == -1)
    got_c = _unpack_int4(codes[:, :, 2:6]).transpose(0, 2, 1, 3)  # -> [B, T, Hkv, d]
    got_s = scales[:, :, 2:6].transpose(0, 2, 1)
    assert got_s[0, 3, 2] == 0 and np.all(got_c[0, 3, 2] == 0)
    amax = np.abs(x).max(-1)
    nz = amax > 0
    assert np.all(np.abs(got_c[nz]).max(-1) == 7) and np.all(np.abs(got_c) <= 7)
    deq = got_c * got_s[..., None].astype(np.float64)
    assert np.all(np.abs(deq - x) <= 0.5 * got_s[..., None] * (1 + 1e-6) + 1e-30)
    assert np.allclose(got_s[nz], amax[nz] / 7.0, rtol=1e-7, atol=0)


def pin_int4_quantizer_matches_torch(lib):
    import workloads as W
    g = torch.Generator().manual_seed(56)
    x = torch.randn(2, 9, 3, 64, generator=g) * 5
    x[1, 4, 0] = 0
    c_ref, s_ref = W.quantize_rows_int4(x)
    c, sc = oracle.kv_quantize_int4(x.numpy(), lib=lib)
    assert np.array_equal(c.transpose(0, 2, 1, 3), c_ref.numpy())
    assert np.array_equal(sc.transpose(0, 2, 1), s_ref.numpy())


def brute_force_varlen(q, k, v, cu_q, cu_k, causal, window, scale):
    """Full packed [total_q, total_k] score matrix with a block-diagonal mask:
    query row i and key row j interact only inside the same sequence."""
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[:2]
    G = Hq // Hkv
    cu_q, cu_k = np.asarray(cu_q), np.asarray(cu_k)
    sq_of = np.searchsorted(cu_q, np.arange(total_q), side="right") - 1
    sk_of = np.searchsorted(cu_k, np.arange(total_k), side="right") - 1
    pq = np.arange(total_q) - cu_q[sq_of]
    pk = np.arange(total_k) - cu_k[sk_of]
    off = (cu_k[sq_of + 1] - cu_k[sq_of]) - (cu_q[sq_of + 1] - cu_q[sq_of])
    vis = sq_of[:, None] == sk_of[None, :]
    if causal:
        vis &= pk[None, :] <= pq[:, None] + off[:, None]
        if window:
            vis &= pk[None, :] > pq[:, None] + off[:, None] - window
    o = np.zeros((total_q, Hq, d))
    lse = np.full((Hq, total_q), -np.inf)
    for h in range(Hq):
        s = np.where(vis, scale * (q[:, h] @ k[:, h // G].T), -np.inf)
        m = s.max(axis=1, keepdims=True)
        ok = np.isfinite(m[:, 0])
        e = np.where(vis, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
        l = e.sum(axis=1, keepdims=True)
        o[:, h] = np.divide(e, l, out=np.zeros_like(e), where=l > 0) @ v[:, h // G]
        lse[h, ok] = (m[:, 0] + np.log(l[:, 0]))[ok]
    return o, lse


def pin_varlen_block_diagonal_brute_force(lib):
    # lengths with an empty query sequence, Sq < Skv and Sq > Skv (bottom-right
    # alignment per sequence), a key-less sequence, GQA
    lq = [5, 0, 3, 9, 4, 2]
    lk = [5, 2, 7, 6, 0, 2]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    Hq, Hkv, d = 4, 2, 8
    q = _rand((cu_q[-1], Hq, d), 57)
    k, v = _rand((cu_k[-1], Hkv, d), 58), _rand((cu_k[-1], Hkv, d), 59)
    for causal, window in ((False, 0), (True, 0), (True, 3)):
        o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_k, causal=causal, window=window, scale=0.35, lib=lib)
        ob, lb = brute_force_varlen(q, k, v, cu_q, cu_k, causal, window, 0.35)
        assert np.allclose(o, ob, atol=1e-12, rtol=0)
        assert np.array_equal(np.isfinite(lse), np.isfinite(lb))
        assert np.allclose(lse[np.isfinite(lb)], lb[np.isfinite(lb)], atol=1e-12, rtol=0)
    # the key-less sequence (index 4): o = 0, lse = -inf
    rows4 = slice(cu_q[4], cu_q[5])
    assert np.all(o[rows4] == 0) and np.all(np.isneginf(lse[:, rows4]))


def pin_varlen_equal_lengths_is_the_batch(lib):
    B, S, Hq, Hkv, d = 3, 6, 4, 1, 8
    q, k, v = _rand((B, S, Hq, d), 60), _rand((B, S, Hkv, d), 61), _rand((B, S, Hkv, d), 62)
    cu = np.arange(B + 1) * S
    for causal in (False, True):
        o, lse = oracle.fwd_varlen(q.reshape(B * S, Hq, d), k.reshape(B * S, Hkv, d),
                                   v.reshape(B * S, Hkv, d), cu, cu, causal=causal, lib=lib)
        ob, lb = oracle.fwd(q, k, v, causal=causal, lib=lib)
        assert np.array_equal(o, ob.reshape(B * S, Hq, d))
        assert np.array_equal(lse, lb.transpose(1, 0, 2).reshape(Hq, B * S))


def pin_decode_seqlens_attend_to_the_prefix(lib):
    B, Hq, Hkv, Skv, d = 3, 4, 2, 13, 8
    q = _rand((B, Hq, d), 63)
    kq, ks = _quantise(_rand((B, Hkv, Skv, d), 64))
    vq, vs = _quantise(_rand((B, Hkv, Skv, d), 65))
    lens = np.array([13, 0, 5], dtype=np.int32)
    o, lse = oracle.decode_int8(q, kq, ks, vq, vs, scale=0.3, seqlens=lens, lib=lib)
    kd = kq.astype(np.float64) * ks.astype(np.float64)[..., None]
    vd = vq.astype(np.float64) * vs.astype(np.float64)[..., None]
    for b in range(B):
        L = lens[b]
        if L == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        ob, lb = brute_force(q[b:b + 1, None], kd[b:b + 1, :, :L].transpose(0, 2, 1, 3),
                             vd[b:b + 1, :, :L].transpose(0, 2, 1, 3), False, 0, 0.3)
        assert np.allclose(o[b], ob[0, 0], atol=1e-12, rtol=0)
        assert np.allclose(lse[b], lb[0, :, 0], atol=1e-12, rtol=0)
    # int4: same prefix rule
    k4 = np.random.default_rng(66).integers(0, 256, (B, Hkv, Skv, d // 2), dtype=np.uint8)
    o4, l4 = oracle.decode_int4(q, k4, ks, k4, vs, scale=0.3, seqlens=lens, lib=lib)
    o4f, l4f = oracle.decode_int4(q[2:3], k4[2:3, :, :5].copy(), ks[2:3, :, :5].copy(),
                                  k4[2:3, :, :5].copy(), vs[2:3, :, :5].copy(), scale=0.3, lib=lib)
    assert np.array_equal(o4[2], o4f[0]) and np.array_equal(l4[2], l4f[0])
    assert np.all(o4[1] == 0) and np.all(np.isneginf(l4[1]))


def pin_bwd_finite_differences(lib):
    # L = sum(O * dO) through the (separately pinned) forward oracle; central
    # differences of L give every element of dq, dk, dv.  GQA, bottom-right causal
    # with Sq > Skv (two rows see no key), and a window.
    B, Sq, Skv, Hq, Hkv, d = 1, 5, 4, 4, 2, 3
    q, k, v = _rand((B, Sq, Hq, d), 67), _rand((B, Skv, Hkv, d), 68), _rand((B, Skv, Hkv, d), 69)
    do = _rand((B, Sq, Hq, d), 70)
    for causal, window in ((False, 0), (True, 0), (True, 2)):
        dq, dk, dv = oracle.bwd(q, k, v, do, causal=causal, window=window, scale=0.8, lib=lib)

        def loss(qq, kk, vv):
            o, _ = oracle.fwd(qq, kk, vv, causal=causal, window=window, scale=0.8)
            return float((o * do).sum())
        eps = 1e-5
        for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert np.allclose(g, num, atol=1e-8, rtol=1e-6), (causal, window, which)
        if causal and Sq > Skv:
            assert np.all(dq[0, :Sq - Skv] == 0)  # rows with no visible key


def pin_bwd_torch_autograd_float64(lib):
    # an independent library: torch autograd through its float64 math attention,
    # GQA via repeat_interleave (its backward sums the repeated heads); Sq = Skv.
    B, S, Hq, Hkv, d = 2, 9, 4, 2, 8
    q, k, v, do = _rand((B, S, Hq, d), 71), _rand((B, S, Hkv, d), 72), _rand((B, S, Hkv, d), 73), _rand((B, S, Hq, d), 74)
    for causal in (False, True):
        dq, dk, dv = oracle.bwd(q, k, v, do, causal=causal, lib=lib)
        t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3).clone().requires_grad_()
        tq, tk, tv = t(q), t(k), t(v)
        rk, rv = tk.repeat_interleave(Hq // Hkv, dim=1), tv.repeat_interleave(Hq // Hkv, dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(tq, rk, rv, is_causal=causal)
        (o * torch.from_numpy(do).permute(0, 2, 1, 3)).sum().backward()
        back = lambda g: g.permute(0, 2, 1, 3).numpy()
        assert np.allclose(dq, back(tq.grad), atol=1e-12, rtol=0)
        assert np.allclose(dk, back(tk.grad), atol=1e-12, rtol=0)
        assert np.allclose(dv, back(tv.grad), atol=1e-12, rtol=0)


def pin_bwd_sum_invariants(lib):
    # each row's probabilities sum to 1 and its dS row sums to 0, so over the keys
    # of a kv head: sum_j dK_j = 0 and sum_j dV_j = sum of dO over its query rows
    # that see a key.
    B, Sq, Skv, Hq, Hkv, d = 2, 7, 9, 6, 3, 5
    q, k, v = _rand((B, Sq, Hq, d), 75), _rand((B, Skv, Hkv, d), 76), _rand((B, Skv, Hkv, d), 77)
    do = _rand((B, Sq, Hq, d), 78)
    for causal, window in ((False, 0), (True, 0), (True, 3)):
        dq, dk, dv = oracle.bwd(q, k, v, do, causal=causal, window=window, lib=lib)
        assert np.allclose(dk.sum(axis=1), 0, atol=1e-12)
        want = do.reshape(B, Sq, Hkv, Hq // Hkv, d).sum(axis=(1, 3))
        assert np.allclose(dv.sum(axis=1), want, atol=1e-12)


def pin_bwd_stored_output(lib):
    # D formed from a stored output: with the exact output it must give the
    # default result (D_i = sum_j P_ij dP_ij = dO_i . O_i); moving one stored
    # element O_ic by delta moves D_i by delta dO_ic, hence dQ_i by
    # -scale delta dO_ic sum_j P_ij K_j (the forward with V := K gives that sum)
    # and leaves other rows' dQ and every dV unchanged.  GQA, Sq > Skv, window.
    B, Sq, Skv, Hq, Hkv, d = 2, 7, 5, 4, 2, 6
    q, k, v = _rand((B, Sq, Hq, d), 79), _rand((B, Skv, Hkv, d), 80), _rand((B, Skv, Hkv, d), 81)
    do = _rand((B, Sq, Hq, d), 82)
    for causal, window in ((False, 0), (True, 0), (True, 2)):
        o, _ = oracle.fwd(q, k, v, causal=causal, window=window, scale=0.7)
        ref = oracle.bwd(q, k, v, do, causal=causal, window=window, scale=0.7, lib=lib)
        got = oracle.bwd(q, k, v, do, causal=causal, window=window, scale=0.7, o=o, lib=lib)
        for a, r in zip(got, ref):
            assert np.allclose(a, r, atol=1e-12, rtol=0), (causal, window)
        b, i, h, c, delta = 1, Sq - 1, 3, 2, 0.25
        o2 = o.copy()
        o2[b, i, h, c] += delta
        dq2, _, dv2 = oracle.bwd(q, k, v, do, causal=causal, window=window, scale=0.7, o=o2, lib=lib)
        pk, _ = oracle.fwd(q, k, k, causal=causal, window=window, scale=0.7)
        want = got[0].copy()
        want[b, i, h] -= 0.7 * delta * do[b, i, h, c] * pk[b, i, h]
        assert np.allclose(dq2, want, atol=1e-12, rtol=0), (causal, window)
        assert np.allclose(dv2, got[2], atol=1e-12, rtol=0)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(None)


# ----------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle source must fail some pin
# ----------------------------------------------------------------------------

MUTANTS = {
    "gqa head h % Hkv": ("i = rows[3 * r + 2];\n      int64_t hk = h / group;",
                         "i = rows[3 * r + 2];\n      int64_t hk = h % Hkv;"),
    "varlen gqa head h % Hkv": ("cu_k[b];\n      int64_t hk = h / group;", "cu_k[b];\n      int64_t hk = h % Hkv;"),
    "scale dropped": ("s[j - jlo] = scale * acc;", "s[j - jlo] = acc;"),
    "causal excludes the diagonal": ("hi = last + 1;", "hi = last;"),
    "window keeps W+1 keys": ("lo = last - window + 1;", "lo = last - window;"),
    "lse without max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "no normalisation": ("double p = s[j - jlo] / l;", "double p = s[j - jlo];"),
    "exp sign flipped": ("s[j - jlo] = exp(s[j - jlo] - m);", "s[j - jlo] = exp(m - s[j - jlo]);"),
    "k batch offset dropped": ("const double* kb = k + (b * Skv * Hkv + hk) * (int64_t)d;",
                               "const double* kb = k + (hk) * (int64_t)d;"),
    "v reads the key rows": ("const double* vb = v + (b * Skv * Hkv + hk) * (int64_t)d;",
                             "const double* vb = k + (b * Skv * Hkv + hk) * (int64_t)d;"),
    "q head stride transposed": ("const double* qrow = q + ((b * Sq + i) * Hq + h) * (int64_t)d;",
                                 "const double* qrow = q + ((b * Hq + h) * Sq + i) * (int64_t)d;"),
    "top-left causal alignment": ("int64_t off = (int64_t)Skv - (int64_t)Sq;", "int64_t off = 0;"),
    "decode ignores k scale": ("double sc = (double)ks[j];", "double sc = 1.0;"),
    "decode v uses k codes": ("const uint8_t* vr = vq + j * row_bytes;", "const uint8_t* vr = kq + j * row_bytes;"),
    "quantiser step absmax/128": ("cap, 127.0f, 8);", "cap, 128.0f, 8);"),
    "int4 quantiser step absmax/8": ("cap, 7.0f, 4);", "cap, 8.0f, 4);"),
    "int4 nibbles swapped": ("(c % 2 == 0) ? (int)(row[c / 2] & 15u) : (int)(row[c / 2] >> 4);",
                             "(c % 2 == 0) ? (int)(row[c / 2] >> 4) : (int)(row[c / 2] & 15u);"),
    "int4 codes read unsigned": ("if (nib >= 8) nib -= 16;", "if (nib >= 16) nib -= 16;"),
    "int4 rows strided like int8": ("const int64_t row_bytes = bits == 8 ? d : d / 2;",
                                    "const int64_t row_bytes = d;"),
    "int4 packing high nibble first": ("(c % 2 == 0 ? nib : nib << 4)", "(c % 2 == 0 ? nib << 4 : nib)"),
    "varlen positions not relative to the sequence": ("visible_range(i - cu_q[b], sq, skv,",
                                                      "visible_range(i, sq, skv,"),
    "varlen row lookup off by one": ("while (cu_q[b + 1] <= i) b++;", "while (cu_q[b + 1] < i) b++;"),
    "varlen keys of the first sequence": ("const double* kb = k + ((int64_t)cu_k[b] * Hkv + hk) * (int64_t)d;",
                                          "const double* kb = k + ((int64_t)cu_k[0] * Hkv + hk) * (int64_t)d;"),
    "decode ignores seqlens": ("int64_t len = seqlens ? seqlens[b] : Skv;", "int64_t len = Skv;"),
    "bwd D from unnormalised weights": ("D += p[j - jlo] * acc;", "D += acc;"),
    "bwd dq without scale": ("dqi[c] += scale * dsq * kh[j * kv_stride + c];", "dqi[c] += dsq * kh[j * kv_stride + c];"),
    "bwd dS sign flipped in dk": ("double dsk = pij * (dpij - row_d[r]);", "double dsk = pij * (row_d[r] - dpij);"),
    "bwd dS sign flipped in dq": ("double dsq = p[j - jlo] * (dp[j - jlo] - D);", "double dsq = p[j - jlo] * (D - dp[j - jlo]);"),
    "bwd weights without lse": ("double pij = exp(scale * s - row_lse[r]);", "double pij = exp(scale * s);"),
    "bwd dk from k": ("dkj[c] += scale * dsk * qi[c];", "dkj[c] += scale * dsk * kj[c];"),
    "bwd dv from q": ("dvj[c] += pij * doi[c];", "dvj[c] += pij * qi[c];"),
    "bwd stored output without dout": ("for (c = 0; c < d; c++) Do += doi[c] * oi[c];", "for (c = 0; c < d; c++) Do += oi[c];"),
    "bwd stored output of head 0": ("const double* oi = o + ((b * Sq + i) * Hq + h) * (int64_t)d;",
                                    "const double* oi = o + ((b * Sq + i) * Hq) * (int64_t)d;"),
    "quantiser rounds half away from zero": ("float r = rintf(qv);", "float r = roundf(qv);"),
    "quantiser ignores the append position": ("int64_t slot = (b * Hkv + h) * (int64_t)cap + pos + t;",
                                             "int64_t slot = (b * Hkv + h) * (int64_t)cap + t;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not unique in oracle.c: {old!r}"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.compile_source(path, os.path.join(tmp, "libmutant.so"))
        caught = []
        for pin in PINS:
            try:
                pin(lib)
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
        assert caught, f"no pin fails on the mutant '{name}'"
