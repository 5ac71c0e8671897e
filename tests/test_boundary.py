"""The C-ABI boundary on the CPU: library loads, exports what include/fattn.h
declares, and rejects every invalid argument before touching a device.

Invalid calls use fake (but aligned) device addresses; validation must reject
them before any HIP call.  Those cases only run where no GPU is visible, so a
validation bug can never send a fake pointer to a real device.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

import tiled_exact_attention_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fattn.h")

FATTN_OK, FATTN_EINVAL, FATTN_EUNSUPPORTED, FATTN_EWORKSPACE = 0, -1, -2, -3


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FATTN_API\s+[\w\s\*]+?\b(fattn_\w+)\s*\(", text)))


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are only passed where no GPU can be reached")


def test_library_is_built_and_loads():
    lib = fa.load()
    assert os.path.exists(fa.library_path())
    assert lib is fa.load()


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert names == sorted(["fattn_fwd", "fattn_fwd_varlen", "fattn_bwd", "fattn_bwd_workspace_size",
                            "fattn_decode_int8", "fattn_decode_int4", "fattn_decode_int8_noalloc",
                            "fattn_decode_int8_varlen", "fattn_decode_int4_varlen",
                            "fattn_decode_num_splits", "fattn_decode_workspace_size",
                            "fattn_kv_append_int8", "fattn_kv_append_int4",
                            "fattn_status_string", "fattn_version"])
    lib = ctypes.CDLL(fa.library_path())
    for n in names:
        assert hasattr(lib, n), n
        assert hasattr(fa, n), n  # the binding mirrors the C names


def test_only_declared_symbols_are_exported():
    # internal launchers are hidden; nothing but the C ABI is visible
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    mine = {s for s in syms if "fattn" in s}
    assert mine == set(_declared_functions())


def test_version_and_status_strings():
    assert fa.fattn_version() == 10000
    assert fa.fattn_status_string(0) == "ok"
    for st in (FATTN_EINVAL, FATTN_EUNSUPPORTED, FATTN_EWORKSPACE, -4):
        assert fa.fattn_status_string(st) not in ("ok", "unknown status")
    assert fa.fattn_status_string(12345) == "unknown status"


def _plan(Skv, req, B=1, Hkv=1, Hq=1):
    """Split plan the header documents: chunks of whole 64-token tiles, no empty split;
    automatic = as many splits as keep one round of 2048 resident waves."""
    if req == 0:
        waves_per_split = B * Hkv * (-(-(Hq // Hkv) // 16))
        req = min(max(2048 // waves_per_split, 1), -(-Skv // 256), 1024)
    req = min(req, Skv)
    chunk = -(-Skv // req)
    chunk = -(-chunk // 64) * 64
    return -(-Skv // chunk), chunk


@pytest.mark.parametrize("B,Hq,Hkv,Skv,d,req", [
    (32, 32, 8, 32768, 128, 0), (1, 4, 1, 1, 64, 0), (2, 8, 2, 1000, 128, 7),
    (1, 1, 1, 65, 64, 3), (3, 6, 3, 4097, 128, 16), (1, 2, 2, 64, 64, 64), (4, 4, 4, 70000, 64, 0),
    (1, 40, 2, 100000, 128, 0), (300, 8, 1, 4096, 64, 0)])
def test_split_plan_and_workspace_size(B, Hq, Hkv, Skv, d, req):
    n = fa.decode_num_splits(B, Hq, Hkv, Skv, d, req)
    if req == 0:  # automatic plans never exceed one round of resident waves (unless 1 split)
        assert n == 1 or B * Hkv * (-(-(Hq // Hkv) // 16)) * n <= 2048
    want_n, chunk = _plan(Skv, req, B, Hkv, Hq)
    assert n == want_n
    assert (n - 1) * chunk < Skv <= n * chunk  # every split non-empty
    rows = B * Hq * n
    want_ws = -(-(rows * d * 4) // 256) * 256 + rows * 4
    assert fa.decode_workspace_size(B, Hq, Hkv, Skv, d, req) == want_ws


def test_size_queries_reject_bad_arguments():
    assert fa.fattn_decode_num_splits(1, 3, 2, 10, 64, 0) == FATTN_EINVAL
    assert fa.fattn_decode_num_splits(1, 2, 2, 10, 96, 0) == FATTN_EUNSUPPORTED
    assert fa.fattn_decode_num_splits(1, 2, 2, 0, 64, 0) == FATTN_EINVAL
    assert fa.fattn_decode_num_splits(1, 2, 2, 10, 64, -1) == FATTN_EINVAL
    assert fa.fattn_decode_workspace_size(1, 3, 2, 10, 64, 0) == 0


P = 0x10000  # fake aligned device address


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=2, Sq=8, Skv=8, d=64, scale=0.125,
             causal=0, window=0, dtype=1, stream=None)
    a.update(kw)
    return fa.fattn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                        a["Sq"], a["Skv"], a["d"], a["scale"], a["causal"], a["window"],
                        a["dtype"], a["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,want", [
    (dict(q=None), FATTN_EINVAL), (dict(k=None), FATTN_EINVAL), (dict(v=None), FATTN_EINVAL),
    (dict(o=None), FATTN_EINVAL), (dict(q=P + 8), FATTN_EINVAL), (dict(o=P + 2), FATTN_EINVAL),
    (dict(lse=P + 4), FATTN_EINVAL), (dict(lse=P + 8), FATTN_EINVAL),
    (dict(B=0), FATTN_EINVAL), (dict(Hq=0), FATTN_EINVAL), (dict(Hkv=0), FATTN_EINVAL),
    (dict(Sq=0), FATTN_EINVAL), (dict(Skv=-1), FATTN_EINVAL), (dict(d=0), FATTN_EINVAL),
    (dict(Hq=3, Hkv=2), FATTN_EINVAL), (dict(scale=math.inf), FATTN_EINVAL),
    (dict(scale=math.nan), FATTN_EINVAL), (dict(causal=2), FATTN_EINVAL),
    (dict(window=-1, causal=1), FATTN_EINVAL), (dict(window=4, causal=0), FATTN_EINVAL),
    (dict(d=96), FATTN_EUNSUPPORTED), (dict(d=256), FATTN_EUNSUPPORTED),
    (dict(dtype=2), FATTN_EUNSUPPORTED), (dict(dtype=-1), FATTN_EUNSUPPORTED),
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1, Sq=1 << 12, Skv=4), FATTN_EINVAL),
    # a 64-key tile of 2^18 kv heads x 128 no longer fits 32-bit offsets
    (dict(Hq=1 << 18, Hkv=1 << 18, Sq=1, Skv=1, d=128), FATTN_EINVAL),
    # ... nor do 128 output rows of 2^17 query heads x 128 (one kv head)
    (dict(Hq=1 << 17, Hkv=1, Sq=1, Skv=1, d=128), FATTN_EINVAL),
])
def test_fwd_rejects_before_any_device_work(kw, want):
    assert _fwd(**kw) == want


def _dec(fn=None, **kw):
    a = dict(q=P, kq=P, ks=P, vq=P, vs=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Skv=100, d=128,
             scale=0.1, num_splits=0, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return (fn or fa.fattn_decode_int8)(a["q"], a["kq"], a["ks"], a["vq"], a["vs"], a["o"], a["lse"],
                                        a["B"], a["Hq"], a["Hkv"], a["Skv"], a["d"], a["scale"],
                                        a["num_splits"], a["ws"], a["ws_bytes"], a["stream"])


@no_gpu_only
@pytest.mark.parametrize("fn", ["fattn_decode_int8", "fattn_decode_int4"])
@pytest.mark.parametrize("kw,want", [
    (dict(q=None), FATTN_EINVAL), (dict(kq=None), FATTN_EINVAL), (dict(ks=None), FATTN_EINVAL),
    (dict(vq=None), FATTN_EINVAL), (dict(vs=None), FATTN_EINVAL), (dict(o=None), FATTN_EINVAL),
    (dict(ks=P + 4), FATTN_EINVAL), (dict(lse=P + 4), FATTN_EINVAL),
    (dict(B=0), FATTN_EINVAL), (dict(Hq=3), FATTN_EINVAL), (dict(Skv=0), FATTN_EINVAL),
    (dict(scale=-math.inf), FATTN_EINVAL), (dict(num_splits=-2), FATTN_EINVAL),
    (dict(d=32), FATTN_EUNSUPPORTED),
    (dict(ws=None), FATTN_EWORKSPACE), (dict(ws_bytes=16), FATTN_EWORKSPACE),
    (dict(ws=P + 8), FATTN_EWORKSPACE),
])
def test_decode_rejects_before_any_device_work(fn, kw, want):
    assert _dec(getattr(fa, fn), **kw) == want


@no_gpu_only
@pytest.mark.parametrize("fn", ["fattn_decode_int8", "fattn_decode_int4"])
def test_decode_workspace_boundary_is_exact(fn):
    need = fa.decode_workspace_size(1, 4, 2, 100, 128, 0)
    assert _dec(getattr(fa, fn), ws_bytes=need - 1) == FATTN_EWORKSPACE


def test_torch_wrappers_reject_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.fwd(q.half(), q.half(), q.half())


def _app(fn=None, **kw):
    a = dict(x=P, codes=P, scales=P, B=1, T=4, Hkv=2, d=128, pos=0, cap=8, dtype=1, stream=None)
    a.update(kw)
    return (fn or fa.fattn_kv_append_int8)(a["x"], a["codes"], a["scales"], a["B"], a["T"], a["Hkv"],
                                           a["d"], a["pos"], a["cap"], a["dtype"], a["stream"])


@no_gpu_only
@pytest.mark.parametrize("fn", ["fattn_kv_append_int8", "fattn_kv_append_int4"])
@pytest.mark.parametrize("kw,want", [
    (dict(x=None), FATTN_EINVAL), (dict(codes=None), FATTN_EINVAL), (dict(scales=None), FATTN_EINVAL),
    (dict(scales=P + 4), FATTN_EINVAL), (dict(B=0), FATTN_EINVAL), (dict(T=0), FATTN_EINVAL),
    (dict(pos=-1), FATTN_EINVAL), (dict(pos=5), FATTN_EINVAL), (dict(T=9), FATTN_EINVAL),
    (dict(d=96), FATTN_EUNSUPPORTED), (dict(dtype=3), FATTN_EUNSUPPORTED),
])
def test_kv_append_rejects_before_any_device_work(fn, kw, want):
    assert _app(getattr(fa, fn), **kw) == want


def test_int4_wrappers_check_the_packed_shape():
    import torch
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    kq = torch.zeros(1, 2, 10, 64, dtype=torch.uint8)  # unpacked width: wrong for int4
    s = torch.zeros(1, 2, 10)
    with pytest.raises(ValueError):
        fa.decode_int4(q, kq, s, kq, s)  # CPU tensors are rejected before any shape use


def _fwdv(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cq=P, ck=P, B=2, Hq=4, Hkv=2, tq=10, tk=12, mq=6, d=64,
             scale=0.1, causal=1, window=0, dtype=1, stream=None)
    a.update(kw)
    return fa.fattn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["B"],
                               a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"], a["d"], a["scale"],
                               a["causal"], a["window"], a["dtype"], a["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,want", [
    (dict(cq=None), FATTN_EINVAL), (dict(ck=None), FATTN_EINVAL), (dict(q=None), FATTN_EINVAL),
    (dict(cq=P + 2), FATTN_EINVAL), (dict(lse=P + 2), FATTN_EINVAL), (dict(o=P + 4), FATTN_EINVAL),
    (dict(B=0), FATTN_EINVAL), (dict(Hq=3), FATTN_EINVAL), (dict(tq=-1), FATTN_EINVAL),
    (dict(tk=-1), FATTN_EINVAL), (dict(mq=11), FATTN_EINVAL), (dict(mq=0), FATTN_EINVAL),
    (dict(mq=-1), FATTN_EINVAL), (dict(scale=math.nan), FATTN_EINVAL), (dict(causal=3), FATTN_EINVAL),
    (dict(window=5, causal=0), FATTN_EINVAL), (dict(d=32), FATTN_EUNSUPPORTED),
    (dict(dtype=2), FATTN_EUNSUPPORTED),
    (dict(tq=0, mq=0), FATTN_OK),  # an empty batch is valid and launches nothing
    (dict(tq=0, mq=0, q=None, o=None), FATTN_OK),  # ... also with null (empty) tensors
    (dict(k=None), FATTN_EINVAL), (dict(v=None), FATTN_EINVAL),  # keys present, no k / v
    (dict(Hq=1 << 17, Hkv=1, d=128), FATTN_EINVAL),  # output rows past 32-bit offsets
])
def test_fwd_varlen_rejects_before_any_device_work(kw, want):
    assert _fwdv(**kw) == want


@no_gpu_only
@pytest.mark.parametrize("fn", ["fattn_decode_int8_varlen", "fattn_decode_int4_varlen"])
@pytest.mark.parametrize("kw,want", [
    (dict(seqlens=None), FATTN_EINVAL), (dict(seqlens=P + 2), FATTN_EINVAL),
    (dict(q=None), FATTN_EINVAL), (dict(Hq=3), FATTN_EINVAL), (dict(d=96), FATTN_EUNSUPPORTED),
    (dict(ws=None), FATTN_EWORKSPACE),
])
def test_decode_varlen_rejects_before_any_device_work(fn, kw, want):
    a = dict(q=P, kq=P, ks=P, vq=P, vs=P, seqlens=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Skv=100,
             d=128, scale=0.1, num_splits=0, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    st = getattr(fa, fn)(a["q"], a["kq"], a["ks"], a["vq"], a["vs"], a["seqlens"], a["o"], a["lse"],
                         a["B"], a["Hq"], a["Hkv"], a["Skv"], a["d"], a["scale"], a["num_splits"],
                         a["ws"], a["ws_bytes"], a["stream"])
    assert st == want


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Sq=8, Skv=8, d=64,
             scale=0.1, causal=1, window=0, dtype=1, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return fa.fattn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                        a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Skv"], a["d"], a["scale"], a["causal"],
                        a["window"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,want", [
    (dict(q=None), FATTN_EINVAL), (dict(lse=None), FATTN_EINVAL), (dict(do=None), FATTN_EINVAL),
    (dict(dq=None), FATTN_EINVAL), (dict(dv=None), FATTN_EINVAL), (dict(o=P + 8), FATTN_EINVAL),
    (dict(lse=P + 4), FATTN_EINVAL), (dict(Sq=0), FATTN_EINVAL), (dict(Hq=3), FATTN_EINVAL),
    (dict(scale=math.inf), FATTN_EINVAL), (dict(window=3, causal=0), FATTN_EINVAL),
    (dict(dtype=0), FATTN_EUNSUPPORTED), (dict(d=96), FATTN_EUNSUPPORTED),
    (dict(ws=None), FATTN_EWORKSPACE), (dict(ws=P + 8), FATTN_EWORKSPACE), (dict(ws_bytes=16), FATTN_EWORKSPACE),
    (dict(Hq=1 << 17, Hkv=1, Sq=1, Skv=1, d=128), FATTN_EINVAL),  # output rows past 32-bit offsets
])
def test_bwd_rejects_before_any_device_work(kw, want):
    assert _bwd(**kw) == want


def _bwd_splits(B, Hq, Hkv, Skv):
    """Query-head splits of the dK/dV grid the header documents: about 1024 blocks."""
    G = Hq // Hkv
    blocks = B * Hkv * -(-Skv // 128)
    want = min(max(-(-1024 // blocks), 1), G)
    hps = -(-G // want)
    return -(-G // hps)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d", [
    (2, 32, 32, 4096, 4096, 128), (1, 32, 8, 4096, 4096, 128), (1, 232, 1, 2048, 2048, 64),
    (1, 3, 3, 5, 5, 64), (3, 8, 2, 100, 70, 128)])
def test_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, d):
    r256 = lambda n: -(-n // 256) * 256
    ns = _bwd_splits(B, Hq, Hkv, Skv)
    want = 2 * r256(B * Hq * Sq * 4) + (2 * r256(ns * B * Skv * Hkv * d * 4) if ns > 1 else 0)
    assert fa.fattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, d) == want


def test_bwd_workspace_size_rejects_bad_arguments():
    assert fa.fattn_bwd_workspace_size(0, 3, 3, 5, 5, 64) == 0
    assert fa.fattn_bwd_workspace_size(1, 3, 2, 5, 5, 64) == 0
    assert fa.fattn_bwd_workspace_size(1, 2, 2, 5, 5, 96) == 0
    if not _gpu_visible():
        need = fa.fattn_bwd_workspace_size(1, 4, 2, 8, 8, 64)
        assert _bwd(ws_bytes=need - 1) == FATTN_EWORKSPACE


def _dec_noalloc(**kw):
    a = dict(q=P, kq=P, ks=P, vq=P, vs=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Skv=100, d=128,
             scale=0.1, num_splits=0, stream=None)
    a.update(kw)
    return fa.fattn_decode_int8_noalloc(a["q"], a["kq"], a["ks"], a["vq"], a["vs"], a["o"], a["lse"],
                                        a["B"], a["Hq"], a["Hkv"], a["Skv"], a["d"], a["scale"],
                                        a["num_splits"], a["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,want", [
    (dict(q=None), FATTN_EINVAL), (dict(vs=None), FATTN_EINVAL), (dict(lse=P + 4), FATTN_EINVAL),
    (dict(Hq=3), FATTN_EINVAL), (dict(num_splits=-1), FATTN_EINVAL), (dict(d=32), FATTN_EUNSUPPORTED),
    # partials of 1024 heads x 1000 splits x (128 + 1) floats: beyond the built-in 32 MiB
    (dict(Hq=1024, Hkv=1, Skv=1 << 20, num_splits=1000), FATTN_EWORKSPACE),
])
def test_decode_noalloc_rejects_before_any_device_work(kw, want):
    assert _dec_noalloc(**kw) == want


@no_gpu_only
def test_decode_noalloc_scratch_limit_is_the_workspace_size():
    # the built-in scratch holds 32 MiB: a plan whose workspace size is just
    # above it is rejected before any device work; the one below it fits
    limit = 32 << 20
    big = dict(Hq=1024, Hkv=1, Skv=1 << 20)
    assert fa.decode_workspace_size(1, 1024, 1, 1 << 20, 128, 64) > limit
    assert _dec_noalloc(num_splits=64, **big) == FATTN_EWORKSPACE
    assert fa.decode_workspace_size(1, 1024, 1, 1 << 20, 128, 63) <= limit
