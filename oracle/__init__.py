"""fp64 CPU oracle for tiled exact attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``tiled_exact_attention_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
output rows); this module only builds that file with gcc and marshals numpy
arrays through ctypes.  See ``oracle.c`` for the definition it follows and the
readings of the source pages it adopts.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_libs: dict = {}


def compile_source(src: str, out: str) -> str:
    """Compile a C source of the oracle into a shared library with gcc."""
    tmp = f"{out}.tmp{os.getpid()}"  # one per process: concurrent builders do not collide
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _stale() -> bool:
    """liboracle.so missing or older than oracle.c (its signatures may differ)."""
    return not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (no fast-math, no intrinsics)."""
    if force or _stale():
        compile_source(SOURCE, _LIB)
    return _LIB


def _load(path: str | None = None):
    if path is None:
        if _stale():
            build(force=False)
        path = _LIB
    if path not in _libs:
        lib = ctypes.CDLL(path)
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.oracle_fwd_rows.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        f64, i32, i32, vp, i64, vp, vp, i32]
        lib.oracle_fwd_rows.restype = i32
        lib.oracle_decode_int8_rows.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                f64, vp, i64, vp, vp, i32]
        lib.oracle_decode_int8_rows.restype = i32
        lib.oracle_decode_int4_rows.argtypes = lib.oracle_decode_int8_rows.argtypes
        lib.oracle_decode_int4_rows.restype = i32
        lib.oracle_kv_quantize_int8.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32]
        lib.oracle_kv_quantize_int8.restype = i32
        lib.oracle_kv_quantize_int4.argtypes = lib.oracle_kv_quantize_int8.argtypes
        lib.oracle_kv_quantize_int4.restype = i32
        lib.oracle_fwd_varlen_rows.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                               f64, i32, i32, vp, i64, vp, vp, i32]
        lib.oracle_fwd_varlen_rows.restype = i32
        lib.oracle_bwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64, i32, i32,
                                   vp, vp, vp, i32]
        lib.oracle_bwd.restype = i32
        lib.oracle_max_threads.argtypes = [i32]
        lib.oracle_max_threads.restype = i32
        _libs[path] = lib
    return _libs[path]


def _f64(x) -> np.ndarray:
    """Widen to a contiguous float64 array (exact for bf16/fp16/fp32 values)."""
    if hasattr(x, "detach"):  # a torch tensor: widen on its own side, then hand over
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _np(x, dtype) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    a = np.asarray(x)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads(threads: int = 0) -> int:
    """Threads the oracle's OpenMP regions use (threads=0: OpenMP default)."""
    return int(_load().oracle_max_threads(int(threads)))


def fwd(q, k, v, *, causal: bool, window: int = 0, scale: float | None = None,
        rows=None, threads: int = 0, lib: str | None = None):
    """Exact attention in fp64.

    q: [B, Sq, Hq, d]; k, v: [B, Skv, Hkv, d] (any real dtype, widened to fp64).
    rows: None for every output row, else an int array of shape [n, 3] holding
    (b, h, i) triples.  Returns (o, lse): with rows=None o is [B, Sq, Hq, d] and
    lse [B, Hq, Sq]; otherwise o is [n, d] and lse [n].  lse is the natural log
    of the sum over visible keys of exp(scale * q.k).
    lib: path of an alternative build of the oracle source (tests only).
    """
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, d = qd.shape
    Bk, Skv, Hkv, dk = kd.shape
    if (Bk, dk) != (B, d) or vd.shape != kd.shape:
        raise ValueError("shape mismatch between q, k and v")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    full = rows is None
    if full:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Sq), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load(lib).oracle_fwd_rows(_ptr(qd), _ptr(kd), _ptr(vd), B, Hq, Hkv, Sq, Skv, d,
                                 float(scale), int(bool(causal)), int(window),
                                 _ptr(rows), n, _ptr(o), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_fwd_rows rejected its arguments (code {rc})")
    if full:
        o = o.reshape(B, Hq, Sq, d).transpose(0, 2, 1, 3).copy()
        lse = lse.reshape(B, Hq, Sq)
    return o, lse


def bwd(q, k, v, dout, *, causal: bool, window: int = 0, scale: float | None = None,
        o=None, threads: int = 0, lib: str | None = None):
    """Gradients (dq, dk, dv) of exact attention for an upstream gradient dout, in fp64.

    q, dout: [B, Sq, Hq, d]; k, v: [B, Skv, Hkv, d].  dk and dv of a kv head sum
    over the query heads sharing it.  Returns arrays shaped like q, k, v.
    o (optional, like q): a stored forward output; the row term D is then formed
    as dout . o (equal to the default for the exact output, see oracle.c).
    """
    qd, kd, vd, dod = _f64(q), _f64(k), _f64(v), _f64(dout)
    od = None if o is None else _f64(o)
    if od is not None and od.shape != qd.shape:
        raise ValueError("o must be shaped like q")
    B, Sq, Hq, d = qd.shape
    Bk, Skv, Hkv, dk_ = kd.shape
    if (Bk, dk_) != (B, d) or vd.shape != kd.shape or dod.shape != qd.shape:
        raise ValueError("shape mismatch between q, k, v and dout")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.empty_like(qd)
    dk = np.empty_like(kd)
    dv = np.empty_like(vd)
    rc = _load(lib).oracle_bwd(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(dod), None if od is None else _ptr(od),
                               B, Hq, Hkv, Sq, Skv, d,
                               float(scale), int(bool(causal)), int(window),
                               _ptr(dq), _ptr(dk), _ptr(dv), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_bwd rejected its arguments (code {rc})")
    return dq, dk, dv


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: bool, window: int = 0,
               scale: float | None = None, rows=None, threads: int = 0, lib: str | None = None):
    """Exact attention over packed sequences of different lengths, in fp64.

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; cu_seqlens_q / cu_seqlens_k:
    [B+1] cumulative lengths from 0.  Sequence b attends only within itself.
    rows: None for every output row, else an int array [n, 2] of (h, i) pairs
    with i a packed query row.  Returns (o, lse): o [total_q, Hq, d] and lse
    [Hq, total_q], or [n, d] and [n] for explicit rows.
    """
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    total_q, Hq, d = qd.shape
    total_k, Hkv, dk = kd.shape
    if dk != d or vd.shape != kd.shape:
        raise ValueError("shape mismatch between q, k and v")
    cq = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
    ck = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int32))
    if cq.shape != ck.shape or cq.ndim != 1 or cq.size < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    B = cq.size - 1
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    full = rows is None
    if full:
        hh, ii = np.meshgrid(np.arange(Hq), np.arange(total_q), indexing="ij")
        rows = np.stack([hh.ravel(), ii.ravel()], axis=1)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load(lib).oracle_fwd_varlen_rows(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(cq), _ptr(ck), B, Hq,
                                           Hkv, total_q, total_k, d, float(scale),
                                           int(bool(causal)), int(window), _ptr(rows), n,
                                           _ptr(o), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_fwd_varlen_rows rejected its arguments (code {rc})")
    if full:
        o = o.reshape(Hq, total_q, d).transpose(1, 0, 2).copy()
        lse = lse.reshape(Hq, total_q)
    return o, lse


def _decode(q, kq, k_scale, vq, v_scale, scale, rows, threads, lib, bits, seqlens=None):
    qd = _f64(q)
    code_t = np.int8 if bits == 8 else np.uint8
    kqa, vqa = _np(kq, code_t), _np(vq, code_t)
    ksa, vsa = _np(k_scale, np.float32), _np(v_scale, np.float32)
    B, Hq, d = qd.shape
    Bk, Hkv, Skv, rb = kqa.shape
    if Bk != B or rb * (8 // bits) != d or vqa.shape != kqa.shape:
        raise ValueError("shape mismatch between q and the cache")
    if ksa.shape != (B, Hkv, Skv) or vsa.shape != (B, Hkv, Skv):
        raise ValueError("scale arrays must be [B, Hkv, Skv]")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    full = rows is None
    if full:
        bb, hh = np.meshgrid(np.arange(B), np.arange(Hq), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel()], axis=1)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    sl = None
    if seqlens is not None:
        sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
        if sl.shape != (B,):
            raise ValueError("seqlens must be [B]")
    fn = _load(lib).oracle_decode_int8_rows if bits == 8 else _load(lib).oracle_decode_int4_rows
    rc = fn(_ptr(qd), _ptr(kqa), _ptr(ksa), _ptr(vqa), _ptr(vsa), None if sl is None else _ptr(sl),
            B, Hq, Hkv, Skv, d, float(scale), _ptr(rows), n, _ptr(o), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError(f"oracle decode (int{bits}) rejected its arguments (code {rc})")
    if full:
        o = o.reshape(B, Hq, d)
        lse = lse.reshape(B, Hq)
    return o, lse


def decode_int8(q, kq, k_scale, vq, v_scale, *, scale: float | None = None, seqlens=None,
                rows=None, threads: int = 0, lib: str | None = None):
    """Decode attention of one query token over an int8 KV cache, in fp64.

    q: [B, Hq, d] (widened to fp64); kq, vq: [B, Hkv, Skv, d] int8;
    k_scale, v_scale: [B, Hkv, Skv] float32.  Every cached key is visible,
    or with seqlens ([B] ints) the first seqlens[b] keys of sequence b.
    rows: None for all (b, h), else an int array [n, 2] of (b, h) pairs.
    Returns (o, lse) shaped [B, Hq, d] and [B, Hq], or [n, d] and [n].
    lib: path of an alternative build of the oracle source (tests only).
    """
    return _decode(q, kq, k_scale, vq, v_scale, scale, rows, threads, lib, 8, seqlens)


def decode_int4(q, kq, k_scale, vq, v_scale, *, scale: float | None = None, seqlens=None,
                rows=None, threads: int = 0, lib: str | None = None):
    """Decode attention over an int4 KV cache, in fp64 (as decode_int8).

    kq, vq: [B, Hkv, Skv, d/2] uint8, two signed 4-bit codes per byte
    (element 2i in the low nibble of byte i, element 2i+1 in the high one).
    """
    return _decode(q, kq, k_scale, vq, v_scale, scale, rows, threads, lib, 4, seqlens)


def _kv_quantize(x, codes, scales, pos, cap, lib, bits):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    B, T, Hkv, d = xa.shape
    rb = d if bits == 8 else d // 2
    code_t = np.int8 if bits == 8 else np.uint8
    if cap is None:
        cap = pos + T
    if codes is None:
        codes = np.zeros((B, Hkv, cap, rb), dtype=code_t)
    if scales is None:
        scales = np.zeros((B, Hkv, cap), dtype=np.float32)
    if codes.shape != (B, Hkv, cap, rb) or scales.shape != (B, Hkv, cap):
        raise ValueError("cache arrays must be [B, Hkv, cap, row bytes] and [B, Hkv, cap]")
    if codes.dtype != code_t or scales.dtype != np.float32 or not codes.flags.c_contiguous \
            or not scales.flags.c_contiguous:
        raise TypeError(f"codes must be contiguous {np.dtype(code_t)} and scales contiguous float32")
    fn = _load(lib).oracle_kv_quantize_int8 if bits == 8 else _load(lib).oracle_kv_quantize_int4
    rc = fn(_ptr(xa), _ptr(codes), _ptr(scales), B, Hkv, T, d, int(pos), int(cap))
    if rc != 0:
        raise ValueError(f"oracle quantiser (int{bits}) rejected its arguments (code {rc})")
    return codes, scales


def kv_quantize_int8(x, codes=None, scales=None, *, pos: int = 0, cap: int | None = None,
                     lib: str | None = None):
    """Quantise new tokens x [B, T, Hkv, d] into an int8 cache (see oracle.c).

    codes [B, Hkv, cap, d] int8 and scales [B, Hkv, cap] float32 are updated in
    place at positions pos .. pos+T-1 (new zero-filled arrays when None).
    Returns (codes, scales).  x is taken as float32 (exact for bf16 values).
    """
    return _kv_quantize(x, codes, scales, pos, cap, lib, 8)


def kv_quantize_int4(x, codes=None, scales=None, *, pos: int = 0, cap: int | None = None,
                     lib: str | None = None):
    """Quantise new tokens into an int4 cache: scale = absmax/7, codes in [-7, 7],
    codes [B, Hkv, cap, d/2] uint8 packed two per byte (see oracle.c)."""
    return _kv_quantize(x, codes, scales, pos, cap, lib, 4)
