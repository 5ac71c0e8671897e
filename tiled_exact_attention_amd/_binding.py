"""ctypes marshalling for libfattn (argument checks and pointers only).

The raw entry points (``fattn_fwd``, ``fattn_fwd_varlen``, ``fattn_bwd``,
``fattn_bwd_workspace_size``, ``fattn_decode_int8``,
``fattn_decode_int4``, their ``_varlen`` forms, ``fattn_decode_int8_noalloc``, ``fattn_kv_append_int8``,
``fattn_kv_append_int4``,
``fattn_decode_workspace_size``, ``fattn_decode_num_splits``,
``fattn_status_string``, ``fattn_version``) have the C names and take plain
integers (device pointers as ints, streams as ints or None).  ``fwd``, ``fwd_varlen``, ``bwd``,
``decode_int8``, ``decode_int4``, ``kv_append_int8`` and ``kv_append_int4``
accept torch tensors, allocate the outputs and call them on the current torch
stream of the tensors' device.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfattn.so")
_lib = None

FATTN_F32 = 0
FATTN_BF16 = 1


class FattnError(RuntimeError):
    """A libfattn call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fattn_status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def load():
    """Loads libfattn.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it first with "
                "`python -m tiled_exact_attention_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.fattn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                  f32, i32, i32, i32, vp]
        lib.fattn_fwd.restype = i32
        lib.fattn_decode_int8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                          f32, i32, vp, sz, vp]
        lib.fattn_decode_int8.restype = i32
        lib.fattn_decode_int4.argtypes = lib.fattn_decode_int8.argtypes
        lib.fattn_decode_int4.restype = i32
        lib.fattn_decode_int8_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                  f32, i32, vp]
        lib.fattn_decode_int8_noalloc.restype = i32
        lib.fattn_bwd.argtypes = [vp] * 9 + [i32] * 6 + [f32, i32, i32, i32, vp, sz, vp]
        lib.fattn_bwd.restype = i32
        lib.fattn_bwd_workspace_size.argtypes = [i32] * 6
        lib.fattn_bwd_workspace_size.restype = sz
        lib.fattn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, f32, i32, i32, i32, vp]
        lib.fattn_fwd_varlen.restype = i32
        for f in (lib.fattn_decode_int8_varlen, lib.fattn_decode_int4_varlen):
            f.argtypes = [vp] * 8 + [i32] * 5 + [f32, i32, vp, sz, vp]
            f.restype = i32
        lib.fattn_kv_append_int8.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
        lib.fattn_kv_append_int8.restype = i32
        lib.fattn_kv_append_int4.argtypes = lib.fattn_kv_append_int8.argtypes
        lib.fattn_kv_append_int4.restype = i32
        lib.fattn_decode_num_splits.argtypes = [i32] * 6
        lib.fattn_decode_num_splits.restype = i32
        lib.fattn_decode_workspace_size.argtypes = [i32] * 6
        lib.fattn_decode_workspace_size.restype = sz
        lib.fattn_status_string.argtypes = [i32]
        lib.fattn_status_string.restype = ctypes.c_char_p
        lib.fattn_version.argtypes = []
        lib.fattn_version.restype = i32
        _lib = lib
    return _lib


# ---------------------------------------------------------------- raw C names

def fattn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, window, dtype, stream) -> int:
    return load().fattn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, window,
                            dtype, stream)


def fattn_decode_int8(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale,
                      num_splits, workspace, workspace_bytes, stream) -> int:
    return load().fattn_decode_int8(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d,
                                    scale, num_splits, workspace, workspace_bytes, stream)


def fattn_decode_int8_noalloc(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale,
                              num_splits, stream) -> int:
    return load().fattn_decode_int8_noalloc(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d,
                                            scale, num_splits, stream)


def fattn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Skv, d, scale, causal, window,
              dtype, workspace, workspace_bytes, stream) -> int:
    return load().fattn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Skv, d, scale, causal,
                            window, dtype, workspace, workspace_bytes, stream)


def fattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, d) -> int:
    return load().fattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, d)


def fattn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k,
                     max_seqlen_q, d, scale, causal, window, dtype, stream) -> int:
    return load().fattn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q,
                                   total_k, max_seqlen_q, d, scale, causal, window, dtype, stream)


def fattn_decode_int8_varlen(q, kq, k_scale, vq, v_scale, seqlens, o, lse, B, Hq, Hkv, Skv, d,
                             scale, num_splits, workspace, workspace_bytes, stream) -> int:
    return load().fattn_decode_int8_varlen(q, kq, k_scale, vq, v_scale, seqlens, o, lse, B, Hq, Hkv,
                                           Skv, d, scale, num_splits, workspace, workspace_bytes,
                                           stream)


def fattn_decode_int4_varlen(q, kq, k_scale, vq, v_scale, seqlens, o, lse, B, Hq, Hkv, Skv, d,
                             scale, num_splits, workspace, workspace_bytes, stream) -> int:
    return load().fattn_decode_int4_varlen(q, kq, k_scale, vq, v_scale, seqlens, o, lse, B, Hq, Hkv,
                                           Skv, d, scale, num_splits, workspace, workspace_bytes,
                                           stream)


def fattn_decode_int4(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale,
                      num_splits, workspace, workspace_bytes, stream) -> int:
    return load().fattn_decode_int4(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d,
                                    scale, num_splits, workspace, workspace_bytes, stream)


def fattn_kv_append_int8(x, codes, scales, B, T, Hkv, d, pos, cap, dtype, stream) -> int:
    return load().fattn_kv_append_int8(x, codes, scales, B, T, Hkv, d, pos, cap, dtype, stream)


def fattn_kv_append_int4(x, codes, scales, B, T, Hkv, d, pos, cap, dtype, stream) -> int:
    return load().fattn_kv_append_int4(x, codes, scales, B, T, Hkv, d, pos, cap, dtype, stream)


def fattn_decode_num_splits(B, Hq, Hkv, Skv, d, num_splits) -> int:
    return load().fattn_decode_num_splits(B, Hq, Hkv, Skv, d, num_splits)


def fattn_decode_workspace_size(B, Hq, Hkv, Skv, d, num_splits) -> int:
    return load().fattn_decode_workspace_size(B, Hq, Hkv, Skv, d, num_splits)


def fattn_status_string(status: int) -> str:
    return load().fattn_status_string(int(status)).decode()


def fattn_version() -> int:
    return load().fattn_version()


# ------------------------------------------------------------- torch wrappers

def _check(t, name, dtype, ndim, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_of(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def fwd(q, k, v, *, causal: bool = False, window: int = 0, scale: float | None = None,
        return_lse: bool = False, out=None):
    """Exact attention o = softmax(scale*q@k^T + mask) @ v (see fattn_fwd).

    q [B, Sq, Hq, d], k/v [B, Skv, Hkv, d], all float32 or all bfloat16,
    contiguous, on one GPU.  Returns o shaped like q (and lse [B, Hq, Sq] fp32).
    """
    import torch
    dtype = q.dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _check(q, "q", dtype, 4)
    _check(k, "k", dtype, 4, q.device)
    _check(v, "v", dtype, 4, q.device)
    B, Sq, Hq, d = q.shape
    Bk, Skv, Hkv, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dtype, 4, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    with torch.cuda.device(q.device):
        st = fattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       lse.data_ptr() if lse is not None else None,
                       B, Hq, Hkv, Sq, Skv, d, float(scale), int(bool(causal)), int(window),
                       FATTN_F32 if dtype == torch.float32 else FATTN_BF16, _stream_of(q.device))
    if st != 0:
        raise FattnError(st, "fattn_fwd")
    return (out, lse) if return_lse else out


def bwd(q, k, v, o, lse, dout, *, causal: bool = False, window: int = 0, scale: float | None = None,
        workspace=None, out=None):
    """Gradients (dq, dk, dv) of fwd for an upstream gradient dout (see fattn_bwd).

    q, o, dout [B, Sq, Hq, d] and k, v [B, Skv, Hkv, d] bfloat16, lse [B, Hq, Sq]
    float32 from fwd(..., return_lse=True) with the same causal / window / scale.
    workspace: optional uint8 GPU tensor of at least fattn_bwd_workspace_size
    bytes.  out: optional (dq, dk, dv) tensors to write.  Returns (dq, dk, dv).
    """
    import torch
    _check(q, "q", torch.bfloat16, 4)
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, n, torch.bfloat16, 4, dev)
    _check(lse, "lse", torch.float32, 3, dev)
    B, Sq, Hq, d = q.shape
    Bk, Skv, Hkv, dk_ = k.shape
    if Bk != B or dk_ != d or tuple(v.shape) != tuple(k.shape) or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o and dout")
    if tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be [B, Hq, Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, d)
    if need == 0:
        raise FattnError(-1, "fattn_bwd_workspace_size")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check(t, n, torch.bfloat16, 4, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have the shape of {n[1:]}")
    with torch.cuda.device(dev):
        st = fattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Sq,
                       Skv, d, float(scale), int(bool(causal)), int(window), FATTN_BF16,
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                       _stream_of(dev))
    if st != 0:
        raise FattnError(st, "fattn_bwd")
    return dq, dk, dv


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, max_seqlen_q: int | None = None,
               causal: bool = False, window: int = 0, scale: float | None = None,
               return_lse: bool = False, out=None):
    """Exact attention over a packed batch of variable-length sequences (see
    fattn_fwd_varlen).

    q [total_q, Hq, d], k/v [total_k, Hkv, d], all float32 or all bfloat16;
    cu_seqlens_q / cu_seqlens_k: int32 GPU tensors [B+1].  max_seqlen_q: the
    longest query sequence (computed from cu_seqlens_q with a device sync if
    None).  Returns o like q (and lse [Hq, total_q] fp32).
    """
    import torch
    dtype = q.dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _check(q, "q", dtype, 3)
    _check(k, "k", dtype, 3, q.device)
    _check(v, "v", dtype, 3, q.device)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, q.device)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, q.device)
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    if dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    B = cu_seqlens_q.numel() - 1
    if B < 1 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B+1 offsets, B >= 1")
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max()) if total_q else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dtype, 3, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if return_lse else None
    with torch.cuda.device(q.device):
        st = fattn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr() if lse is not None else None,
                              cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv,
                              total_q, total_k, int(max_seqlen_q), d, float(scale),
                              int(bool(causal)), int(window),
                              FATTN_F32 if dtype == torch.float32 else FATTN_BF16, _stream_of(q.device))
    if st != 0:
        raise FattnError(st, "fattn_fwd_varlen")
    return (out, lse) if return_lse else out


def decode_num_splits(B, Hq, Hkv, Skv, d, num_splits=0) -> int:
    n = fattn_decode_num_splits(B, Hq, Hkv, Skv, d, num_splits)
    if n < 1:
        raise FattnError(n, "fattn_decode_num_splits")
    return n


def decode_workspace_size(B, Hq, Hkv, Skv, d, num_splits=0) -> int:
    n = fattn_decode_workspace_size(B, Hq, Hkv, Skv, d, num_splits)
    if n == 0:
        raise FattnError(-1, "fattn_decode_workspace_size")
    return n


def _decode(q, kq, k_scale, vq, v_scale, scale, num_splits, workspace, return_lse, out, bits,
            seqlens=None):
    import torch
    _check(q, "q", torch.bfloat16, 3)
    dev = q.device
    code_t = torch.int8 if bits == 8 else torch.uint8
    _check(kq, "kq", code_t, 4, dev)
    _check(vq, "vq", code_t, 4, dev)
    _check(k_scale, "k_scale", torch.float32, 3, dev)
    _check(v_scale, "v_scale", torch.float32, 3, dev)
    B, Hq, d = q.shape
    Bk, Hkv, Skv, rb = kq.shape
    if Bk != B or rb * (8 // bits) != d or tuple(vq.shape) != tuple(kq.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kq {tuple(kq.shape)}, vq {tuple(vq.shape)}")
    if tuple(k_scale.shape) != (B, Hkv, Skv) or tuple(v_scale.shape) != (B, Hkv, Skv):
        raise ValueError("k_scale and v_scale must be [B, Hkv, Skv]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_size(B, Hq, Hkv, Skv, d, num_splits)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None
    lse_p = lse.data_ptr() if lse is not None else None
    with torch.cuda.device(dev):
        if seqlens is None:
            fn, name = (fattn_decode_int8, "fattn_decode_int8") if bits == 8 else \
                (fattn_decode_int4, "fattn_decode_int4")
            st = fn(q.data_ptr(), kq.data_ptr(), k_scale.data_ptr(), vq.data_ptr(),
                    v_scale.data_ptr(), out.data_ptr(), lse_p, B, Hq, Hkv, Skv, d, float(scale),
                    int(num_splits), workspace.data_ptr(), ws_bytes, _stream_of(dev))
        else:
            _check(seqlens, "seqlens", torch.int32, 1, dev)
            if seqlens.numel() != B:
                raise ValueError("seqlens must hold B lengths")
            fn, name = (fattn_decode_int8_varlen, "fattn_decode_int8_varlen") if bits == 8 else \
                (fattn_decode_int4_varlen, "fattn_decode_int4_varlen")
            st = fn(q.data_ptr(), kq.data_ptr(), k_scale.data_ptr(), vq.data_ptr(),
                    v_scale.data_ptr(), seqlens.data_ptr(), out.data_ptr(), lse_p, B, Hq, Hkv, Skv,
                    d, float(scale), int(num_splits), workspace.data_ptr(), ws_bytes,
                    _stream_of(dev))
    if st != 0:
        raise FattnError(st, name)
    return (out, lse) if return_lse else out


def decode_int8(q, kq, k_scale, vq, v_scale, *, scale: float | None = None, num_splits: int = 0,
                workspace=None, return_lse: bool = False, out=None, seqlens=None):
    """Decode attention of one token over an int8 KV cache (see fattn_decode_int8).

    q [B, Hq, d] bf16; kq/vq [B, Hkv, Skv, d] int8; k_scale/v_scale [B, Hkv, Skv] fp32.
    workspace: optional uint8 GPU tensor of at least decode_workspace_size(...)
    bytes (allocated here if None).  seqlens: optional int32 GPU tensor [B];
    sequence b then attends to its first seqlens[b] tokens (fattn_decode_int8_varlen).
    Returns o [B, Hq, d] bf16 (and lse [B, Hq]).
    """
    return _decode(q, kq, k_scale, vq, v_scale, scale, num_splits, workspace, return_lse, out, 8,
                   seqlens)


def decode_int4(q, kq, k_scale, vq, v_scale, *, scale: float | None = None, num_splits: int = 0,
                workspace=None, return_lse: bool = False, out=None, seqlens=None):
    """Decode attention of one token over an int4 KV cache (see fattn_decode_int4).

    As decode_int8, with kq/vq [B, Hkv, Skv, d/2] uint8 holding two signed
    4-bit codes per byte (element 2i in the low nibble of byte i).
    """
    return _decode(q, kq, k_scale, vq, v_scale, scale, num_splits, workspace, return_lse, out, 4,
                   seqlens)


def _kv_append(x, codes, scales, pos, bits):
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _check(x, "x", x.dtype, 4)
    _check(codes, "codes", torch.int8 if bits == 8 else torch.uint8, 4, x.device)
    _check(scales, "scales", torch.float32, 3, x.device)
    B, T, Hkv, d = x.shape
    Bc, Hc, cap, rb = codes.shape
    if (Bc, Hc, rb * (8 // bits)) != (B, Hkv, d) or tuple(scales.shape) != (B, Hkv, cap):
        raise ValueError(f"cache shapes {tuple(codes.shape)}, {tuple(scales.shape)} do not match x {tuple(x.shape)}")
    fn, name = (fattn_kv_append_int8, "fattn_kv_append_int8") if bits == 8 else \
        (fattn_kv_append_int4, "fattn_kv_append_int4")
    with torch.cuda.device(x.device):
        st = fn(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, T, Hkv, d, int(pos), cap,
                FATTN_F32 if x.dtype == torch.float32 else FATTN_BF16, _stream_of(x.device))
    if st != 0:
        raise FattnError(st, name)
    return codes, scales


def kv_append_int8(x, codes, scales, *, pos: int):
    """Quantise new tokens x [B, T, Hkv, d] (float32 or bfloat16) into the int8
    cache codes [B, Hkv, cap, d] / scales [B, Hkv, cap] at positions pos .. pos+T-1
    (see fattn_kv_append_int8).  Updates codes and scales in place and returns them."""
    return _kv_append(x, codes, scales, pos, 8)


def kv_append_int4(x, codes, scales, *, pos: int):
    """As kv_append_int8 for the int4 cache: codes [B, Hkv, cap, d/2] uint8
    (see fattn_kv_append_int4)."""
    return _kv_append(x, codes, scales, pos, 4)
