"""libfattn: tiled exact attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI declared in ``include/fattn.h``.  Every
step of the computation runs in the HIP kernels of ``libfattn.so``; this
package only checks tensors, allocates outputs with torch (device memory and
streams are all torch is used for) and passes raw pointers.  There is no
fallback: if the library is not built, every call raises.

    import tiled_exact_attention_amd as fa
    o = fa.fwd(q, k, v, causal=True)                 # q [B,S,Hq,d], k/v [B,S,Hkv,d]
    o, lse = fa.decode_int8(q, kq, ks, vq, vs, return_lse=True)
    o = fa.decode_int4(q, k4, ks4, v4, vs4)          # two 4-bit codes per byte
    o = fa.fwd_varlen(q, k, v, cu_q, cu_k, causal=True)  # packed variable-length batch
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)   # backward by recomputation
"""
from ._binding import (  # noqa: F401
    FATTN_BF16,
    FATTN_F32,
    FattnError,
    bwd,
    decode_int4,
    decode_int8,
    decode_num_splits,
    decode_workspace_size,
    fattn_bwd,
    fattn_bwd_workspace_size,
    fattn_decode_int4,
    fattn_decode_int4_varlen,
    fattn_decode_int8,
    fattn_decode_int8_noalloc,
    fattn_decode_int8_varlen,
    fattn_decode_num_splits,
    fattn_decode_workspace_size,
    fattn_fwd,
    fattn_fwd_varlen,
    fattn_kv_append_int4,
    fattn_kv_append_int8,
    fattn_status_string,
    fattn_version,
    fwd,
    fwd_varlen,
    kv_append_int4,
    kv_append_int8,
    library_path,
    load,
)
