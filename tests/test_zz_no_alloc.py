"""fattn_decode_int8_noalloc (partials in the library's built-in scratch) against
fattn_decode_int8 (partials in a caller workspace), through the C ABI: the
same kernels and split plan, so the outputs must be the same bits.  Two calls
in a row on the scratch path, the second with a smaller input (the scratch
keeps the first call's contents), then the on-chip-merge and single-split
plans, which use no scratch at all."""
from __future__ import annotations

import sys

import pytest
import torch

import tiled_exact_attention_amd as fa
import workloads as W
from guard import Guarded

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(B, Hq, Hkv, Skv, d, num_splits, seed, dev):
    q, kq, ks, vq, vs = W.decode_inputs(B, Hq, Hkv, Skv, d, seed=seed, device=dev)
    scale = d ** -0.5
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptrs = [t.data_ptr() for t in (q, kq, ks, vq, vs)]
    outs = []
    for noalloc in (False, True):
        o = Guarded((B, Hq, d), torch.bfloat16, dev, fill=float("nan"))
        lse = Guarded((B, Hq), torch.float32, dev, fill=float("nan"))
        if noalloc:
            st = fa.fattn_decode_int8_noalloc(*ptrs, o.ptr, lse.ptr, B, Hq, Hkv, Skv, d, scale,
                                              num_splits, stream)
        else:
            need = fa.decode_workspace_size(B, Hq, Hkv, Skv, d, num_splits)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            st = fa.fattn_decode_int8(*ptrs, o.ptr, lse.ptr, B, Hq, Hkv, Skv, d, scale, num_splits,
                                      ws.data_ptr(), need, stream)
        assert st == 0, fa.fattn_status_string(st)
        torch.cuda.synchronize()
        o.assert_intact("o")
        lse.assert_intact("lse")
        outs.append((o.t, lse.t))
    return outs


# B, Hq, Hkv, Skv, d, num_splits: the first two merge through partials (more
# than 8 splits), the second smaller than the first; then an 8-split plan
# merged on chip and a single split
CASES = [
    (4, 16, 4, 5000, 128, 20),
    (2, 8, 2, 1000, 64, 12),
    (3, 8, 2, 3000, 128, 0),
    (2, 4, 1, 300, 128, 1),
]


def test_noalloc_decode_equals_the_workspace_decode(cuda_device):
    for i, case in enumerate(CASES):
        _say(f"case noalloc decode {case}")
        nsplit = fa.decode_num_splits(*case[:5], case[5])
        (o_ws, l_ws), (o_na, l_na) = _both(*case, seed=900 + i, dev=cuda_device)
        assert bool(torch.isfinite(o_ws.float()).all()) and bool(torch.isfinite(l_ws).all())
        assert torch.equal(o_ws, o_na), f"{case}: outputs differ"
        assert torch.equal(l_ws, l_na), f"{case}: lse differs"
        _say(f"  {nsplit} splits: bit-identical")
