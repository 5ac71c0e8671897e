"""Registers, scratch and occupancy of every kernel, from the compiler's report.

The kernels are designed around a number of waves per SIMD (the prefill
pipelines two waves per SIMD at d = 128 and three at d = 64; the dK/dV
backward kernel runs one), and none may spill to scratch memory.  A change
that adds a few registers can silently drop a kernel to fewer resident waves
(the d = 64 prefill kernel uses 149 of the 168 registers that three waves
allow), so this compiles each HIP source's device code to gfx950 assembly and
checks the per-kernel figures hipcc writes there.  CPU only (hipcc
cross-compiles).
"""
from __future__ import annotations

import os
import re

import pytest

from tiled_exact_attention_amd import build as B

# minimum resident waves per SIMD, by kernel name and template arguments
MIN_OCCUPANCY = {
    "fwd_bf16_kernel<64>": 3,
    "fwd_bf16_kernel<128>": 2,
    "fwd_f32_kernel<64>": 2,
    "fwd_f32_kernel<128>": 1,
    # <D, code bits, workgroup form, non-temporal loads>
    "decode_split_kernel<64,8,0,0>": 3,
    "decode_split_kernel<64,8,0,1>": 3,
    "decode_split_kernel<64,8,1,0>": 3,
    "decode_split_kernel<64,8,1,1>": 3,
    "decode_split_kernel<64,4,0,0>": 4,
    "decode_split_kernel<64,4,0,1>": 4,
    "decode_split_kernel<64,4,1,0>": 4,
    "decode_split_kernel<64,4,1,1>": 4,
    "decode_split_kernel<128,8,0,0>": 2,
    "decode_split_kernel<128,8,0,1>": 2,
    "decode_split_kernel<128,8,1,0>": 2,
    "decode_split_kernel<128,8,1,1>": 2,
    "decode_split_kernel<128,4,0,0>": 2,
    "decode_split_kernel<128,4,0,1>": 2,
    "decode_split_kernel<128,4,1,0>": 2,
    "decode_split_kernel<128,4,1,1>": 2,
    "decode_merge_kernel<64>": 8,
    "decode_merge_kernel<128>": 8,
    "bwd_dq_kernel<64>": 3,
    "bwd_dq_kernel<128>": 2,
    "bwd_dkdv_kernel<64>": 2,
    "bwd_dkdv_kernel<128>": 1,
    "bwd_reduce_kernel": 8,
    "kv_quant_kernel": 8,
}


def _short_name(mangled: str) -> str:
    """fattn::(anon)::<name><ints...> from an Itanium-mangled kernel symbol."""
    m = re.search(r"_GLOBAL__N_1\d+(\w+?_kernel)", mangled)
    name = m.group(1)
    if name == "kv_quant_kernel" or name == "bwd_reduce_kernel":
        return name
    ints = re.findall(r"L[ib](\d+)E", mangled)  # int and bool template arguments
    return f"{name}<{','.join(ints)}>"


def _report(asm: str):
    """Per kernel: (NumVgprs, ScratchSize, Occupancy) from the comment block hipcc
    writes after each function's body."""
    out, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.match(r"^; (NumVgprs|ScratchSize|Occupancy): (\d+)", line)
        if m and cur is not None:
            out[cur][m.group(1)] = int(m.group(2))
    return out


HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_kernels_keep_their_occupancy_and_do_not_spill(src, tmp_path):
    asm = os.path.join(tmp_path, src + ".s")
    B.device_assembly(os.path.join(B.CSRC, src), asm)
    report = _report(open(asm).read())
    kernels = {k: v for k, v in report.items() if "_kernel" in k}
    assert kernels, f"no kernels found in {src}"
    for mangled, r in kernels.items():
        name = _short_name(mangled)
        assert r.get("ScratchSize") == 0, f"{name} spills ({r.get('ScratchSize')} bytes of scratch)"
        want = MIN_OCCUPANCY.get(name)
        assert want is not None, f"{name}: no occupancy target listed"
        assert r.get("Occupancy", 0) >= want, \
            f"{name}: {r.get('Occupancy')} waves per SIMD ({r.get('NumVgprs')} VGPRs), designed for {want}"
