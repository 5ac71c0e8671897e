"""Builds libfattn.so (the HIP library behind include/fattn.h) for gfx950.

Every HIP source is compiled with hipcc for --offload-arch=gfx950 only and
linked into one shared library next to this file.  Packed fp32 VALU ops are
disabled on purpose (-packed-fp32-ops): they are not needed by these kernels
and keeping them out makes the generated code independent of their behaviour.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfattn.so")
SOURCES = ["fattn_api.cpp", "fwd_f32.hip", "fwd_bf16.hip", "decode_kv.hip", "kv_quant.hip", "bwd_bf16.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libfattn needs ROCm's hipcc to build")


# Code-generation flags shared by the library build and the kernel-resource
# check (the order is kept: hipcc derives its compilation-unit ids from it).
ARCH_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17"]
FEATURE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-I", os.path.join(ROOT, "include")]
DEVICE_FLAGS = ARCH_FLAGS + FEATURE_FLAGS


def _compile(src: str, obj: str) -> None:
    cmd = ([hipcc()] + ARCH_FLAGS + ["-fPIC", "-Wall", "-Wno-unused-result", "-fvisibility=hidden"]
           + FEATURE_FLAGS + ["-c", src, "-o", obj])
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def device_assembly(src: str, out: str) -> None:
    """Compile one HIP source's device code to gfx950 assembly (for the
    register and occupancy report the compiler writes into it)."""
    res = subprocess.run([hipcc()] + DEVICE_FLAGS + ["-S", "--cuda-device-only", src, "-o", out],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {os.path.basename(src)}:\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Compile all sources and link libfattn.so; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        list(ex.map(lambda so: _compile(os.path.join(CSRC, so[0]), so[1]), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs,
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
