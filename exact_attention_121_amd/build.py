"""Build the HIP library libattn_fwd.so for gfx950, in-tree.

    python -m exact_attention_121_amd.build        # or __graft_entry__.build()

The library is compiled with hipcc (cross-compilation works without a GPU)
into ``exact_attention_121_amd/lib/libattn_fwd.so``; object files go to
``exact_attention_121_amd/_build/``.  Every HIP source is compiled with the
packed-fp32 instructions disabled (``-target-feature -packed-fp32-ops``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libattn_fwd.so")
ARCH = "gfx950"

HIP_SOURCES = ["attn_fwd_kernel.hip", "attn_decode_kernel.hip", "attn_bwd_kernel.hip"]
CXX_SOURCES = ["attn_api.cpp"]
DEPS = ["attn_launch.h", "attn_tile.h", os.path.join("..", "..", "include", "attn_fwd.h")]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libattn_fwd.so")


def hip_flags(extra=()) -> list[str]:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", *extra]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose and (res.stdout or res.stderr):
        print(res.stdout + res.stderr, flush=True)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link libattn_fwd.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([hipcc, *hip_flags(extra_flags), "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([hipcc, "-x", "c++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
