"""Build the HIP library libattn_fwd.so for gfx950, in-tree.

    python -m exact_attention_121_amd.build        # or __graft_entry__.build()

The library is compiled with hipcc (cross-compilation works without a GPU)
into ``exact_attention_121_amd/lib/libattn_fwd.so``; object files go to
``exact_attention_121_amd/_build/``.  Every HIP source is compiled with the
packed-fp32 instructions disabled (``-target-feature -packed-fp32-ops``).

Besides the default library, ``build()`` compiles the variants in VARIANTS
into ``lib/variants/libattn_fwd_<name>.so``: the same sources with other
compile-time settings, loaded only by the tests that hold them to the default
build or to the oracle:

* ``paranoid``: -DATTN_PARANOID_SYNC, every copy and LDS access completed and
  a workgroup barrier at each phase boundary of the pipelined loops (the
  race check: its outputs must equal the default build's bit for bit);
* ``bn32``: the runner-up tiles of the offline sweep (32-key tiles at
  head_dim 128; one query block per wave and 64-key tiles at head_dim 64);
* ``pp``: the 8-wave ping-pong form of the head_dim 128 non-causal forward
  (two wave groups a phase apart, operands staged in registers a phase
  ahead), measured slower than the default on gfx950;
the GPU tests hold the last two to the oracle.  It also builds
``lib/libattn_probe.so``, the benchmark's shader-clock probe (sclk_probe.hip).

The sources compile in parallel (one hipcc per source and variant).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libattn_fwd.so")
VARIANT_DIR = os.path.join(LIB_DIR, "variants")
ARCH = "gfx950"

HIP_SOURCES = ["attn_fwd_kernel.hip", "attn_fwd_kernel_d64_one_block.hip", "attn_decode_kernel.hip",
               "attn_bwd_kernel.hip"]
CXX_SOURCES = ["attn_api.cpp"]
DEPS = ["attn_launch.h", "attn_tile.h", os.path.join("..", "..", "include", "attn_fwd.h")]

# name -> (extra hipcc flags, the HIP sources they change; the others are
# shared with the default build)
VARIANTS = {
    "paranoid": (["-DATTN_PARANOID_SYNC"], HIP_SOURCES),
    # the runner-up tiles of the sweep: 32-key tiles at head_dim 128, and at
    # head_dim 64 one 32-row query block per wave with 64-key tiles
    "bn32": (["-DATTN_BN128=32", "-DATTN_QB64=1", "-DATTN_BN64=64", "-DATTN_WG64=0"], ["attn_fwd_kernel.hip"]),
    # the 8-wave ping-pong kernel for the head_dim 128 non-causal forward
    "pp": (["-DATTN_FWD_PP=1"], ["attn_fwd_kernel.hip"]),
}


# The benchmark's shader-clock probe: its own small library, not part of the
# attention path (bench.py loads it; nothing in the package does).
PROBE_SOURCE = "sclk_probe.hip"
PROBE_PATH = os.path.join(LIB_DIR, "libattn_probe.so")


def variant_path(name: str) -> str:
    return os.path.join(VARIANT_DIR, f"libattn_fwd_{name}.so")


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
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(" ".join(cmd), flush=True)
        if res.stdout or res.stderr:
            print(res.stdout + res.stderr, flush=True)


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return min(int(v), 16)
    return max(1, min(8, len(os.sched_getaffinity(0))))


def build(verbose: bool = False, extra_flags=(), variants=True) -> str:
    """Compile every source and link libattn_fwd.so (and the variants unless
    variants is False); returns the default library's path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    compiles = []  # (command, object)
    default_objs = {}
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        compiles.append([hipcc, *hip_flags(extra_flags), "-c", os.path.join(CSRC, src), "-o", obj])
        default_objs[src] = obj
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        compiles.append([hipcc, "-x", "c++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c",
                         os.path.join(CSRC, src), "-o", obj])
        default_objs[src] = obj
    probe_obj = os.path.join(BUILD_DIR, PROBE_SOURCE + ".o")
    compiles.append([hipcc, *hip_flags(extra_flags), "-c", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_obj])
    links = [(LIB_PATH, [default_objs[s] for s in HIP_SOURCES + CXX_SOURCES]), (PROBE_PATH, [probe_obj])]
    if variants:
        os.makedirs(VARIANT_DIR, exist_ok=True)
        for name, (flags, changed) in VARIANTS.items():
            objs = []
            for src in HIP_SOURCES + CXX_SOURCES:
                if src in changed:
                    obj = os.path.join(BUILD_DIR, f"{src}.{name}.o")
                    compiles.append([hipcc, *hip_flags([*extra_flags, *flags]), "-c", os.path.join(CSRC, src),
                                     "-o", obj])
                    objs.append(obj)
                else:
                    objs.append(default_objs[src])
            links.append((variant_path(name), objs))
    with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in compiles]:
            f.result()
    for path, objs in links:
        tmp = path + ".tmp"
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
