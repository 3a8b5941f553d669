"""Offline tile sweep for the fused forward kernel.

The pages tie the block size to head_dim and the on-chip buffer ([CANN-FA]
section "Key design points") and leave the best block size per sequence
length to CANN's tuning engine ([FA-Infer] section 5, the item on AOE).
This is the same idea for this kernel, offline: rebuild the forward kernel
with other tile choices, check and time each on the GPU, and report the best
per (head_dim, causal) case.

    python -m exact_attention_121_amd.tile_sweep build    # compile the variants (no GPU needed)
    python -m exact_attention_121_amd.tile_sweep run      # check and time them on cuda:0
    (--dims 96,160 restricts either step to those head_dims)

Choices swept (the compile-time hooks of csrc/attn_tile.h, per head_dim):
keys per K/V tile (ATTN_BN*), matrix operands read ahead of their MFMA
(ATTN_KAHEAD*) and, for head_dims above 128, workgroups per CU (ATTN_WG*:
the register budget of 256 or 512 per lane).  (64-row waves, ATTN_QB* = 2, are left out: one wave per
SIMD, 35-40 % slower where they fit, spilling where they do not.)  Only the
forward translation unit is rebuilt; the decode and backward objects of the
default build are linked unchanged (they keep the default tiles).

A variant is accepted only if its output matches the default build's on the
same inputs within max |dO| <= 1e-2 and |dLSE| <= 1e-3 (other tile sizes
reorder the sums, so bitwise equality is not expected); the default build is
the one the test suite holds to the oracle.  Results (JSON lines, one per
variant and case, then the best per case) go to stdout.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from .build import ARCH, CSRC, LIB_DIR, LIB_PATH, _hipcc, hip_flags

SWEEP_DIR = os.path.join(LIB_DIR, "sweep")  # beside the library, so that the variants reach the GPU host

# (head_dim, causal, B, H, N): the head_dim/causal combinations of the named
# workloads at sizes that time in milliseconds, and the LLaMA-7B layer shape
# (B=2, H=32, N=2048, non-causal) at the other head_dims.
CASES = [(64, True, 8, 16, 4096), (128, False, 2, 32, 2048), (128, True, 1, 32, 8192), (256, True, 1, 32, 8192),
         (32, False, 2, 32, 2048), (96, False, 2, 32, 2048), (160, False, 2, 32, 2048), (192, False, 2, 32, 2048),
         (224, False, 2, 32, 2048)]

VARIANTS = {
    32: [dict(BN=bn, KAHEAD=ka) for bn in (32, 64, 128) for ka in (2, 4)],
    64: [dict(BN=bn, KAHEAD=ka) for bn in (32, 64, 128) for ka in (2, 4, 6)],
    96: [dict(BN=bn, KAHEAD=ka) for bn in (32, 64, 128) for ka in (2, 4, 6)],
    128: [dict(BN=bn, KAHEAD=ka) for bn in (32, 64, 128) for ka in (2, 4, 6)],
    160: [dict(BN=bn, KAHEAD=ka, WG=wg) for bn in (32, 64) for ka in (4, 6, 8) for wg in (1, 2)],
    192: [dict(BN=bn, KAHEAD=ka, WG=wg) for bn in (32, 64) for ka in (4, 6, 8) for wg in (1, 2)],
    224: [dict(BN=bn, KAHEAD=ka, WG=wg) for bn in (32, 64) for ka in (4, 6, 8) for wg in (1, 2)],
    256: [dict(BN=bn, KAHEAD=ka, WG=wg) for bn in (32, 64) for ka in (4, 6, 8) for wg in (1, 2)],
}
# The default build's choices (csrc/attn_launch.h default_key_tile and
# default_wg_per_cu, csrc/attn_tile.h k_ahead).
DEFAULT = {d: dict(BN=64 if d <= 128 else 32, KAHEAD=4 if d <= 224 else 6) for d in VARIANTS}
for _d in (160, 192, 224, 256):
    DEFAULT[_d]["WG"] = 2   # d = 256: the default of the causal kernel (the swept case); non-causal d = 256 takes 1


def variant_name(d: int, v: dict) -> str:
    return f"d{d}_bn{v['BN']}_ka{v['KAHEAD']}" + (f"_wg{v['WG']}" if "WG" in v else "")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{res.stderr[-2000:]}")


def build_variants(jobs: int = 8, dims=None) -> list[str]:
    """Compile the default decode/backward/API objects once and one forward
    object per variant; link one library per variant into lib/sweep/."""
    os.makedirs(SWEEP_DIR, exist_ok=True)
    hipcc = _hipcc()
    common = []
    for src in ("attn_decode_kernel.hip", "attn_bwd_kernel.hip"):
        obj = os.path.join(SWEEP_DIR, src + ".o")
        _run([hipcc, *hip_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
        common.append(obj)
    api = os.path.join(SWEEP_DIR, "attn_api.cpp.o")
    _run([hipcc, "-x", "c++", "-O2", "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, "attn_api.cpp"), "-o", api])
    common.append(api)

    def one(item):
        d, v = item
        name = variant_name(d, v)
        obj = os.path.join(SWEEP_DIR, f"fwd_{name}.o")
        lib = os.path.join(SWEEP_DIR, f"lib_{name}.so")
        flags = [f"-DATTN_BN{d}={v['BN']}", f"-DATTN_KAHEAD{d}={v['KAHEAD']}"]
        if "WG" in v:
            flags.append(f"-DATTN_WG{d}={v['WG']}")
        try:
            _run([hipcc, *hip_flags(flags), "-c", os.path.join(CSRC, "attn_fwd_kernel.hip"), "-o", obj])
            _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, *common, "-o", lib])
            return name, "built"
        except RuntimeError as e:
            return name, f"build failed: {str(e).splitlines()[-1][:200]}"

    items = [(d, v) for d in VARIANTS if dims is None or d in dims for v in VARIANTS[d]]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        out = list(ex.map(one, items))
    for name, status in out:
        print(json.dumps({"variant": name, "status": status}), flush=True)
    return [n for n, st in out if st == "built"]


def _load(path):
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd.restype = ctypes.c_int
    return lib


# Timing: the GPU is first kept busy for WARMUP_S seconds (its clock ramps up
# over the first ~40 ms of load after idle, which would penalise whichever
# variant ran first), then the case's variants are timed round-robin,
# LAUNCHES launches per variant and round, the order reversed every other
# round; the median over the rounds is reported.
WARMUP_S = 0.3
LAUNCHES = 10


def run_sweep(repeats: int = 5, dims=None) -> None:
    import time

    import torch

    dev = torch.device("cuda:0")
    default = _load(LIB_PATH)
    best = {}
    for d, causal, B, H, N in CASES:
        if dims is not None and d not in dims:
            continue
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + d + N)
        q = torch.randn(B, H, N, d, device=dev, generator=g).half()
        k = torch.randn(B, H, N, d, device=dev, generator=g).half()
        v = torch.randn(B, H, N, d, device=dev, generator=g).half()
        scale = 1.0 / math.sqrt(d)
        stream = torch.cuda.current_stream(dev)
        flops = 4 * d * (N * (N + 1) // 2 if causal else N * N) * B * H
        case = f"d={d} causal={causal} B={B} H={H} N={N}"

        def call(lib, o, lse):
            st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H, N, d,
                              scale, int(causal), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"attn_fwd status {st}")

        o_ref, l_ref = torch.empty_like(q), torch.empty(B, H, N, device=dev)
        call(default, o_ref, l_ref)
        torch.cuda.synchronize()
        # Load and check every variant first.
        ready = []
        for vdef in VARIANTS[d]:
            name = variant_name(d, vdef)
            path = os.path.join(SWEEP_DIR, f"lib_{name}.so")
            rec = {"case": case, "variant": name}
            if not os.path.exists(path):
                rec["status"] = "not built"
                print(json.dumps(rec), flush=True)
                continue
            lib = _load(path)
            o, lse = torch.empty_like(q), torch.empty(B, H, N, device=dev)
            call(lib, o, lse)
            torch.cuda.synchronize()
            dmax = (o.float() - o_ref.float()).abs().max().item()
            lmax = (lse - l_ref).abs().max().item()
            rec.update(max_abs_diff_O=dmax, max_abs_diff_LSE=lmax)
            if not (dmax <= 1e-2 and lmax <= 1e-3):
                rec["status"] = "rejected: output differs from the default build"
                print(json.dumps(rec), flush=True)
                continue
            ready.append((vdef, name, lib, o, lse, rec))
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < WARMUP_S:
            for _ in range(5):
                call(default, o_ref, l_ref)
            torch.cuda.synchronize()
        times = {name: [] for _, name, *_ in ready}
        for r in range(repeats):
            for vdef, name, lib, o, lse, rec in (ready if r % 2 == 0 else ready[::-1]):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(LAUNCHES):
                    call(lib, o, lse)
                e1.record(stream)
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1) / LAUNCHES)
        for vdef, name, lib, o, lse, rec in ready:
            t = sorted(times[name])[len(times[name]) // 2]
            rec.update(status="ok", median_ms=round(t, 4), tflops=round(flops / (t * 1e-3) / 1e12, 1),
                       default=vdef == DEFAULT[d])
            print(json.dumps(rec), flush=True)
            if case not in best or rec["tflops"] > best[case]["tflops"]:
                best[case] = rec
    for case, rec in best.items():
        print(json.dumps({"best": case, "variant": rec["variant"], "tflops": rec["tflops"]}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("what", choices=("build", "run"))
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--dims", default="", help="comma-separated head_dims (default: all)")
    args = ap.parse_args()
    dims = {int(x) for x in args.dims.split(",")} if args.dims else None
    if args.what == "build":
        build_variants(args.jobs, dims)
    else:
        run_sweep(dims=dims)
    return 0


if __name__ == "__main__":
    sys.exit(main())
