"""Offline tile sweep for the fused forward kernel.

The pages tie the block size to head_dim and the on-chip buffer ([CANN-FA]
section "Key design points") and leave the best block size per sequence
length to CANN's tuning engine ([FA-Infer] section 5, the item on AOE).
This is the same idea for this kernel, offline: rebuild the forward kernel
with other tile choices, hold each to the fp64 oracle, time the accepted ones
on the GPU at several sequence lengths, and report the best per (head_dim,
causal, sequence length) case.

    python -m exact_attention_121_amd.tile_sweep build            # compile the variants (no GPU needed)
    python tests/sweep_accept.py > gpurun_out/accepted.jsonl      # oracle check of every variant (GPU)
    python -m exact_attention_121_amd.tile_sweep run --accepted gpurun_out/accepted.jsonl   # time them
    (--dims 64,128 restricts any step to those head_dims)

Axes (compile-time hooks of csrc/attn_tile.h and csrc/attn_fwd_kernel.hip,
per head_dim):
  QB      32-row query blocks per wave (ATTN_QB*; 1 or 2: 128 or 256 query
          rows per workgroup of 4 waves), at head_dims 64, 128, 256;
  BN      keys per K/V tile (ATTN_BN*);
  WG      workgroups per CU the kernel is compiled for (ATTN_WG*: the
          register budget per lane);
  KAHEAD  matrix operands read from LDS ahead of their MFMA (ATTN_KAHEAD*);
  FORM    "pp": the 8-wave ping-pong kernel (two wave groups a phase apart,
          operands read into registers a phase ahead; head_dim 128,
          non-causal).
Each variant compiles only its head_dim and fp16 (ATTN_ONLY_D), so a variant
builds in seconds; it is linked with the default build's C-ABI object and
stand-ins for the decode and backward launchers (variants serve attn_fwd
only).

Acceptance is by the oracle, never by comparison with the default build:
tests/sweep_accept.py (test infrastructure, the only code that may call the
oracle) runs every built variant on validation problems of its head_dim
(ragged N, GQA, spiky logits, causal and not) against the fp64 oracle at the
parity bar, and `run` times only the variants it accepted.  Results (JSON
lines: one per variant and case, the best per case, and the choice per
(head_dim, causal) over the sequence lengths) go to stdout.
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

from .build import ARCH, BUILD_DIR, CSRC, LIB_DIR, LIB_PATH, _hipcc, hip_flags

SWEEP_DIR = os.path.join(LIB_DIR, "sweep")  # beside the library, so that the variants reach the GPU host


def _v(qb=1, bn=64, wg=2, ka=4, form=""):
    return dict(QB=qb, BN=bn, WG=wg, KAHEAD=ka, FORM=form)


VARIANTS = {
    32: [_v(1, bn, 2, ka) for bn in (32, 64) for ka in (2, 4)],
    64: [_v(qb, bn, wg, ka) for qb, bn, wg in ((1, 32, 2), (1, 64, 2), (1, 64, 3), (2, 32, 2), (2, 64, 1),
                                               (2, 32, 1)) for ka in (2, 4)],
    96: [_v(1, bn, 2, ka) for bn in (32, 64) for ka in (2, 4)],
    128: [_v(qb, bn, wg, ka) for qb, bn, wg in ((1, 32, 2), (1, 64, 2), (1, 64, 1), (2, 32, 1))
          for ka in (2, 4, 6)] + [_v(1, 32, 1, 4, "pp")],
    160: [_v(1, bn, wg, ka) for bn, wg in ((32, 1), (32, 2), (64, 2)) for ka in (4, 6)],
    192: [_v(1, bn, wg, ka) for bn, wg in ((32, 1), (32, 2), (64, 2)) for ka in (4, 6)],
    224: [_v(1, bn, wg, ka) for bn, wg in ((32, 1), (32, 2), (64, 2)) for ka in (4, 6)],
    256: [_v(1, bn, wg, ka) for bn, wg in ((32, 1), (32, 2), (64, 1)) for ka in (4, 6, 8)],
}
QB_HOOK_DIMS = (64, 128, 256)   # head_dims with an ATTN_QB* hook

# (head_dim, causal, N): every head_dim at the LLaMA-7B layer's N = 2048
# non-causal; the head_dims of the named workloads (64, 128, 256) causal and
# not at three or four sequence lengths.  H = Hkv = 32, B = max(1, 4096 / N)
# so that every case has at least ~1 000 workgroups.
CASES = ([(d, False, 2048) for d in (32, 96, 160, 192, 224)]
         + [(64, c, n) for c in (False, True) for n in (1024, 4096, 16384)]
         + [(128, c, n) for c in (False, True) for n in (1024, 2048, 8192)]
         + [(256, c, n) for c in (False, True) for n in (2048, 8192)])


def case_shape(d: int, causal: bool, N: int):
    return max(1, 4096 // N), 32, N


def variant_name(d: int, v: dict) -> str:
    name = f"d{d}_qb{v['QB']}_bn{v['BN']}_wg{v['WG']}_ka{v['KAHEAD']}"
    return name + (f"_{v['FORM']}" if v["FORM"] else "")


def variant_flags(d: int, v: dict) -> list[str]:
    flags = [f"-DATTN_ONLY_D={d}", "-DATTN_FP16_ONLY", f"-DATTN_BN{d}={v['BN']}", f"-DATTN_WG{d}={v['WG']}",
             f"-DATTN_KAHEAD{d}={v['KAHEAD']}"]
    if d in QB_HOOK_DIMS:
        flags.append(f"-DATTN_QB{d}={v['QB']}")
    elif v["QB"] != 1:
        raise ValueError(f"no query-block hook at head_dim {d}")
    if v["FORM"] == "pp":
        flags.append("-DATTN_FWD_PP=1")
    return flags


def variant_path(name: str) -> str:
    return os.path.join(SWEEP_DIR, f"lib_{name}.so")


def all_variants(dims=None):
    return [(d, v, variant_name(d, v)) for d in VARIANTS if dims is None or d in dims for v in VARIANTS[d]]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{res.stderr[-2000:]}")


# The variant libraries serve only attn_fwd: the decode and backward
# launchers are replaced by stand-ins that refuse the launch, so that a
# variant library holds one head_dim's forward kernels (~0.2 MB) instead of
# the whole library, and the head_dim 64 tile choice of the C-ABI front end
# is routed to the variant itself.
_STUBS = """#include "attn_launch.h"
namespace attn {
// the variant itself at every head_dim 64 shape (no second tile choice)
int launch_forward_d64_one_block(const LaunchArgs& a, void* s) { return launch_forward(a, s); }
int launch_decode(const DecodeArgs&, void*) { return 1; }
int launch_backward(const BwdArgs&, void*) { return 1; }
int launch_backward_noalloc(const BwdArgs&, void*) { return 1; }
}
"""


def build_variants(jobs: int = 8, dims=None) -> list[str]:
    """Compile one forward object per variant (its head_dim only) and link it
    with the default build's C-ABI object and stand-ins for the decode and
    backward launchers into lib/sweep/lib_<variant>.so."""
    os.makedirs(SWEEP_DIR, exist_ok=True)
    hipcc = _hipcc()
    api = os.path.join(BUILD_DIR, "attn_api.cpp.o")
    if not os.path.exists(api):
        raise RuntimeError("build the library first (python -m exact_attention_121_amd.build)")
    stub_src = os.path.join(SWEEP_DIR, "launch_stubs.cpp")
    with open(stub_src, "w") as f:
        f.write(_STUBS)
    stub = os.path.join(SWEEP_DIR, "launch_stubs.o")
    _run([hipcc, "-x", "c++", "-O2", "-std=c++17", "-fPIC", f"-I{CSRC}", "-c", stub_src, "-o", stub])
    common = [api, stub]

    def one(item):
        d, v, name = item
        obj = os.path.join(SWEEP_DIR, f"fwd_{name}.o")
        try:
            _run([hipcc, *hip_flags(variant_flags(d, v)), "-c", os.path.join(CSRC, "attn_fwd_kernel.hip"), "-o",
                  obj])
            _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, *common, "-o", variant_path(name)])
            os.remove(obj)
            return name, "built"
        except RuntimeError as e:
            return name, f"build failed: {str(e).splitlines()[-1][:200]}"

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        out = list(ex.map(one, all_variants(dims)))
    for name, status in out:
        print(json.dumps({"variant": name, "status": status}), flush=True)
    return [n for n, st in out if st == "built"]


def load_variant(path):
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd.restype = ctypes.c_int
    return lib


# Timing: the GPU is first kept busy for WARMUP_S seconds (its clock ramps up
# over the first ~40 ms of load after idle, which would penalise whichever
# variant ran first), then the case's variants and the default build are
# timed round-robin, LAUNCHES launches per variant and round, the order
# reversed every other round; the median over the rounds is reported.
WARMUP_S = 0.3
LAUNCHES = 10
# A variant replaces the default for a case only when it is faster by more
# than this (the spread of repeated timings of one build on one box).
MARGIN = 0.02


def run_sweep(accepted: set, repeats: int = 5, dims=None) -> None:
    import time

    import torch

    dev = torch.device("cuda:0")
    default = load_variant(LIB_PATH)
    per_case = {}
    for d, causal, N in CASES:
        if dims is not None and d not in dims:
            continue
        B, H, _ = case_shape(d, causal, N)
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

        runs = [("default", default, {"variant": "default"})]
        for dd, vdef, name in all_variants({d}):
            rec = {"case": case, "variant": name}
            if name not in accepted:
                rec["status"] = "not timed: not accepted by the oracle check"
                print(json.dumps(rec), flush=True)
                continue
            if vdef["FORM"] == "pp" and causal:
                continue  # the ping-pong form is built for the non-causal kernel only
            runs.append((name, load_variant(variant_path(name)), rec))
        bufs = {name: (torch.empty_like(q), torch.empty(B, H, N, device=dev)) for name, _, _ in runs}
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < WARMUP_S:
            for _ in range(5):
                call(default, *bufs["default"])
            torch.cuda.synchronize()
        times = {name: [] for name, _, _ in runs}
        for r in range(repeats):
            for name, lib, _ in (runs if r % 2 == 0 else runs[::-1]):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(LAUNCHES):
                    call(lib, *bufs[name])
                e1.record(stream)
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1) / LAUNCHES)
        res = {}
        for name, _, rec in runs:
            t = sorted(times[name])[len(times[name]) // 2]
            rec.update(case=case, status="ok", median_ms=round(t, 4), tflops=round(flops / (t * 1e-3) / 1e12, 1))
            print(json.dumps(rec), flush=True)
            res[name] = rec["tflops"]
        best = max(res, key=res.get)
        per_case[(d, causal, N)] = (best, res[best], res["default"])
        print(json.dumps({"best": case, "variant": best, "tflops": res[best], "default_tflops": res["default"],
                          "gain_over_default": round(res[best] / res["default"] - 1, 4)}), flush=True)
    # The choice per (head_dim, causal): a variant that beats the default by
    # more than MARGIN at some sequence lengths, or the default.
    for (d, causal) in sorted({(d, c) for d, c, _ in per_case}):
        rows = sorted((n, *per_case[(d, causal, n)]) for dd, c, n in per_case if (dd, c) == (d, causal))
        pick = {n: (b if tf > df * (1 + MARGIN) else "default") for n, b, tf, df in rows}
        print(json.dumps({"choice": f"d={d} causal={causal}", "per_N": pick}), flush=True)


def read_accepted(path: str) -> set:
    acc = set()
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                rec = json.loads(line)
                if rec.get("accepted"):
                    acc.add(rec["variant"])
    return acc


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("what", choices=("build", "run"))
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--dims", default="", help="comma-separated head_dims (default: all)")
    ap.add_argument("--accepted", default="", help="JSON lines of tests/sweep_accept.py (run: required)")
    args = ap.parse_args()
    dims = {int(x) for x in args.dims.split(",")} if args.dims else None
    if args.what == "build":
        build_variants(args.jobs, dims)
    else:
        if not args.accepted:
            print("run needs --accepted: variants are timed only after the oracle check "
                  "(tests/sweep_accept.py)", file=sys.stderr)
            return 2
        run_sweep(read_accepted(args.accepted), dims=dims)
    return 0


if __name__ == "__main__":
    sys.exit(main())
