#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

Every run first runs untimed steps for 0.3 s (the GPU clock ramps up over
the first ~40 ms of load; the line reports this as "clock_warmup"), then the
--warmup steps (default 10), then times --steps steps (default: about 0.25 s
of them); the JSON line reports the counts used and the kernel time per step
(mean, median, min from HIP events around every step).  The forward and
backward lines also carry "gemm_reference": the rate of a plain fp16 GEMM
(torch.matmul, i.e. hipBLASLt) measured right after the timed steps on the
same GPU, the practical matrix-core ceiling under the chip's power limit;
and "sclk": the shader clock measured live by a one-wave probe on a second
stream during a repeat of the timed steps ("live"), and the clock and
matrix-core busy fraction that rocprofv3 counters measured for the same kernel
code ("counters": the committed counter summary, keyed by a hash of the
kernel sources; null once the code has changed).

A step is one call of the whole hot path (one fused forward kernel) over one
batch of synthetic fp16 inputs already resident in device memory.  The default
workload is the LLaMA-7B layer shape (B=2, H=32, N=2048, d=128, non-causal),
the configuration the headline TFLOP/s metric is quoted on.  Prints ONE JSON
line with the throughput, the roofline of the kernel (timed with HIP events on
the launch stream), the CPU oracle timed on a bounded sample of the same
workload, and a parity check of the timed output against that sample.

    python bench.py --cold 50

also times 50 steps each after a 512 MiB write that evicts the inputs from the
256 MB last-level cache (a secondary "cold" object; the default is warm).

    python bench.py --backward [--workload 2]

times the backward pass instead: a step is one attn_bwd call (two kernels)
given the forward's O and LSE; FLOPs are 10 d per visible (query, key) pair
(the four gradient products and the recomputed scores).

    python bench.py --decode 1 [--steps K] [--warmup W]

times the decode (KV-cache) path instead: a step is one attn_decode call (the
per-chunk kernel and the merge kernel) on a named decode workload; the line
reports HBM GB/s against the 8 TB/s peak.  When one copy of the cache is
smaller than 1 GiB, the steps cycle over enough copies to exceed the chip's
256 MB last-level cache, so that every step reads HBM.

--head-dim D runs any of these on the chosen workload with head_dim D instead
of its own (same seeds and other sizes, scale 1/sqrt(D)).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of MI355X fp16 MFMA peak (N=2048, d=128)"
DECODE_METRIC = "attention decode HBM GB/s + % of MI355X HBM peak"
BACKWARD_METRIC = "attention bwd TFLOP/s + % of MI355X fp16 MFMA peak"
PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published figure
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published figure
FORWARD_SOURCES = ["exact_attention_121_amd/csrc/attn_tile.h", "exact_attention_121_amd/csrc/attn_fwd_kernel.hip",
                   "exact_attention_121_amd/csrc/attn_fwd_kernel_d64_one_block.hip"]
DECODE_SOURCES = ["exact_attention_121_amd/csrc/attn_tile.h", "exact_attention_121_amd/csrc/attn_decode_kernel.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_decode_traffic.json")
BACKWARD_SOURCES = ["exact_attention_121_amd/csrc/attn_tile.h", "exact_attention_121_amd/csrc/attn_bwd_kernel.hip"]
BACKWARD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bwd_traffic.json")


# Before the requested warm-up steps, steps run for CLOCK_WARMUP_S seconds
# (always, with the count reported as its own field): the MI355X clock ramps
# up over the first ~40 ms of load after idle (a forward step of the LLaMA-7B
# layer shape takes 266 us in its first 20 steps, 145 us after 20 ms and
# 138 us from ~60 ms on), so a few warm-up steps on an idle GPU would time
# the ramp, not the kernel.  Without --steps, the timed region is about
# TIMED_S seconds of steps (at least 5).
CLOCK_WARMUP_S = 0.3
TIMED_S = 0.25
DEFAULT_WARMUP = 10


def gemm_reference(dev, n: int = 8192, seconds: float = 0.5) -> dict:
    """TFLOP/s of a plain n x n x n fp16 GEMM (torch.matmul, which dispatches
    to hipBLASLt) on the same GPU: warmed up for `seconds`, then timed with
    HIP events.  A measured ceiling for dense fp16 matrix work on this chip
    at the clock its power limit allows, next to the published peak."""
    import torch

    a = torch.randn(n, n, device=dev, dtype=torch.float16)
    b = torch.randn(n, n, device=dev, dtype=torch.float16)
    c = torch.empty(n, n, device=dev, dtype=torch.float16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # The same again with the clock probe beside it (not timed).
    probe = ClockProbe(dev)
    torch.cuda.synchronize()
    probe.start(0.6 * ms * reps)
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"tflops": round(tflops, 1), "frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
            "shape": f"{n}x{n}x{n} fp16, fp32 accumulate", "library": "torch.matmul (hipBLASLt)",
            "ms": round(ms, 4), "sclk_live_mhz": probe.result()["mhz"]}


class ClockProbe:
    """Mean shader clock of one CU under the timed kernels' load: a one-wave
    kernel (exact_attention_121_amd/csrc/sclk_probe.hip, its own small
    library) on a second stream of default priority counts shader-clock
    cycles against the constant-rate wall counter over a window of the
    per-step-event pass, which repeats the timed steps (so the timed pass
    itself runs unperturbed)."""

    def __init__(self, dev):
        import ctypes

        import torch

        from exact_attention_121_amd.build import PROBE_PATH

        self.lib, self.error, self.khz = None, None, 0
        try:
            lib = ctypes.CDLL(PROBE_PATH)
            lib.attn_sclk_probe.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
            lib.attn_sclk_probe.restype = ctypes.c_int
            lib.attn_wall_clock_khz.restype = ctypes.c_int
            self.khz = lib.attn_wall_clock_khz()
            if self.khz <= 0:
                raise OSError("no wall clock rate")
            self.lib = lib
        except OSError as e:
            self.error = f"probe library not usable: {e}"
        self.out = torch.zeros(2, dtype=torch.int64, device=dev)
        self.stream = torch.cuda.Stream(device=dev)
        self.window_ms = 0.0

    def start(self, window_ms: float):
        """Queue the probe (call before queuing the kernels it should see)."""
        if self.lib is None:
            return
        self.window_ms = max(0.2, min(window_ms, 2000.0))
        if self.lib.attn_sclk_probe(self.out.data_ptr(), int(self.khz * self.window_ms), self.stream.cuda_stream):
            self.error, self.lib = "probe launch failed", None

    def result(self) -> dict:
        """Call after a device synchronisation."""
        rec = {"source": "shader-clock cycles / wall-clock ticks of a one-wave probe on a second stream during the "
                         "per-step-event pass (one CU)"}
        if self.lib is None:
            rec.update(mhz=None, error=self.error)
            return rec
        cycles, ticks = (int(x) for x in self.out.tolist())
        rec.update(mhz=round(cycles / (ticks / (self.khz * 1e3)) / 1e6, 1) if ticks > 0 else None,
                   window_ms=round(ticks / self.khz, 3))
        return rec


def device_peak() -> dict:
    """The dense fp16 matrix peak from the device's own figures: compute units
    x maximum shader clock x 4 096 FLOP per CU per clock (4 SIMDs, one
    32x32x16 fp16 MFMA of 32 768 FLOP per 32 clocks each)."""
    import ctypes

    from exact_attention_121_amd.build import PROBE_PATH

    try:
        lib = ctypes.CDLL(PROBE_PATH)
        cus, khz = ctypes.c_int(0), ctypes.c_int(0)
        if lib.attn_device_info(ctypes.byref(cus), ctypes.byref(khz)) != 0:
            raise OSError("attn_device_info failed")
    except (OSError, AttributeError) as e:
        return {"tflops": None, "error": str(e)}
    return {"cus": cus.value, "max_mhz": khz.value / 1e3,
            "tflops": round(cus.value * khz.value * 1e3 * 4096 / 1e12, 1),
            "source": "hipDeviceAttributeMultiprocessorCount x hipDeviceAttributeClockRate x 4096 FLOP/CU/clk"}


def cold_steps(step, dev, steps: int, flush_mib: int = 512) -> dict:
    """Kernel time of `steps` forward steps, each after writing a flush_mib
    buffer (larger than the 256 MB last-level cache), so that the step reads
    its inputs from HBM; HIP events around each step only."""
    import torch

    buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    times = []
    for i in range(steps):
        buf.fill_(i & 255)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del buf
    times.sort()
    return {"steps": steps, "median_ms": round(times[len(times) // 2], 5), "min_ms": round(times[0], 5),
            "flush_bytes": flush_mib << 20}


def counter_clock(workload_name: str, path=TRAFFIC_FILE, sources=FORWARD_SOURCES):
    """Shader clock and matrix-core busy fraction of the dominant kernel from
    the committed rocprofv3 counter record (GRBM_GUI_ACTIVE over the kernel's
    duration; SQ_VALU_MFMA_BUSY_CYCLES over cycles x 1024 SIMDs), or None
    when there is none for this workload or the kernel changed since."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload_name)
    if not entry or entry.get("kernel_code_sha256_16") != kernel_source_hash(sources) or "clock_mhz" not in entry:
        return None
    return {"mhz": entry["clock_mhz"], "mfma_busy": entry.get("mfma_busy"),
            "source": "rocprofv3 counters of the same kernel code (" + entry.get("mfma_summary", "") + ")"}


def run_timed(step, args, dev):
    """Runs the clock warm-up, the requested warm-up steps and the timed
    steps of `step(i)`; sets args.warmup and args.steps to the counts used.
    Returns (wall ms per step, kernel-time stats, clock-warm-up record, live
    shader-clock record).  The timed steps are bracketed by one pair of HIP events on the
    launch stream (their mean is the region's time over the steps; it agrees
    with a rocprofv3 kernel trace of the same dispatches).  Median, min and
    max come from a second pass of as many steps right after it with events
    around every step: each such interval also holds the few microseconds the
    event markers add between dispatches, so they are slightly above the
    kernel time."""
    import torch

    n, t_start = 0, time.perf_counter()
    while True:
        t_batch = time.perf_counter()
        for _ in range(10):
            step(n)
            n += 1
        torch.cuda.synchronize()
        now = time.perf_counter()
        per_step = (now - t_batch) / 10
        if now - t_start >= CLOCK_WARMUP_S:
            break
    ramp = {"seconds": CLOCK_WARMUP_S, "steps": n,
            "why": "untimed steps before the warm-up count, so that the timed steps do not see the clock ramp "
                   "of an idle GPU"}
    if args.warmup is None:
        args.warmup = DEFAULT_WARMUP
    for i in range(args.warmup):
        step(n + i)
    n += args.warmup
    torch.cuda.synchronize()
    if args.steps is None:
        args.steps = max(5, min(5000, int(round(TIMED_S / per_step))))
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(n + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n += args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    probe = ClockProbe(dev)
    torch.cuda.synchronize()
    probe.start(0.6 * (t1 - t0) * 1e3)
    for i in range(args.steps):
        evs[i].record(stream)
        step(n + i)
    evs[-1].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    stats = {"mean": ev0.elapsed_time(ev1) / args.steps, "median": per[len(per) // 2], "min": per[0],
             "max": per[-1], "mean_per_step_events": sum(per) / len(per)}
    return (t1 - t0) * 1e3 / args.steps, stats, ramp, probe.result()


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def kernel_ms_record(stats, steps: int, kernels: str) -> dict:
    return {"mean": round(stats["mean"], 5), "median": round(stats["median"], 5), "min": round(stats["min"], 5),
            "max": round(stats["max"], 5), "mean_with_per_step_events": round(stats["mean_per_step_events"], 5),
            "timing": f"mean: one pair of HIP events on the launch stream around the {steps} timed steps "
                      f"({kernels}); median/min/max: a second pass of {steps} steps right after, with HIP events "
                      "around every step (each interval also holds the gap the event markers add between "
                      "dispatches; its mean is mean_with_per_step_events)"}


def kernel_source_hash(sources=FORWARD_SOURCES) -> str:
    """Hash of the kernel sources with comments and blank lines removed, so
    that only a change of the code itself invalidates the stored counters."""
    import re

    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, path=TRAFFIC_FILE, sources=FORWARD_SOURCES,
                     key="hbm_bytes_per_launch"):
    """HBM bytes per launch (per step for decode) from the committed rocprofv3
    counter summary, or None when there is none for this workload or the
    kernel changed since."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload_name)
    if not entry or entry.get("kernel_code_sha256_16") != kernel_source_hash(sources):
        return None
    return entry.get(key)


def with_head_dim(w, d: int):
    """The workload w with head_dim d instead of its own (0: unchanged), named
    `<name>_d<d>`; the same seeds and every other size."""
    if not d or d == w.d:
        return w
    import dataclasses
    return dataclasses.replace(w, d=d, name=f"{w.name}_d{d}")


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, q, k, v, o_gpu, lse_gpu, budget_s: float, bf16: bool = False):
    """Time the fp64 oracle on whole heads of the workload (on the workload's
    seeded sample of query rows per head where it names one, the long-context
    workload's 256) until ~budget_s of CPU work is done; also check the GPU
    output of those rows against it."""
    import numpy as np

    from exact_attention_121_amd.inputs import sample_rows
    from oracle.attention import attention_ref

    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    rows = sample_rows(w) if w.sample_rows else None
    done, elapsed, pairs = 0, 0.0, 0
    max_err = mean_acc = lse_err = 0.0
    G = w.Hq // w.Hkv
    for b, h in heads:
        g = h // G
        qs, ks, vs = q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1]
        r = None if rows is None else rows[b, h]
        t0 = time.perf_counter()
        O_ref, L_ref = attention_ref(qs, ks, vs, w.scale, causal=w.causal, rows=r)
        elapsed += time.perf_counter() - t0
        og = o_gpu[b, h] if r is None else o_gpu[b, h][r]
        lg = lse_gpu[b, h] if r is None else lse_gpu[b, h][r]
        err = np.abs(og.astype(np.float64) - O_ref[0, 0])
        max_err = max(max_err, float(err.max()))
        mean_acc += float(err.mean())
        lse_err = max(lse_err, float(np.abs(lg - L_ref[0, 0]).max()))
        if r is None:
            pairs += w.pairs // len(heads)
        else:
            pairs += int(np.sum(r + 1)) if w.causal else len(r) * w.N
        done += 1
        if elapsed >= budget_s:
            break
    value = pairs * 4 * w.d / elapsed / 1e12
    what = (f"all {w.N} query rows each" if rows is None
            else f"the seeded sample of {rows.shape[2]} query rows each (rows 0 and N-1 and {rows.shape[2] - 2} "
                 "drawn without replacement)")
    base = {
        "value": value,
        "unit": "TFLOP/s",
        "cores": cpu_threads(),
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (batch, head) pairs, {what}, {elapsed:.1f} s of fp64 numpy two-pass "
                  "attention; TFLOP/s counts 4 d FLOPs per visible (query, key) pair of those rows",
    }
    bar = (4e-2, 4e-3, 4e-3) if bf16 else (1e-2, 1e-3, 1e-3)
    parity = {"heads_checked": done, "rows_per_head": "all" if rows is None else int(rows.shape[2]),
              "max_abs_err_O": max_err, "mean_abs_err_O": mean_acc / done,
              "max_abs_err_LSE": lse_err, "bar": bar,
              "ok": bool(max_err <= bar[0] and mean_acc / done <= bar[1] and lse_err <= bar[2])}
    return base, parity


def calibration_copy(mib: int, dev):
    """A plain elementwise copy of known traffic (y = -x in fp16, three
    launches), against which hardware byte counters are scaled."""
    import torch

    n = mib * (1 << 20) // 2
    x = torch.ones(n, dtype=torch.float16, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y
    return {"kernel": "torch.neg fp16 (elementwise)", "bytes_read": 2 * n, "bytes_written": 2 * n,
            "launches": 3}


def cpu_baseline_decode(w, q, k, v, o_gpu, lse_gpu, budget_s: float):
    """Time the fp64 decode oracle one batch entry at a time until ~budget_s
    of CPU work is done; check the GPU output of those entries against it."""
    import numpy as np

    from oracle.attention import attention_decode_ref

    done, elapsed = 0, 0.0
    max_err = mean_acc = lse_err = 0.0
    for b in range(w.B):
        t0 = time.perf_counter()
        O_ref, L_ref = attention_decode_ref(q[b:b + 1], k[b:b + 1], v[b:b + 1], w.scale, causal=w.causal)
        elapsed += time.perf_counter() - t0
        err = np.abs(o_gpu[b].astype(np.float64) - O_ref[0])
        max_err = max(max_err, float(err.max()))
        mean_acc += float(err.mean())
        lse_err = max(lse_err, float(np.abs(lse_gpu[b] - L_ref[0]).max()))
        done += 1
        if elapsed >= budget_s:
            break
    value = done * (w.hbm_bytes / w.B) / elapsed / 1e9
    base = {
        "value": value,
        "unit": "GB/s",
        "cores": cpu_threads(),
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": f"{done} of {w.B} batch entries (all {w.Hq} query heads, all {w.Nk} keys each), "
                  f"{elapsed:.1f} s of fp64 numpy two-pass attention; GB/s counts the same "
                  "algorithmic bytes as the GPU figure",
    }
    parity = {"batch_entries_checked": done, "max_abs_err_O": max_err, "mean_abs_err_O": mean_acc / done,
              "max_abs_err_LSE": lse_err,
              "ok": bool(max_err <= 1e-2 and mean_acc / done <= 1e-3 and lse_err <= 1e-3)}
    return base, parity


def run_decode(args) -> int:
    import torch

    import exact_attention_121_amd as ea
    from exact_attention_121_amd.inputs import DECODE_WORKLOADS, make_decode_inputs

    w = with_head_dim(DECODE_WORKLOADS[args.decode], args.head_dim)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ea.load_library()
    q_np, k_np, v_np = make_decode_inputs(w)
    kv_bytes = 2 * k_np.nbytes
    copies = max(1, -(-(1 << 30) // kv_bytes))
    q = torch.from_numpy(q_np).to(dev)
    k0, v0 = torch.from_numpy(k_np).to(dev), torch.from_numpy(v_np).to(dev)
    kvs = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, ea.attn_decode_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)),
                     dtype=torch.uint8, device=dev)

    def step(i):
        kc, vc = kvs[i % copies]
        ea.attn_decode(q, kc, vc, scale=w.scale, causal=w.causal, out=o, lse=lse, workspace=ws)

    ms_per_step, stats, ramp, live_clock = run_timed(step, args, dev)
    avg_step_ms = stats["mean"]
    value = w.hbm_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = w.hbm_bytes / (avg_step_ms * 1e-3) / 1e9
    result = {
        "metric": DECODE_METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: seeded N(0,sigma^2) fp16 Q and K/V cache at the workload's shape (no model weights)",
        "config": {"workload": f"{w.name}: {w.describe()}", "global_batch": w.B, "new_queries": w.Nq,
                   "cached_keys": w.Nk, "heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "causal": w.causal, "cache_copies_cycled": copies, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(w.name, DECODE_TRAFFIC_FILE, DECODE_SOURCES, "hbm_bytes_per_step"),
                     "bytes_per_step": w.hbm_bytes,
                     "scope": "whole step: per-chunk kernel plus merge kernel"},
        "kernel_ms": kernel_ms_record(stats, args.steps, "one or two kernels per step"),
        "clock_warmup": ramp,
        "sclk": {"live": live_clock, "counters": counter_clock(w.name, DECODE_TRAFFIC_FILE, DECODE_SOURCES)},
        "kernel_code_sha256_16": kernel_source_hash(DECODE_SOURCES),
    }
    if args.calibrate_copy_mib > 0:
        result["copy_calibration"] = calibration_copy(args.calibrate_copy_mib, dev)
    if not args.no_cpu_baseline:
        step(0)  # the output of the first cache copy, which the oracle sees
        torch.cuda.synchronize()
        base, parity = cpu_baseline_decode(w, q_np, k_np, v_np, o.cpu().numpy(), lse.cpu().numpy(),
                                           args.cpu_budget)
        result["cpu_baseline"] = base
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_backward(w, q, k, v, do, grads, budget_s: float, bf16: bool = False):
    """Time the fp64 backward oracle on whole (batch, query head) pairs (for
    GQA, the group's key/value head gets that query head's share) until about
    budget_s of CPU work is done; check dQ of those heads against it and dK,
    dV where the group has one query head."""
    import numpy as np

    from oracle.backward import attention_bwd_ref

    G = w.Hq // w.Hkv
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    done, elapsed = 0, 0.0
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    ok = True
    for b, h in heads:
        g = h // G
        sl_q = (slice(b, b + 1), slice(h, h + 1))
        sl_k = (slice(b, b + 1), slice(g, g + 1))
        t0 = time.perf_counter()
        ref = attention_bwd_ref(q[sl_q], k[sl_k], v[sl_k], do[sl_q], w.scale, causal=w.causal)
        elapsed += time.perf_counter() - t0
        checks = [("dQ", grads[0][sl_q], ref[0])]
        if G == 1:
            checks += [("dK", grads[1][sl_k], ref[1]), ("dV", grads[2][sl_k], ref[2])]
        for name, x, r in checks:
            err = np.abs(x.astype(np.float64) - r)
            worst[name] = max(worst[name], float(err.max() / np.abs(r).max()))
            bar = (4e-2, 8e-3) if bf16 else (1e-2, 2e-3)
            ok &= bool(err.max() <= bar[0] * np.abs(r).max() and err.mean() <= bar[1] * np.abs(r).mean())
        done += 1
        if elapsed >= budget_s:
            break
    per_head = 10 * w.d * (w.pairs // w.B // w.Hq)
    base = {
        "value": done * per_head / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": cpu_threads(),
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (batch, head) pairs, all {w.N} rows each, {elapsed:.1f} s of fp64 "
                  "numpy chain-rule backward",
    }
    parity = {"heads_checked": done, "max_rel_err": worst, "ok": ok}
    return base, parity


def run_backward(args) -> int:
    import numpy as np
    import torch

    import exact_attention_121_amd as ea
    from exact_attention_121_amd.inputs import WORKLOADS, make_inputs

    w = with_head_dim(WORKLOADS[args.workload], args.head_dim)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ea.load_library()
    bf16 = args.dtype == "bf16"
    if bf16:
        from exact_attention_121_amd.inputs import make_qkv_bf16, round_to_bf16
        q_np, k_np, v_np = make_qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, w.sigma, w.spike_frac, w.spike_mult)
        do_np = round_to_bf16(np.random.default_rng(w.seed + 7).standard_normal(q_np.shape, dtype=np.float32))
        q, k, v, do = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q_np, k_np, v_np, do_np))
    else:
        q_np, k_np, v_np = make_inputs(w)
        do_np = np.random.default_rng(w.seed + 7).standard_normal(q_np.shape, dtype=np.float32).astype(np.float16)
        q, k, v, do = (torch.from_numpy(x).to(dev) for x in (q_np, k_np, v_np, do_np))
    o, lse = ea.attn_fwd(q, k, v, scale=w.scale, causal=w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, ea.attn_bwd_workspace_size(w.B, w.Hq, w.N, w.d)), dtype=torch.uint8, device=dev)

    def step(_i):
        ea.attn_bwd(q, k, v, o, lse, do, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=ws)

    ms_per_step, stats, ramp, live_clock = run_timed(step, args, dev)
    avg_step_ms = stats["mean"]
    flops = 10 * w.d * w.pairs
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_step_ms * 1e-3) / 1e12
    result = {
        "metric": BACKWARD_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": f"synthetic: seeded N(0,1) {'bf16' if bf16 else 'fp16'} Q/K/V and upstream gradient dO at the "
                "workload's shape",
        "config": {"workload": f"{w.name} backward{' bf16' if bf16 else ''}: {w.describe()}", "global_batch": w.B, "seq_len": w.N,
                   "heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "causal": w.causal,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": None if bf16 else measured_traffic(w.name, BACKWARD_TRAFFIC_FILE, BACKWARD_SOURCES,
                                                                   "hbm_bytes_per_step"),
                     "flops_per_step": flops,
                     "scope": "whole step: dQ (with the row terms) and dK/dV kernels; 10 d FLOPs per visible pair"},
        "kernel_ms": kernel_ms_record(stats, args.steps, "two kernels per step"),
        "clock_warmup": ramp,
        "sclk": {"live": live_clock,
                 "counters": None if bf16 else counter_clock(w.name, BACKWARD_TRAFFIC_FILE, BACKWARD_SOURCES)},
        "kernel_code_sha256_16": kernel_source_hash(BACKWARD_SOURCES),
    }
    if not args.no_gemm_reference:
        g = gemm_reference(dev)
        g["attention_over_gemm"] = round(value / g["tflops"], 4)
        result["gemm_reference"] = g
    if args.calibrate_copy_mib > 0:
        result["copy_calibration"] = calibration_copy(args.calibrate_copy_mib, dev)
    if not args.no_cpu_baseline:
        grads = [x.float().cpu().numpy() for x in (dq, dk, dv)]
        base, parity = cpu_baseline_backward(w, q_np, k_np, v_np, do_np, grads, args.cpu_budget, bf16=bf16)
        result["cpu_baseline"] = base
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: about %.2f s of them)" % TIMED_S)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps after the %.1f s clock warm-up (default %d)"
                         % (CLOCK_WARMUP_S, DEFAULT_WARMUP))
    ap.add_argument("--workload", type=int, default=2, help="named workload id (1-5)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", type=int, default=0,
                    help="time the decode path on this named decode workload (1-4) instead")
    ap.add_argument("--dtype", choices=("f16", "bf16"), default="f16",
                    help="element type of Q, K, V, O for the forward (bf16 inputs are the same draws rounded to "
                         "bfloat16)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dQ, dK, dV) on --workload instead")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="run the chosen workload with this head_dim instead of its own (a multiple of 32 "
                         "from 32 to 256; scale 1/sqrt(head_dim))")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain elementwise copy of this many MiB (fp16 -> fp16, "
                         "y = -x) three times, so that hardware byte counters can be "
                         "calibrated against a kernel of known traffic")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the fp16 GEMM reference measured after the timed steps")
    ap.add_argument("--cold", type=int, default=0,
                    help="forward: also time this many steps each after a 512 MiB write that evicts the inputs "
                         "from the last-level cache (reported as a secondary 'cold' object)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards over heads with no communication, but no multi-GPU run "
              "is part of it", file=sys.stderr)
        return 2
    if args.decode:
        return run_decode(args)
    if args.backward:
        return run_backward(args)

    import numpy as np
    import torch

    import exact_attention_121_amd as ea
    from exact_attention_121_amd.inputs import WORKLOADS, make_inputs

    w = with_head_dim(WORKLOADS[args.workload], args.head_dim)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ea.load_library()
    if args.dtype == "bf16":
        from exact_attention_121_amd.inputs import make_qkv_bf16
        q_np, k_np, v_np = make_qkv_bf16(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, w.sigma, w.spike_frac, w.spike_mult)
        q, k, v = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q_np, k_np, v_np))
    else:
        q_np, k_np, v_np = make_inputs(w)
        q, k, v = (torch.from_numpy(x).to(dev) for x in (q_np, k_np, v_np))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)

    def step(_i):
        ea.attn_fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)

    ms_per_step, stats, ramp, live_clock = run_timed(step, args, dev)
    avg_kernel_ms = stats["mean"]

    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (avg_kernel_ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name)
    result = {
        "metric": METRIC if (w.N, w.d) == (2048, 128) else METRIC.replace("(N=2048, d=128)", f"(N={w.N}, d={w.d})"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": f"synthetic: seeded N(0,1) {'bf16' if args.dtype == 'bf16' else 'fp16'} Q/K/V at the workload's "
                "shape (no model weights)",
        "config": {"workload": f"{w.name}{' bf16' if args.dtype == 'bf16' else ''}: {w.describe()}",
                   "global_batch": w.B, "seq_len": w.N,
                   "heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "causal": w.causal,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                     "traffic": traffic if args.dtype == "f16" else None},
        "kernel_ms": kernel_ms_record(stats, args.steps, "one kernel per step"),
        "clock_warmup": ramp,
        "sclk": {"live": live_clock, "counters": counter_clock(w.name) if args.dtype == "f16" else None},
        "kernel_code_sha256_16": kernel_source_hash(),
    }
    result["roofline"]["peak_from_device"] = device_peak()
    if args.cold > 0:
        cold = cold_steps(step, dev, args.cold)
        cold["tflops_median"] = round(w.flops / (cold["median_ms"] * 1e-3) / 1e12, 2)
        result["cold"] = cold
    if not args.no_gemm_reference:
        g = gemm_reference(dev)
        g["attention_over_gemm"] = round(value / g["tflops"], 4)
        result["gemm_reference"] = g
    if args.calibrate_copy_mib > 0:
        result["copy_calibration"] = calibration_copy(args.calibrate_copy_mib, dev)
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(w, q_np, k_np, v_np, o.float().cpu().numpy(), lse.cpu().numpy(),
                                    args.cpu_budget, bf16=args.dtype == "bf16")
        result["cpu_baseline"] = base
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
