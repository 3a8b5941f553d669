"""The benchmark's JSON line on the GPU (bench.py run as a child process).

One short forward run with a bounded oracle sample (and a few cold-cache
steps), and one short decode run: the line has the fields its contract names,
a parity check that passed, a live shader clock in the range the part can run
at, and the device-derived peak.
"""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    print(f"[bench] {' '.join(args)}", file=sys.stderr, flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                         timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    return json.loads(res.stdout.strip().splitlines()[-1])


def _clock_ok(line):
    live = line["sclk"]["live"]
    assert live["mhz"] is not None, live
    assert 500.0 <= live["mhz"] <= 3000.0, live


def test_forward_line():
    line = _bench("--steps", "20", "--warmup", "5", "--cpu-budget", "1", "--no-gemm-reference", "--cold", "5")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "kernel_ms", "clock_warmup"):
        assert key in line, key
    assert line["steps"] == 20 and line["warmup"] == 5 and line["n_gpus"] == 1
    assert line["value"] > 0 and 0 < line["roofline"]["frac"] < 1
    assert line["parity"]["ok"], line["parity"]
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] >= 1
    _clock_ok(line)
    peak = line["roofline"]["peak_from_device"]
    assert peak["cus"] >= 1 and peak["tflops"] > 0, peak
    assert line["cold"]["steps"] == 5 and line["cold"]["median_ms"] > 0


def test_decode_line():
    line = _bench("--decode", "2", "--steps", "10", "--warmup", "2", "--cpu-budget", "1")
    assert line["unit"] == "GB/s" and line["value"] > 0
    assert line["parity"]["ok"], line["parity"]
    _clock_ok(line)
