"""Smoke test of bench.py on the GPU: a short decode run and a short prefill run, each in a child process, print one
JSON line with the fields the benchmark reports (the metric, the step time, the roofline object of the dominant
kernel with the kernel's own launch-event time)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


def test_decode_line():
    d = run_bench("--steps", "8", "--warmup", "2", "--no-cpu", "--no-extras", "--event-every", "2")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["value"] == pytest.approx(16 / (28 * d["ms_per_step"] * 1e-3), rel=1e-9)
    assert d["config"]["workload"] and d["config"]["global_batch"] == 16
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["event_samples"] == 4  # steps 1, 3, 5, 7
    # the kernel's own interval: shorter than the step, and the achieved rate below the peak
    assert 0 < rf["launch_us_events"] < d["ms_per_step"] * 1e3
    assert rf["achieved"] == pytest.approx(rf["bytes_per_launch"] / (rf["launch_us_events"] * 1e-6) / 1e9)
    assert 0 < rf["frac"] < 1 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])


def test_prefill_line():
    d = run_bench("--workload", "prefill", "--steps", "4", "--warmup", "2", "--no-cpu")
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s"
    assert 0 < rf["frac"] < 1 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert d["prefill"]["kernel_us_events"] < d["prefill"]["us_per_step"]
