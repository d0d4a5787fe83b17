"""The bench line's contract, checked on a short run of bench.py in a child process.

One JSON line per run with the metric, value (tokens/s), ms_per_step, steps and
warm-up as asked, the roofline object (bound, achieved, peak, unit, frac,
traffic) and the CPU baseline; bf16 inputs are HBM-bound, fp32 inputs report the
fp32 matrix-core roof.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def run_bench(*args):
    print("case bench.py %s" % " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + list(args), cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_common(j, steps, warmup):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == steps and j["warmup"] == warmup
    assert j["higher_is_better"] is True and j["vs_baseline"] is None and j["unit"] == "tokens/s"
    assert j["value"] > 0 and j["ms_per_step"] > 0
    assert "workload" in j["config"]
    r = j["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    # the kernel time the roofline uses is the timed region's mean per call
    assert abs(r["kernel_ms"] - j["ms_per_step"]) < 1e-9


def test_headline_bench_line():
    j = run_bench("--steps", "5", "--warmup", "2")
    check_common(j, 5, 2)
    B, T = j["config"]["global_batch"], j["config"]["seq_len"]
    assert (B, T) == (8, 4096) and j["dtype"] == "bf16"
    assert abs(j["value"] - B * T / (j["ms_per_step"] / 1e3)) / j["value"] < 1e-9
    r = j["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    # traffic comes from the committed counter record while it matches the kernel
    # sources (null otherwise); measured traffic is the algorithmic bytes, no re-reads
    if r["traffic"] is not None:
        assert 0.99 < r["traffic"] / r["algorithmic_bytes"] < 1.05
    c = j["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0
    assert j["gate"]["replays_bitwise_equal"] is True


def test_float32_bench_line_reports_the_fp32_matrix_roof():
    j = run_bench("--workload", "train_f32", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    check_common(j, 3, 1)
    r = j["roofline"]
    assert j["dtype"] == "f32" and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["peak"] == 157.3 and r["hbm"]["unit"] == "GB/s"
