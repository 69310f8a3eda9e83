"""bench.py on the GPU, shortened: the one JSON line it prints holds the
fields the benchmark contract names, and its figures agree with each other
-- the value with the step time, the roofline object with the GEMM's window,
and the two kernel windows with the timed step they make up."""
import json
import os
import subprocess
import sys

import pytest

from _util import need_gpu, say

pytestmark = [pytest.mark.gpu]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
T, N, K = 8192, 14336, 4096          # the gate/up Wgrad the default run measures


def bench_line(*args):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_short_default_run_is_consistent():
    need_gpu()
    say("bench.py short run")
    b = bench_line("--steps", "10", "--warmup", "5", "--settle-ms", "50", "--no-cpu-baseline",
                   "--no-mfma-ceiling")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "breakdown", "settle",
                "timed_clock"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 10 and b["warmup"] == 5
    assert b["unit"] == "TFLOP/s" and b["higher_is_better"] is True
    flops = 2.0 * T * N * K
    assert b["value"] == pytest.approx(flops / (b["ms_per_step"] * 1e-3) / 1e12, rel=1e-9)
    rf, br = b["roofline"], b["breakdown"]
    assert rf["bound"] == "mfma" and rf["peak"] == 10100.0 and rf["unit"] == "TFLOP/s"
    assert rf["achieved"] == pytest.approx(flops / (br["gemm_ms"] * 1e-3) / 1e12, rel=1e-9)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-12)
    assert 0.0 < rf["frac"] < 1.0
    # the quantizer and GEMM windows make up the timed step (launch gaps and
    # in-step differences well under a tenth of it)
    assert br["quant_dY_X_ms"] > 0 and br["gemm_ms"] > 0
    assert abs(br["step_minus_kernels_ms"]) < 0.1 * b["ms_per_step"]
    assert br["gemm_ms"] < b["ms_per_step"] and br["quant_dY_X_ms"] < b["ms_per_step"]
    assert br["quantizer_frac_hbm"] == pytest.approx(br["quantizer_GBps"] / 8000.0, rel=1e-12)
    assert b["settle"]["steps"] > 0
