"""bench.py's command line without a GPU: more than one GPU is refused with a
message (this build has no multi-GPU path), and the option sets the
benchmark offers parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_workload_and_variant_are_refused():
    assert run("--workload", "nope").returncode != 0
    assert run("--variant", "nope").returncode != 0


def test_help_lists_the_modes():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--variant", "--layer", "--autograd", "--nvfp4", "--mfma-ceiling",
                "--counters", "--copy-calibration"):
        assert opt in r.stdout
