"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the C
oracle and a driver that calls every entry point on small inputs with the
method's special cases (tests/helpers/oracle_sanitize_main.c) are built with
gcc -fsanitize=address,undefined (no OpenMP: one thread) and must run to the
end with no report.  Host code only; no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "helpers", "oracle_sanitize_main.c"),
       os.path.join(ROOT, "oracle", "fp4_oracle.c")]


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=gnu11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-Wno-unknown-pragmas", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           *SRC, "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitizer" in (build.stderr or "").lower():
        pytest.skip("gcc cannot link the sanitizers here: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.returncode, run.stdout[-500:],
                                                               run.stderr[-3000:])
