"""The C ABI's host code (fp4_precision_gemms_amd/csrc/fp4_abi.cpp) built
with g++ and AddressSanitizer + UBSan against stub launchers that record
their arguments (tests/helpers/abi_host_main.cpp): every entry point's
dispatch (operand roles, sizes, enums) and every documented refusal, with no
sanitizer report.  Host code only; no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("g++ or the HIP headers not available")
    exe = str(tmp_path / "abi_host")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "fp4_precision_gemms_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "helpers", "abi_host_main.cpp"),
           os.path.join(ROOT, "fp4_precision_gemms_amd", "csrc", "fp4_abi.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), (run.returncode, run.stdout[-2000:],
                                                                       run.stderr[-3000:])
