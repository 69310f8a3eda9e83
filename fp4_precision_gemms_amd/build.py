"""Builds libfp4.so (the HIP kernels and the C ABI) in-tree for gfx950, and
beside it libfp4calib.so, the MFMA-rate measurement aid (include/fp4_calib.h).

    python -m fp4_precision_gemms_amd.build

Every source is compiled by hipcc for gfx950 only, with contraction of
a*b+c into FMAs disabled (the quantizers' rounding is specified operation by
operation) and packed-fp32 instructions disabled; objects go to _build/ and
the library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libfp4.so")
CALIB_LIB_PATH = os.path.join(HERE, "libfp4calib.so")

SOURCES = ["fp4_abi.cpp", "quant_mx.hip", "gemm_mx.hip", "nvfp4.hip"]
CALIB_SOURCES = ["calib_mfma.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp4.so)")


def compile_flags() -> list[str]:
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source and link libfp4.so and libfp4calib.so; returns
    the path of libfp4.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB_PATH)
    if verbose:
        print("built", LIB_PATH, "and", CALIB_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
