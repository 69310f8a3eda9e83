"""CPU oracle for the block-quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product library never imports it, and it never
imports the product library: the two share no code.

The arithmetic lives in ``fp4_oracle.c`` (plain C99, built with gcc, no HIP);
this module builds it, loads it with ctypes and moves numpy arrays in and out.
Every function states the definition it computes; the C source cites the pages
step by step.

Enumerations are the oracle's own:
    axis:     AXIS_COLS (blocks along the contiguous dim), AXIS_ROWS (along rows)
    had:      HAD_NONE, HAD_DET (plain Hadamard), HAD_SIGNED (Hadamard after
              seeded random sign flips)
    rounding: RND_RTN (nearest, ties to even), RND_SR (stochastic)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

AXIS_COLS, AXIS_ROWS = 0, 1
HAD_NONE, HAD_DET, HAD_SIGNED = 0, 1, 2
RND_RTN, RND_SR = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_FLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
             "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile fp4_oracle.c into liboracle.so next to it (gcc, no HIP)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _P(dt):
    return np.ctypeslib.ndpointer(dtype=dt, flags="C_CONTIGUOUS")


def lib():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    L = ctypes.CDLL(_LIB_PATH)
    i64, u64, i32, u32, u8 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint8
    f32, f64 = ctypes.c_float, ctypes.c_double
    sig = {
        "oracle_bf16_to_f32": (f32, [ctypes.c_uint16]),
        "oracle_e2m1_decode": (f64, [u8]),
        "oracle_e2m1_rtn": (u8, [f32]),
        "oracle_e2m1_sr": (u8, [f32, u32]),
        "oracle_e4m3_decode": (f64, [u8]),
        "oracle_e4m3_rne": (u8, [f32]),
        "oracle_e4m3_sr": (u8, [f32, u32]),
        "oracle_philox4x32_10": (None, [_P(np.uint32), _P(np.uint32), _P(np.uint32)]),
        "oracle_stream_word": (u32, [u64, u32, u64]),
        "oracle_hadamard_signs": (None, [i32, i32, u64, _P(np.float32)]),
        "oracle_hadamard_norm": (f32, [i32]),
        "oracle_fwht": (None, [_P(np.float32), i32, _P(np.float32)]),
        "oracle_mx_exponent": (i32, [f32]),
        "oracle_quant_mx": (i32, [_P(np.uint16), i64, i64, i32, i32, i32, u64, i32, u64,
                                  i64, i64, _P(np.uint8), _P(np.uint8)]),
        "oracle_mx_value": (f64, [_P(np.uint8), _P(np.uint8), i64, i64, i64]),
        "oracle_dequant_mx": (None, [_P(np.uint8), _P(np.uint8), i64, i64, i64, _P(np.float64)]),
        "oracle_gemm_mx_entries": (None, [_P(np.uint8), _P(np.uint8), _P(np.uint8), _P(np.uint8),
                                          i64, _P(np.int64), _P(np.int64), i64,
                                          _P(np.float64), _P(np.float64)]),
        "oracle_gemm_mx_rows": (None, [_P(np.uint8), _P(np.uint8), _P(np.uint8), _P(np.uint8),
                                       i64, i64, i64, i64, i64, _P(np.float64), _P(np.float64)]),
        "oracle_nvfp4_amax": (f32, [_P(np.uint16), i64, i64, i32, u64]),
        "oracle_nvfp4_quantize": (i32, [_P(np.uint16), i64, i64, i32, u64, i32, u64,
                                        ctypes.c_void_p, _P(np.uint8), _P(np.uint8),
                                        ctypes.POINTER(f32)]),
        "oracle_num_threads": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _bits16(x) -> np.ndarray:
    """bf16 input as a C-contiguous uint16 array of its bit patterns."""
    a = np.asarray(x)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16), got %s" % a.dtype)
    return np.ascontiguousarray(a)


# --- scalar formats ----------------------------------------------------------

def e2m1_rtn(v: float) -> int:
    return lib().oracle_e2m1_rtn(float(v))


def e2m1_sr(v: float, u: int) -> int:
    return lib().oracle_e2m1_sr(float(v), int(u))


def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(int(code))


def e4m3_rne(x: float) -> int:
    return lib().oracle_e4m3_rne(float(x))


def e4m3_sr(x: float, u: int) -> int:
    return lib().oracle_e4m3_sr(float(x), int(u))


def e4m3_decode(b: int) -> float:
    return lib().oracle_e4m3_decode(int(b))


def mx_exponent(m: float) -> int:
    """Shared exponent e of a block whose largest magnitude is m."""
    return lib().oracle_mx_exponent(float(m))


# --- random streams ----------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(c, k, out)
    return out


def stream_word(seed: int, purpose: int, index: int) -> int:
    return lib().oracle_stream_word(seed, purpose, index)


# --- Hadamard ----------------------------------------------------------------

def hadamard_signs(had: int, n: int, seed: int) -> np.ndarray:
    s = np.zeros(n, dtype=np.float32)
    lib().oracle_hadamard_signs(had, n, seed, s)
    return s


def hadamard_norm(n: int) -> np.float32:
    return np.float32(lib().oracle_hadamard_norm(n))


def fwht(block, signs=None) -> np.ndarray:
    """Normalized FWHT of one block (n = 16 or 32) in binary32."""
    a = np.array(block, dtype=np.float32)
    n = a.shape[0]
    s = np.ones(n, dtype=np.float32) if signs is None else np.ascontiguousarray(signs, np.float32)
    lib().oracle_fwht(a, n, s)
    return a


# --- MXFP4 -------------------------------------------------------------------

def mx_shape(rows: int, cols: int, axis: int):
    """(R, C) of the logical matrix whose rows are quantized along C."""
    return (rows, cols) if axis == AXIS_COLS else (cols, rows)


def quant_mx(x, axis=AXIS_COLS, had_n=32, had=HAD_NONE, sign_seed=0, rnd=RND_RTN,
             sr_seed=0, r0=0, r1=None):
    """MXFP4 codes [R, C/2] and E8M0 scales [R, C/32] of bf16 x[rows, cols].

    With r0/r1 only logical rows r0..r1-1 are computed and returned."""
    x = _bits16(x)
    rows, cols = x.shape
    R, C = mx_shape(rows, cols, axis)
    r1 = R if r1 is None else r1
    codes = np.zeros((R, C // 2), dtype=np.uint8)
    scales = np.zeros((R, C // 32), dtype=np.uint8)
    rc = lib().oracle_quant_mx(x, rows, cols, axis, had_n, had, sign_seed, rnd, sr_seed,
                               r0, r1, codes, scales)
    if rc:
        raise ValueError("oracle_quant_mx rejected its arguments")
    if (r0, r1) != (0, R):
        return codes[r0:r1].copy(), scales[r0:r1].copy()
    return codes, scales


def dequant_mx(codes, scales) -> np.ndarray:
    """Exact binary64 values of an MXFP4 matrix [R, C]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    R, C = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((R, C), dtype=np.float64)
    lib().oracle_dequant_mx(codes, scales, C, 0, R, out)
    return out


def gemm_rows(aq, as_, bq, bs, m0=0, m1=None):
    """Rows m0..m1-1 of C = A B^T (binary64) and S = |A| |B|^T."""
    aq, as_, bq, bs = (np.ascontiguousarray(t, np.uint8) for t in (aq, as_, bq, bs))
    M, K = aq.shape[0], aq.shape[1] * 2
    N = bq.shape[0]
    assert bq.shape[1] * 2 == K and as_.shape == (M, K // 32) and bs.shape == (N, K // 32)
    m1 = M if m1 is None else m1
    if not 0 <= m0 <= m1 <= M:
        raise ValueError("rows %d..%d outside 0..%d" % (m0, m1, M))
    c = np.zeros((m1 - m0, N), dtype=np.float64)
    s = np.zeros((m1 - m0, N), dtype=np.float64)
    lib().oracle_gemm_mx_rows(aq, as_, bq, bs, M, N, K, m0, m1, c, s)
    return c, s


def gemm_entries(aq, as_, bq, bs, mi, ni):
    """Entries (mi[t], ni[t]) of C = A B^T (binary64) and of S."""
    aq, as_, bq, bs = (np.ascontiguousarray(t, np.uint8) for t in (aq, as_, bq, bs))
    K = aq.shape[1] * 2
    mi = np.ascontiguousarray(mi, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    if mi.shape != ni.shape or (mi.size and (mi.min() < 0 or mi.max() >= aq.shape[0] or
                                            ni.min() < 0 or ni.max() >= bq.shape[0])):
        raise ValueError("entry indices outside the product")
    c = np.zeros(mi.shape[0], dtype=np.float64)
    s = np.zeros(mi.shape[0], dtype=np.float64)
    lib().oracle_gemm_mx_entries(aq, as_, bq, bs, K, mi, ni, mi.shape[0], c, s)
    return c, s


# --- NVFP4 -------------------------------------------------------------------

def nvfp4_amax(x, had=HAD_SIGNED, sign_seed=0) -> np.float32:
    x = _bits16(x)
    return np.float32(lib().oracle_nvfp4_amax(x, x.shape[0], x.shape[1], had, sign_seed))


NV_RTN, NV_RENORM_SR, NV_ELEMENT_SR = 0, 1, 2


def nvfp4_quantize(x, had=HAD_SIGNED, sign_seed=0, mode=NV_RENORM_SR, sr_seed=0, amax_in=None):
    """NVFP4 codes [rows, cols/2], E4M3 scales [rows, cols/16], tensor scale.
    mode: NV_RTN, NV_RENORM_SR (renormalized scales by SR) or NV_ELEMENT_SR."""
    x = _bits16(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    ts = ctypes.c_float(0.0)
    amax_ptr = None
    if amax_in is not None:
        amax_buf = ctypes.c_float(float(amax_in))
        amax_ptr = ctypes.cast(ctypes.pointer(amax_buf), ctypes.c_void_p)
    rc = lib().oracle_nvfp4_quantize(x, rows, cols, had, sign_seed, mode, sr_seed,
                                     amax_ptr, codes, scales, ctypes.byref(ts))
    if rc:
        raise ValueError("oracle_nvfp4_quantize rejected its arguments")
    return codes, scales, np.float32(ts.value)


def num_threads() -> int:
    return lib().oracle_num_threads()
