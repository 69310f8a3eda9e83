"""The C ABI without a GPU: libfp4.so loads, exports every entry point that
include/fp4.h declares, and rejects bad arguments with the documented status
codes before making any HIP call (fake pointers below are never touched)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import fp4_precision_gemms_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ENUM, ERR_LAUNCH, ERR_WORKSPACE = range(7)
A = 0x10000          # a fake 16-byte aligned device address (never dereferenced)
MIS = 0x10008        # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(F.LIB_PATH):
        pytest.skip("libfp4.so not built")
    return F.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp4_hadamard_quantize", "fp4_gemm_fprop", "fp4_gemm_dgrad", "fp4_gemm_wgrad",
              "fp4_gemm_mx", "fp4_hadamard_quantize_dual", "fp4_wgrad_quantize", "nvfp4_quantize",
              "nvfp4_workspace_bytes", "fp4_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    out = subprocess.check_output(["nm", "-D", "--defined-only", F.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in declared_functions():
        assert n in exported, n
        assert getattr(L, n) is not None


def test_status_strings(L):
    for s in range(7):
        assert F.fp4_status_string(s).startswith("FP4_")
    assert F.fp4_status_string(99) == "FP4_ERR_UNKNOWN"


def q(L, x=A, rows=64, cols=64, axis=0, had_n=32, had=1, rnd=0, codes=A, scales=A):
    return L.fp4_hadamard_quantize(x, rows, cols, axis, had_n, had, 0, rnd, 0, codes, scales, None)


def test_quantize_errors(L):
    assert q(L, axis=2) == ERR_ENUM
    assert q(L, had=3) == ERR_ENUM
    assert q(L, had_n=8) == ERR_ENUM
    assert q(L, rnd=2) == ERR_ENUM
    assert q(L, x=None) == ERR_NULL
    assert q(L, codes=None) == ERR_NULL
    assert q(L, scales=None) == ERR_NULL
    assert q(L, rows=0) == ERR_SHAPE
    assert q(L, cols=-32) == ERR_SHAPE
    assert q(L, cols=48) == ERR_SHAPE                  # contraction along cols
    assert q(L, rows=48, axis=1) == ERR_SHAPE          # contraction along rows
    assert q(L, rows=2 ** 40, cols=2 ** 40) == ERR_SHAPE
    assert q(L, x=MIS) == ERR_ALIGN
    assert q(L, codes=MIS) == ERR_ALIGN
    # had_n is not checked when there is no rotation, but the shape still is
    assert q(L, had=0, had_n=7, cols=40) == ERR_SHAPE


@pytest.mark.parametrize("name", ["fp4_gemm_fprop", "fp4_gemm_dgrad", "fp4_gemm_wgrad"])
def test_gemm_errors(L, name):
    fn = getattr(L, name)
    # contraction dim per role: fprop K, dgrad N, wgrad T
    contraction = {"fp4_gemm_fprop": 2, "fp4_gemm_dgrad": 1, "fp4_gemm_wgrad": 0}[name]

    def call(ptrs=(A, A, A, A), dims=(64, 64, 64), out=A):
        return fn(*ptrs, *dims, out, None)

    assert call(ptrs=(None, A, A, A)) == ERR_NULL
    assert call(ptrs=(A, A, A, None)) == ERR_NULL
    assert call(out=None) == ERR_NULL
    for bad in (0, -1):
        for d in range(3):
            dims = [64, 64, 64]
            dims[d] = bad
            assert call(dims=tuple(dims)) == ERR_SHAPE
    dims = [64, 64, 64]
    dims[contraction] = 48
    assert call(dims=tuple(dims)) == ERR_SHAPE
    dims[contraction] = 2 ** 24                        # beyond the 32-bit tile offsets
    assert call(dims=tuple(dims)) == ERR_SHAPE
    dims[contraction] = 2 ** 24 - 32
    assert call(dims=tuple(dims), out=MIS) == ERR_ALIGN
    # a non-contraction dim of 48 is fine shape-wise: prove it with a misaligned out
    dims = [64, 64, 64]
    dims[(contraction + 1) % 3] = 48
    assert call(dims=tuple(dims), out=MIS) == ERR_ALIGN
    assert call(ptrs=(A, MIS, A, A)) == ERR_ALIGN


def test_quantize_dual_errors(L):
    def call(x=A, rows=64, cols=64, hn=(32, 32), had=(1, 0), rnd=(0, 0), ptrs=(A, A, A, A)):
        return L.fp4_hadamard_quantize_dual(x, rows, cols, hn[0], had[0], 0, rnd[0], 0, ptrs[0], ptrs[1],
                                            hn[1], had[1], 0, rnd[1], 0, ptrs[2], ptrs[3], None)

    assert call(had=(3, 0)) == ERR_ENUM
    assert call(had=(0, 5)) == ERR_ENUM
    assert call(hn=(8, 32)) == ERR_ENUM
    assert call(hn=(32, 8), had=(1, 2)) == ERR_ENUM
    assert call(rnd=(0, 2)) == ERR_ENUM
    assert call(x=None) == ERR_NULL
    assert call(ptrs=(A, A, A, None)) == ERR_NULL
    assert call(rows=48) == ERR_SHAPE                  # both axes are contractions
    assert call(cols=80) == ERR_SHAPE
    assert call(rows=0) == ERR_SHAPE
    assert call(ptrs=(A, A, MIS, A)) == ERR_ALIGN
    assert call(x=MIS) == ERR_ALIGN


def test_wgrad_quantize_errors(L):
    def call(T=64, N=64, K=64, hn=32, had=1, rnd=0, p=(A, A, A, A, A, A)):
        return L.fp4_wgrad_quantize(p[0], p[1], T, N, K, hn, had, 0, rnd, 0, 0, p[2], p[3], p[4], p[5], None)

    assert call(had=3) == ERR_ENUM
    assert call(hn=8) == ERR_ENUM
    assert call(rnd=2) == ERR_ENUM
    assert call(p=(A, None, A, A, A, A)) == ERR_NULL
    assert call(p=(A, A, A, A, A, None)) == ERR_NULL
    assert call(T=48) == ERR_SHAPE
    assert call(K=0) == ERR_SHAPE
    assert call(N=-1) == ERR_SHAPE
    assert call(p=(A, A, A, MIS, A, A)) == ERR_ALIGN


def test_gemm_mx_errors(L):
    def call(ptrs=(A, A, A, A), dims=(64, 64, 64), out=A, dtype=0, acc=0):
        return L.fp4_gemm_mx(*ptrs, *dims, out, dtype, acc, None)

    assert call(dtype=2) == ERR_ENUM
    assert call(dtype=-1) == ERR_ENUM
    assert call(acc=2) == ERR_ENUM
    assert call(ptrs=(A, None, A, A)) == ERR_NULL
    assert call(out=None, dtype=1) == ERR_NULL
    assert call(dims=(64, 64, 48)) == ERR_SHAPE
    assert call(dims=(64, 0, 64), dtype=1, acc=1) == ERR_SHAPE
    assert call(out=MIS, dtype=1) == ERR_ALIGN
    assert call(out=MIS, acc=1) == ERR_ALIGN


def test_nvfp4_errors(L):
    def call(x=A, rows=32, cols=64, had=2, mode=1, amax=None, codes=A, scales=A, ts=A,
             ws=A, wsb=256):
        return L.nvfp4_quantize(x, rows, cols, had, 0, mode, 0, amax, codes, scales, ts, ws, wsb,
                                None)

    assert call(had=5) == ERR_ENUM
    assert call(mode=3) == ERR_ENUM
    assert call(mode=-1) == ERR_ENUM
    assert call(x=None) == ERR_NULL
    assert call(ts=None) == ERR_NULL
    assert call(cols=24) == ERR_SHAPE
    assert call(rows=0) == ERR_SHAPE
    assert call(x=MIS) == ERR_ALIGN
    assert call(ts=A + 2) == ERR_ALIGN
    assert call(ws=None) == ERR_WORKSPACE
    assert call(wsb=4) == ERR_WORKSPACE
    assert L.nvfp4_workspace_bytes(32, 64) >= 4


def test_nvfp4_noalloc_errors(L):
    """The allocation-free NVFP4 entry point checks its arguments like
    nvfp4_quantize, before any HIP call."""
    def call(x=A, rows=32, cols=64, had=2, mode=1, amax=None, codes=A, scales=A, ts=A):
        return L.nvfp4_quantize_noalloc(x, rows, cols, had, 0, mode, 0, amax, codes, scales, ts, None)

    assert call(had=5) == ERR_ENUM
    assert call(mode=3) == ERR_ENUM
    assert call(x=None) == ERR_NULL
    assert call(codes=None) == ERR_NULL
    assert call(ts=None) == ERR_NULL
    assert call(cols=24) == ERR_SHAPE
    assert call(rows=-1) == ERR_SHAPE
    assert call(scales=MIS) == ERR_ALIGN
    assert call(amax=A + 2) == ERR_ALIGN
    assert "nvfp4_quantize_noalloc" in declared_functions()


def test_binding_refuses_cpu_tensors():
    import torch
    if not os.path.exists(F.LIB_PATH):
        pytest.skip("libfp4.so not built")
    with pytest.raises((ValueError, TypeError)):
        F.fp4_hadamard_quantize(torch.zeros(32, 32, dtype=torch.bfloat16))


def test_grouped_scale_layout_helpers():
    """The k-grouped MXFP4 scale layout of include/fp4.h: block b of row r at
    byte ((b // 8) * R + r) * 8 + b % 8 of a [ceil(nb/8), R, 8] array."""
    from _util import group_scales, ungroup_scales
    rng = np.random.default_rng(3)
    R, nb = 37, 13
    s = rng.integers(0, 255, (R, nb), dtype=np.uint8)
    g = group_scales(s)
    assert g.shape == (2, R, 8)
    flat = g.reshape(-1)
    for r in range(R):
        for b in range(nb):
            assert flat[((b // 8) * R + r) * 8 + b % 8] == s[r, b]
    assert (g[1, :, nb - 8:] == 0xFF).all()
    assert np.array_equal(ungroup_scales(g, nb), s)
    assert F.mx_shapes(64, 416, F.AXIS_COLS) == ((2, 13, 512), (2, 64, 8))
    assert F.mx_shapes(416, 64, F.AXIS_ROWS) == ((2, 13, 512), (2, 64, 8))
    assert F.mx_shapes(3, 256, F.AXIS_COLS) == ((1, 8, 512), (1, 3, 8))
    assert F.mx_shapes(33, 96, F.AXIS_COLS)[0] == (2, 3, 512)


def test_binding_checks_output_extents():
    """Outputs that the kernels would write past the end of are refused
    before any launch (the shape checks come before the device checks)."""
    import torch
    T, N, K = 64, 96, 32
    dy, x = torch.zeros(T, N, dtype=torch.bfloat16), torch.zeros(T, K, dtype=torch.bfloat16)
    (a, b), (c, d) = F.mx_shapes(T, N, F.AXIS_ROWS), F.mx_shapes(T, K, F.AXIS_ROWS)
    u8 = lambda sh: torch.zeros(sh, dtype=torch.uint8)
    # the two operands' buffers swapped: dY's outputs too small
    with pytest.raises(ValueError, match="shape"):
        F.fp4_wgrad_quantize(dy, x, out=(u8(c), u8(d), u8(a), u8(b)))
    with pytest.raises(ValueError, match="out must be"):
        F.fp4_wgrad_quantize(dy, x, out=(u8(a), u8(b), u8(c)))
    xn = torch.zeros(32, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="codes must have shape"):
        F.nvfp4_quantize(xn, codes=u8((32, 16)))
    with pytest.raises(ValueError, match="scales must have shape"):
        F.nvfp4_quantize(xn, scales=u8((32, 2)))
    with pytest.raises(ValueError, match="tensor_scale"):
        F.nvfp4_quantize(xn, tensor_scale=torch.zeros(2))
    # right extents on CPU tensors: refused as not on the GPU, not for shape
    with pytest.raises(ValueError, match="GPU"):
        F.fp4_wgrad_quantize(dy, x, out=(u8(a), u8(b), u8(c), u8(d)))
