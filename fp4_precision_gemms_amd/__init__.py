"""Python binding of libfp4.so, the MXFP4 / NVFP4 block-quantized linear layer
for AMD Instinct MI355X (gfx950).

The functions below carry the names of the C entry points (include/fp4.h)
and only marshal arguments: shapes and pointers of torch tensors in, status
codes out.  Every step of the computation runs in the HIP kernels of the
library.  torch supplies device memory and the current HIP stream.

If libfp4.so has not been built (``python -m fp4_precision_gemms_amd.build``)
every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

AXIS_COLS, AXIS_ROWS = 0, 1
HAD_NONE, HAD_DET, HAD_SIGNED = 0, 1, 2
RTN, SR = 0, 1
OUT_F32, OUT_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4.so")
_lib = None


class Fp4Error(RuntimeError):
    """A nonzero fp4_status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libfp4.so with argument types set; raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfp4.so is not built: run `python -m fp4_precision_gemms_amd.build` "
                           "(expected at %s)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, u64, i32, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
    L.fp4_hadamard_quantize.argtypes = [vp, i64, i64, i32, i32, i32, u64, i32, u64, vp, vp, vp]
    L.fp4_hadamard_quantize.restype = i32
    for name in ("fp4_gemm_fprop", "fp4_gemm_dgrad", "fp4_gemm_wgrad"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp]
        fn.restype = i32
    L.fp4_hadamard_quantize_dual.argtypes = [vp, i64, i64, i32, i32, u64, i32, u64, vp, vp,
                                             i32, i32, u64, i32, u64, vp, vp, vp]
    L.fp4_hadamard_quantize_dual.restype = i32
    L.fp4_wgrad_quantize.argtypes = [vp, vp, i64, i64, i64, i32, i32, u64, i32, u64, u64,
                                     vp, vp, vp, vp, vp]
    L.fp4_wgrad_quantize.restype = i32
    L.fp4_gemm_mx.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, i32, vp]
    L.fp4_gemm_mx.restype = i32
    L.nvfp4_quantize.argtypes = [vp, i64, i64, i32, u64, i32, u64, vp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    L.nvfp4_quantize.restype = i32
    L.nvfp4_quantize_noalloc.argtypes = [vp, i64, i64, i32, u64, i32, u64, vp, vp, vp, vp, vp]
    L.nvfp4_quantize_noalloc.restype = i32
    L.nvfp4_workspace_bytes.argtypes = [i64, i64]
    L.nvfp4_workspace_bytes.restype = ctypes.c_size_t
    L.fp4_status_string.argtypes = [i32]
    L.fp4_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def fp4_status_string(status: int) -> str:
    return lib().fp4_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise Fp4Error(status, fp4_status_string(status))


def _stream_ptr(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def code_shape(R: int, C: int):
    """Shape of the MXFP4 codes of R rows of C contraction elements in the
    library's 32-row tiled layout: for each group of 32 rows and each
    32-element block, the 32 rows' 16 code bytes are one 512-byte chunk
    ([ceil(R/32), C/32, 512]; row r at bytes 16 (r mod 32) of its chunk)."""
    return ((R + 31) // 32, C // 32, 512)


def scale_shape(R: int, C: int):
    """k-grouped E8M0 scale shape of R rows of C contraction elements:
    [ceil(C/256), R, 8], block b of row r at [b // 8, r, b % 8]."""
    return ((C // 32 + 7) // 8, R, 8)


def mx_shapes(rows: int, cols: int, axis: int):
    """(codes shape, scales shape) of fp4_hadamard_quantize's outputs for
    x[rows, cols] along `axis` (the logical operand has R rows of C
    contraction elements: (rows, cols) along cols, (cols, rows) along rows)."""
    R, C = (rows, cols) if axis == AXIS_COLS else (cols, rows)
    return code_shape(R, C), scale_shape(R, C)


def mx_dims(codes: torch.Tensor, scales: torch.Tensor):
    """(R, C) of an MXFP4 operand from its codes and scales, checking that
    the two agree."""
    if codes.dim() != 3 or scales.dim() != 3:
        raise ValueError("MXFP4 operands are codes [ceil(R/32), C/32, 512] and scales [ceil(C/256), R, 8]")
    R, C = scales.shape[1], codes.shape[1] * 32
    if tuple(codes.shape) != code_shape(R, C) or tuple(scales.shape) != scale_shape(R, C):
        raise ValueError("codes %s and scales %s do not describe one operand"
                         % (tuple(codes.shape), tuple(scales.shape)))
    return R, C


def fp4_hadamard_quantize(x: torch.Tensor, axis: int = AXIS_COLS, had_n: int = 32,
                          had: int = HAD_NONE, sign_seed: int = 0, rnd: int = RTN,
                          sr_seed: int = 0, codes: torch.Tensor | None = None,
                          scales: torch.Tensor | None = None, stream=None):
    """MXFP4 codes and E8M0 scales of bf16 x[rows, cols] (see include/fp4.h)."""
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    cshape, sshape = mx_shapes(rows, cols, axis)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if tuple(codes.shape) != cshape or tuple(scales.shape) != sshape:
        raise ValueError("output shapes must be %s and %s" % (cshape, sshape))
    _check(lib().fp4_hadamard_quantize(x.data_ptr(), rows, cols, axis, had_n, had,
                                       sign_seed & (2 ** 64 - 1), rnd, sr_seed & (2 ** 64 - 1),
                                       codes.data_ptr(), scales.data_ptr(),
                                       _stream_ptr(stream, x.device)))
    return codes, scales


def fp4_hadamard_quantize_dual(x: torch.Tensor, had_n_rows: int = 32, had_rows: int = HAD_NONE,
                               sign_seed_rows: int = 0, rnd_rows: int = RTN, sr_seed_rows: int = 0,
                               had_n_cols: int = 32, had_cols: int = HAD_NONE, sign_seed_cols: int = 0,
                               rnd_cols: int = RTN, sr_seed_cols: int = 0, out=None, stream=None):
    """Both quantizations of bf16 x[rows, cols] from one read: (codes, scales)
    along rows (as AXIS_ROWS) and along cols (as AXIS_COLS), each with its own
    rotation and rounding (see include/fp4.h).  `out`: optional preallocated
    (codes_rows, scales_rows, codes_cols, scales_cols)."""
    _need(x, torch.bfloat16, "x")
    rows, cols = x.shape
    (cr, sr), (cc, sc) = mx_shapes(rows, cols, AXIS_ROWS), mx_shapes(rows, cols, AXIS_COLS)
    dev = x.device
    if out is None:
        out = [torch.empty(sh, dtype=torch.uint8, device=dev) for sh in (cr, sr, cc, sc)]
    for t, sh in zip(out, (cr, sr, cc, sc)):
        _need(t, torch.uint8, "output")
        if tuple(t.shape) != tuple(sh):
            raise ValueError("output of shape %s expected, got %s" % (sh, tuple(t.shape)))
    m = 2 ** 64 - 1
    _check(lib().fp4_hadamard_quantize_dual(
        x.data_ptr(), rows, cols, had_n_rows, had_rows, sign_seed_rows & m, rnd_rows, sr_seed_rows & m,
        out[0].data_ptr(), out[1].data_ptr(), had_n_cols, had_cols, sign_seed_cols & m, rnd_cols,
        sr_seed_cols & m, out[2].data_ptr(), out[3].data_ptr(), _stream_ptr(stream, dev)))
    return tuple(out)


def fp4_wgrad_quantize(dy: torch.Tensor, x: torch.Tensor, had_n: int = 32, had: int = HAD_DET,
                       sign_seed: int = 0, rnd: int = RTN, sr_seed_dy: int = 0, sr_seed_x: int = 0,
                       out=None, stream=None):
    """The Wgrad operand pair: dY[T, N] and X[T, K] quantized along T with one
    rotation; returns (dytq, dyts, xtq, xts) (see include/fp4.h)."""
    T, N = dy.shape
    if x.shape[0] != T:
        raise ValueError("dy and x must have the same number of rows")
    K = x.shape[1]
    (a, b), (c, d) = mx_shapes(T, N, AXIS_ROWS), mx_shapes(T, K, AXIS_ROWS)
    if out is not None:
        # the kernels write exactly these extents: a smaller buffer would be
        # written past its end
        if len(out) != 4:
            raise ValueError("out must be (dytq, dyts, xtq, xts)")
        for t, sh, n in zip(out, (a, b, c, d), ("dytq", "dyts", "xtq", "xts")):
            if tuple(t.shape) != tuple(sh):
                raise ValueError("%s must have shape %s, got %s" % (n, tuple(sh), tuple(t.shape)))
    _need(dy, torch.bfloat16, "dy")
    _need(x, torch.bfloat16, "x")
    if out is None:
        out = tuple(torch.empty(sh, dtype=torch.uint8, device=dy.device) for sh in (a, b, c, d))
    for t in out:
        _need(t, torch.uint8, "output")
    m = 2 ** 64 - 1
    _check(lib().fp4_wgrad_quantize(dy.data_ptr(), x.data_ptr(), T, N, K, had_n, had, sign_seed & m, rnd,
                                    sr_seed_dy & m, sr_seed_x & m, *(t.data_ptr() for t in out),
                                    _stream_ptr(stream, dy.device)))
    return out


def _gemm(fn, aq, as_, bq, bs, T, N, K, out_shape, out, stream):
    for t, n in ((aq, "a codes"), (as_, "a scales"), (bq, "b codes"), (bs, "b scales")):
        _need(t, torch.uint8, n)
    if out is None:
        out = torch.empty(out_shape, dtype=torch.float32, device=aq.device)
    _need(out, torch.float32, "out")
    if tuple(out.shape) != tuple(out_shape):
        raise ValueError("out must have shape %s" % (out_shape,))
    _check(fn(aq.data_ptr(), as_.data_ptr(), bq.data_ptr(), bs.data_ptr(), T, N, K,
              out.data_ptr(), _stream_ptr(stream, aq.device)))
    return out


def _operands(aq, as_, bq, bs, what):
    M, Ka = mx_dims(aq, as_)
    N, Kb = mx_dims(bq, bs)
    if Ka != Kb:
        raise ValueError("%s operands have different contraction sizes (%d, %d)" % (what, Ka, Kb))
    return M, N, Ka


def fp4_gemm_fprop(xq, xs, wq, ws, out=None, stream=None):
    """y[T, N] = X W^T from X and W quantized along K."""
    T, N, K = _operands(xq, xs, wq, ws, "fprop")
    return _gemm(lib().fp4_gemm_fprop, xq, xs, wq, ws, T, N, K, (T, N), out, stream)


def fp4_gemm_dgrad(dyq, dys, wtq, wts, out=None, stream=None):
    """dx[T, K] = dY W from dY quantized along N and W^T (W along its rows)."""
    T, K, N = _operands(dyq, dys, wtq, wts, "dgrad")
    return _gemm(lib().fp4_gemm_dgrad, dyq, dys, wtq, wts, T, N, K, (T, K), out, stream)


def fp4_gemm_wgrad(dytq, dyts, xtq, xts, out=None, stream=None):
    """dw[N, K] = dY^T X from dY^T and X^T (both quantized along T)."""
    N, K, T = _operands(dytq, dyts, xtq, xts, "wgrad")
    return _gemm(lib().fp4_gemm_wgrad, dytq, dyts, xtq, xts, T, N, K, (N, K), out, stream)


def fp4_gemm_mx(aq, as_, bq, bs, out=None, out_dtype: int = OUT_F32, accumulate: bool = False,
                stream=None):
    """C[M, N] = A B^T (+ C when accumulate) from MXFP4 operands A [M, Kc] and
    B [N, Kc] (codes and scales as the quantizers write them); C fp32 or
    bf16 (see include/fp4.h)."""
    M, N, Kc = _operands(aq, as_, bq, bs, "gemm")
    for t, n in ((aq, "a codes"), (as_, "a scales"), (bq, "b codes"), (bs, "b scales")):
        _need(t, torch.uint8, n)
    dt = {OUT_F32: torch.float32, OUT_BF16: torch.bfloat16}[out_dtype]
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out")
        out = torch.empty((M, N), dtype=dt, device=aq.device)
    _need(out, dt, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must have shape %s" % ((M, N),))
    _check(lib().fp4_gemm_mx(aq.data_ptr(), as_.data_ptr(), bq.data_ptr(), bs.data_ptr(), M, N, Kc,
                             out.data_ptr(), out_dtype, int(bool(accumulate)),
                             _stream_ptr(stream, aq.device)))
    return out


def nvfp4_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().nvfp4_workspace_bytes(rows, cols))


NV_RTN, NV_RENORM_SR, NV_ELEMENT_SR = 0, 1, 2   # nvfp4_mode


def nvfp4_quantize(x: torch.Tensor, had: int = HAD_SIGNED, sign_seed: int = 0, mode: int = NV_RENORM_SR,
                   sr_seed: int = 0, amax_in: torch.Tensor | None = None,
                   codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   tensor_scale: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None):
    """NVFP4 codes [rows, cols/2], E4M3 scales [rows, cols/16] and the fp32
    tensor scale (a 1-element device tensor) of bf16 x (see include/fp4.h)."""
    rows, cols = x.shape
    for t, sh, n in ((codes, (rows, cols // 2), "codes"), (scales, (rows, cols // 16), "scales"),
                     (tensor_scale, (1,), "tensor_scale")):
        if t is not None and tuple(t.shape) != sh:
            raise ValueError("%s must have shape %s, got %s" % (n, sh, tuple(t.shape)))
    if amax_in is not None and amax_in.numel() != 1:
        raise ValueError("amax_in must hold one float")
    _need(x, torch.bfloat16, "x")
    dev = x.device
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev) if codes is None else codes
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev) if scales is None else scales
    tensor_scale = torch.empty(1, dtype=torch.float32, device=dev) if tensor_scale is None else tensor_scale
    for t, dt, n in ((codes, torch.uint8, "codes"), (scales, torch.uint8, "scales"),
                     (tensor_scale, torch.float32, "tensor_scale")):
        _need(t, dt, n)
    if amax_in is not None:
        _need(amax_in, torch.float32, "amax_in")
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
    if amax_in is None and workspace is None:
        workspace = torch.empty(nvfp4_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
    _check(lib().nvfp4_quantize(x.data_ptr(), rows, cols, had, sign_seed & (2 ** 64 - 1), mode,
                                sr_seed & (2 ** 64 - 1), _ptr(amax_in), codes.data_ptr(),
                                scales.data_ptr(), tensor_scale.data_ptr(), _ptr(workspace),
                                0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream_ptr(stream, dev)))
    return codes, scales, tensor_scale


def nvfp4_quantize_noalloc(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                           tensor_scale: torch.Tensor, had: int = HAD_SIGNED, sign_seed: int = 0,
                           mode: int = NV_RENORM_SR, sr_seed: int = 0,
                           amax_in: torch.Tensor | None = None, stream=None):
    """nvfp4_quantize into caller-provided outputs, with the in-library amax
    in the library's own device scratch instead of a workspace (see
    include/fp4.h: calls that overlap on one GPU race on it)."""
    rows, cols = x.shape
    for t, sh, dt, n in ((codes, (rows, cols // 2), torch.uint8, "codes"),
                         (scales, (rows, cols // 16), torch.uint8, "scales"),
                         (tensor_scale, (1,), torch.float32, "tensor_scale")):
        if tuple(t.shape) != sh:
            raise ValueError("%s must have shape %s, got %s" % (n, sh, tuple(t.shape)))
        _need(t, dt, n)
    _need(x, torch.bfloat16, "x")
    if amax_in is not None:
        if amax_in.numel() != 1:
            raise ValueError("amax_in must hold one float")
        _need(amax_in, torch.float32, "amax_in")
    _check(lib().nvfp4_quantize_noalloc(x.data_ptr(), rows, cols, had, sign_seed & (2 ** 64 - 1), mode,
                                        sr_seed & (2 ** 64 - 1), _ptr(amax_in), codes.data_ptr(),
                                        scales.data_ptr(), tensor_scale.data_ptr(),
                                        _stream_ptr(stream, x.device)))
    return codes, scales, tensor_scale


from . import linear  # noqa: E402  (the autograd layer built on the calls above)
