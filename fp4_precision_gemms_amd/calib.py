"""Binding of libfp4calib.so (include/fp4_calib.h): the scaled FP4 MFMA rate
the card sustains under its power limit, on random operands or on a real
product's own quantized operands, with the shader clock it ran at.  A
measurement aid for the GEMM's roofline, not part of the quantized-GEMM
path."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4calib.so")
REFCLK_HZ = 100e6          # the reference clock behind s_memrealtime
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp4calib.so is not built: run `python -m fp4_precision_gemms_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.fp4_calib_mfma_src_bytes.argtypes = [ctypes.c_int]
        L.fp4_calib_mfma_src_bytes.restype = ctypes.c_size_t
        L.fp4_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        L.fp4_calib_mfma_flops.restype = ctypes.c_double
        L.fp4_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.fp4_calib_mfma.restype = ctypes.c_int
        L.fp4_calib_clock_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.fp4_calib_clock_stamp.restype = ctypes.c_int
        _lib = L
    return _lib


def operand_fragments(a_codes, b_codes, waves: int):
    """The MFMA-only loop's operands taken from real MXFP4 operands in the
    library's 32-row tiled layout (whose consecutive 1 KB pieces are the
    32x32x64 MFMA operands in lane order): wave w's A fragments are pieces
    14 w .. 14 w + 13 of `a_codes` and its B fragments pieces 4 w .. 4 w + 3
    of `b_codes` (modulo their piece counts), in the loop's fragment order."""
    fa, fb = a_codes.reshape(-1, 1024), b_codes.reshape(-1, 1024)
    dev = a_codes.device
    w = torch.arange(waves, device=dev)
    ia = (w[:, None, None] * 14 + torch.arange(2, device=dev)[None, :, None] * 7 +
          torch.arange(7, device=dev)[None, None, :]) % fa.shape[0]
    ib = (w[:, None, None] * 4 + torch.arange(2, device=dev)[None, :, None] * 2 +
          torch.arange(2, device=dev)[None, None, :]) % fb.shape[0]
    # [waves, set, 7 A + 2 B, 1024]
    return torch.cat([fa[ia], fb[ib]], dim=2).reshape(-1).contiguous()


def mfma_ceiling(device, iters: int = 20000, warmup: int = 20, launches: int = 10, seed: int = 0,
                 operands=None) -> dict:
    """Runs the MFMA-only loop on one workgroup per CU: `warmup` launches to
    let the clocks settle, then `launches` timed ones (HIP events on the
    launch stream).  Operands: random E2M1 bytes, or `operands` = (A codes,
    B codes) of a real product (see operand_fragments) -- the matrix cores'
    power, and so their rate under the power limit, depends on the data.
    Returns TFLOP/s and the median shader clock over all waves of the timed
    launches."""
    L = lib()
    grid = torch.cuda.get_device_properties(device).multi_processor_count
    if operands is None:
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        src = torch.randint(0, 256, (L.fp4_calib_mfma_src_bytes(grid),), dtype=torch.uint8,
                            device=device, generator=g)
    else:
        src = operand_fragments(operands[0], operands[1], grid * 4)
        if src.numel() != L.fp4_calib_mfma_src_bytes(grid):
            raise ValueError("operand fragments: %d bytes, the loop takes %d"
                             % (src.numel(), L.fp4_calib_mfma_src_bytes(grid)))
    out = torch.empty(grid * 256, dtype=torch.float32, device=device)
    clocks = torch.zeros((launches, grid * 4, 2), dtype=torch.int64, device=device)
    stream = torch.cuda.current_stream(device)

    def launch(ck):
        st = L.fp4_calib_mfma(src.data_ptr(), grid, iters, out.data_ptr(), ck.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError("fp4_calib_mfma failed with status %d" % st)

    for _ in range(warmup):
        launch(clocks[0])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(launches):
        launch(clocks[i])
    e1.record(stream)
    torch.cuda.synchronize(device)
    sec = e0.elapsed_time(e1) * 1e-3 / launches
    ck = clocks.double().cpu()
    sclk = (ck[..., 0] / ck[..., 1]).median().item() * REFCLK_HZ
    tflops = L.fp4_calib_mfma_flops(grid, iters) / sec / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "sclk_GHz": sclk / 1e9, "grid": grid, "iters": iters,
            "ms_per_launch": sec * 1e3,
            "what": "scaled FP4 MFMA 32x32x64 only, %s E2M1 operands in registers, the Wgrad "
                    "GEMM's wave tile (7x2 accumulators, two fragment sets), one workgroup of 4 "
                    "waves per CU" % ("random" if operands is None else "the product's own")}


STAMPS = 32                  # workgroups per clock stamp (FP4_CALIB_STAMPS)


def span_ghz(begin, end) -> float:
    """Shader clock in GHz between two clock stamps (lists of [shader ticks,
    reference ticks, XCD id, 0] records): each XCD's first record in `begin`
    is paired with its first in `end`; the median ratio over the pairs.
    NaN if no XCD appears in both."""
    first = {}
    for rec in begin:
        first.setdefault(rec[2], rec)
    ratios = []
    for rec in end:
        f = first.pop(rec[2], None)
        if f is not None and rec[1] > f[1]:
            ratios.append((rec[0] - f[0]) / (rec[1] - f[1]))
    if not ratios:
        return float("nan")
    ratios.sort()
    return ratios[len(ratios) // 2] * REFCLK_HZ / 1e9


class ClockSpan:
    """The average shader clock over the work enqueued on `stream` between
    begin() and end(): a clock-stamp launch at each end, read per XCD (the
    median over the XCDs both stamps reached)."""

    def __init__(self, device, stream=None):
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        self.buf = torch.zeros((2, STAMPS, 4), dtype=torch.int64, device=device)

    def _stamp(self, i):
        st = lib().fp4_calib_clock_stamp(self.buf[i].data_ptr(), self.stream.cuda_stream)
        if st != 0:
            raise RuntimeError("fp4_calib_clock_stamp failed with status %d" % st)

    def begin(self):
        self._stamp(0)

    def end(self):
        self._stamp(1)

    def ghz(self) -> float:
        """Shader clock in GHz (synchronizes); NaN if no XCD was stamped twice."""
        torch.cuda.synchronize(self.buf.device)
        b = self.buf.cpu().tolist()
        return span_ghz(b[0], b[1])
