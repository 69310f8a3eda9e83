"""Whole-tensor parity at the Llama-3.1-8B layer sizes, through the launches
the benchmark and the linear layer make:

  * fp4_wgrad_quantize (both Wgrad operands in one launch) on the whole of
    dY and X of q_proj, gate_up and down_proj, under the deterministic and
    the random-sign rotation with RTN and under SR without rotation: every
    code and scale byte equal to the oracle's;
  * fp4_hadamard_quantize_dual on the whole of X, W and dY of gate_up: both
    outputs byte-equal to the oracle's two quantizations;
  * the Wgrad GEMM on oracle-quantized operands: every entry of the dW of
    q_proj [4096 x 4096], gate_up [14336 x 4096] and down_proj
    [4096 x 14336] within 1e-5 sum |a b| of the binary64 oracle product;
  * the linear layer (MXFP4LinearFunction) at q_proj's size: all of Y, dX
    and dW within the bf16-output bound of test_gpu_linear.py.

Inputs are the seeded workload tensors (workloads.py); no expected value
comes from the GPU path."""
import functools

import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
import workloads as W
from _util import (gemm_check, group_scales, need_gpu, say, sentinel_u8, tile_codes, to_gpu_bf16,
                   to_gpu_u8, ungroup_scales, untile_codes)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = 1e-5
O_HAD = {F.HAD_NONE: O.HAD_NONE, F.HAD_DET: O.HAD_DET, F.HAD_SIGNED: O.HAD_SIGNED}
O_RND = {F.RTN: O.RND_RTN, F.SR: O.RND_SR}
# (rotation, sign seed, rounding, SR seed of dY, SR seed of X)
WGRAD_MODES = {"det_rtn": (F.HAD_DET, 0, F.RTN, 0, 0),
               "signed_rtn": (F.HAD_SIGNED, 7, F.RTN, 0, 0),
               "none_sr": (F.HAD_NONE, 0, F.SR, 1, 2)}


@functools.lru_cache(maxsize=8)
def tensor(wname, tname):
    return W.tensor(W.WORKLOADS[wname], tname)


def host(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("mode", sorted(WGRAD_MODES))
@pytest.mark.parametrize("wname", ["q_proj", "gate_up", "down_proj"])
def test_wgrad_quantize_whole(wname, mode):
    need_gpu()
    w = W.WORKLOADS[wname]
    had, seed, rnd, sr_dy, sr_x = WGRAD_MODES[mode]
    dyb, xb = tensor(wname, "dY"), tensor(wname, "X")
    shapes = (*F.mx_shapes(w.T, w.N, F.AXIS_ROWS), *F.mx_shapes(w.T, w.K, F.AXIS_ROWS))
    out = tuple(sentinel_u8(s) for s in shapes)
    say("whole wgrad quantize", wname, mode, w.T, w.N, w.K)
    F.fp4_wgrad_quantize(to_gpu_bf16(dyb), to_gpu_bf16(xb), 32, had, seed, rnd, sr_dy, sr_x, out=out)
    torch.cuda.synchronize()
    nb = w.T // 32
    for (c, s), bits, sr, cols, what in (((out[0], out[1]), dyb, sr_dy, w.N, "dY^T"),
                                         ((out[2], out[3]), xb, sr_x, w.K, "X^T")):
        rc, rs = O.quant_mx(bits, O.AXIS_ROWS, 32, O_HAD[had], seed, O_RND[rnd], sr)
        gc, gs = host(c), host(s)
        assert np.array_equal(untile_codes(gc, cols), rc), "%s codes" % what
        assert np.array_equal(ungroup_scales(gs, nb), rs), "%s scales" % what
        # the padding rows of the last code tile and scale-group tail: none
        # here (row counts are multiples of 32, T/32 of 8), so every byte of
        # both buffers was written
        assert gc.size == rc.size and gs.size == rs.size


# (tensor, rows output: had_n, rotation, rounding; cols output: the same)
DUAL = [("X", (32, F.HAD_DET, F.RTN), (32, F.HAD_NONE, F.RTN)),
        ("W", (32, F.HAD_NONE, F.RTN), (16, F.HAD_SIGNED, F.RTN)),
        ("dY", (32, F.HAD_SIGNED, F.SR), (32, F.HAD_NONE, F.SR))]


@pytest.mark.parametrize("tname,rows_mode,cols_mode", DUAL, ids=[d[0] for d in DUAL])
def test_dual_whole(tname, rows_mode, cols_mode):
    need_gpu()
    bits = tensor("gate_up", tname)
    R, C = bits.shape
    (hr, ar, rr), (hc, ac, rc_) = rows_mode, cols_mode
    say("whole dual quantize gate_up", tname, R, C)
    rq, rs, cq, cs = F.fp4_hadamard_quantize_dual(to_gpu_bf16(bits), hr, ar, 2024, rr, 11, hc, ac, 2025, rc_, 12)
    torch.cuda.synchronize()
    want_r = O.quant_mx(bits, O.AXIS_ROWS, hr, O_HAD[ar], 2024, O_RND[rr], 11)
    want_c = O.quant_mx(bits, O.AXIS_COLS, hc, O_HAD[ac], 2025, O_RND[rc_], 12)
    assert np.array_equal(untile_codes(host(rq), C), want_r[0]), "rows-output codes"
    assert np.array_equal(ungroup_scales(host(rs), R // 32), want_r[1]), "rows-output scales"
    assert np.array_equal(untile_codes(host(cq), R), want_c[0]), "cols-output codes"
    assert np.array_equal(ungroup_scales(host(cs), C // 32), want_c[1]), "cols-output scales"


def wgrad_operands(wname):
    """The oracle's deterministic-Hadamard RTN quantization of dY and X
    along tokens (dW = dY^T X)."""
    a = O.quant_mx(tensor(wname, "dY"), O.AXIS_ROWS, 32, O.HAD_DET, 0, O.RND_RTN, 0)
    b = O.quant_mx(tensor(wname, "X"), O.AXIS_ROWS, 32, O.HAD_DET, 0, O.RND_RTN, 0)
    return a, b


def gpu_wgrad(a, b, M, N):
    g = [to_gpu_u8(x) for x in (tile_codes(a[0], 0xCD), group_scales(a[1]), tile_codes(b[0], 0xCD),
                                group_scales(b[1]))]
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    F.fp4_gemm_wgrad(*g, out=out)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("wname", ["q_proj", "gate_up", "down_proj"])
def test_wgrad_gemm_whole(wname):
    need_gpu()
    w = W.WORKLOADS[wname]
    M, N = w.N, w.K
    a, b = wgrad_operands(wname)
    say("whole wgrad gemm", wname, M, N, w.T)
    got = gpu_wgrad(a, b, M, N)
    assert np.isfinite(got).all()
    # in bands of 2048 rows (bounded host memory for the binary64 reference)
    for r0 in range(0, M, 2048):
        r1 = min(M, r0 + 2048)
        ref, mag = O.gemm_rows(*a, *b, r0, r1)
        gemm_check(got[r0:r1], ref, mag, TOL)


def test_linear_layer_q_proj_size():
    """Y = X W^T, dX = dY W, dW = dY^T X of MXFP4LinearFunction at
    T = 8192, K = N = 4096, random-sign rotation with SR on the Wgrad pair."""
    need_gpu()
    from test_gpu_linear import SR_COLS_SEED_XOR, check
    xb, wb, dyb = tensor("q_proj", "X"), tensor("q_proj", "W"), tensor("q_proj", "dY")
    seed, sr = 1234, 77
    say("linear q_proj size", xb.shape, wb.shape, dyb.shape)
    x = to_gpu_bf16(xb).requires_grad_(True)
    wt = to_gpu_bf16(wb).requires_grad_(True)
    y = F.linear.MXFP4LinearFunction.apply(x, wt, F.HAD_SIGNED, 32, seed, F.SR, sr)
    y.backward(to_gpu_bf16(dyb))
    torch.cuda.synchronize()
    ref, mag = O.gemm_rows(*O.quant_mx(xb, O.AXIS_COLS), *O.quant_mx(wb, O.AXIS_COLS))
    check(y, ref, mag, "Y")
    dyc = O.quant_mx(dyb, O.AXIS_COLS, 32, O.HAD_NONE, 0, O.RND_SR, sr ^ SR_COLS_SEED_XOR)
    ref, mag = O.gemm_rows(*dyc, *O.quant_mx(wb, O.AXIS_ROWS))
    check(x.grad, ref, mag, "dX")
    dyt = O.quant_mx(dyb, O.AXIS_ROWS, 32, O.HAD_SIGNED, seed, O.RND_SR, sr)
    xt = O.quant_mx(xb, O.AXIS_ROWS, 32, O.HAD_SIGNED, seed)
    ref, mag = O.gemm_rows(*dyt, *xt)
    check(wt.grad, ref, mag, "dW")
