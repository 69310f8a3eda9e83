"""GPU check of the MFMA-rate measurement aid (libfp4calib.so): the loop
really performs the documented scaled FP4 products.  Each lane's output (the
sum of its accumulators) equals a CPU evaluation of iters x (A0 B0^T + A1 B1^T)
over the wave's 7 x 2 tiles, summed over the lane's entries of the 32 x 32
accumulator layout (row m = lane mod 32; columns 8 (r / 4) + 4 (lane / 32) +
r mod 4), and the clock readings are positive."""
import numpy as np
import pytest
import torch

from _util import need_gpu

pytestmark = pytest.mark.gpu

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)
FM, FN, NSET = 7, 2, 2


def lane_frag(src, wave, idx):
    """[64 lanes, 32 values] of 16-byte fragment `idx` of a wave: lane l
    holds row l mod 32, contraction half l div 32 (low nibble first)."""
    base = (wave * NSET * (FM + FN) + idx) * 64
    b = src[(base * 16):(base + 64) * 16].reshape(64, 16)
    codes = np.empty((64, 32), np.uint8)
    codes[:, 0::2] = b & 15
    codes[:, 1::2] = b >> 4
    return E2M1[codes]


def operand(src, wave, idx):
    """The 32 x 64 operand slice of fragment idx: [row, k]."""
    f = lane_frag(src, wave, idx)
    out = np.empty((32, 64))
    out[:, :32] = f[:32]
    out[:, 32:] = f[32:]
    return out


def test_mfma_ceiling_kernel_work():
    need_gpu()
    from fp4_precision_gemms_amd import calib
    L = calib.lib()
    grid, iters = 2, 3
    rng = np.random.default_rng(0)
    src = rng.integers(0, 256, L.fp4_calib_mfma_src_bytes(grid), dtype=np.uint8)
    dsrc = torch.from_numpy(src).cuda()
    out = torch.full((grid * 256,), float("nan"), dtype=torch.float32, device="cuda")
    clocks = torch.zeros((grid * 4, 2), dtype=torch.int64, device="cuda")
    assert L.fp4_calib_mfma(dsrc.data_ptr(), grid, iters, out.data_ptr(), clocks.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(grid * 4, 64)
    lanes = np.arange(64)
    for wave in range(grid * 4):
        acc = np.zeros((64,))
        for i in range(FM):
            for j in range(FN):
                c = np.zeros((32, 32))
                for s in range(NSET):
                    a = operand(src, wave, s * (FM + FN) + i)
                    b = operand(src, wave, s * (FM + FN) + FM + j)
                    c += a @ b.T                                  # C[m, n] = sum_k a[m,k] b[n,k]
                c *= iters
                for r in range(16):
                    n = 8 * (r // 4) + 4 * (lanes // 32) + r % 4
                    acc += c[lanes % 32, n]
        np.testing.assert_allclose(got[wave], acc, rtol=1e-6, atol=1e-3)
    ck = clocks.cpu().numpy()
    assert (ck > 0).all()
