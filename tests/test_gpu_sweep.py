"""A seeded sweep of random shapes and modes through the C ABI, each case
checked against the oracle: MXFP4 quantization along either axis (codes and
scales bit-exact) for every rotation, size and rounding, then the scaled FP4
GEMM of the quantized pair (|err| <= 1e-5 sum|a b|).  The row counts are
arbitrary for blocks along columns and multiples of 32 along rows; the
contraction sizes are multiples of 32 with and without a partial 256-wide
stage."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
from _util import bf16_bits, gemm_check, group_scales, need_gpu, say, tile_codes, to_gpu_u8
from test_gpu_quant_mx import AX, HD, RN, gpu_quant

pytestmark = pytest.mark.gpu

MODES = [(O.HAD_NONE, 32), (O.HAD_DET, 32), (O.HAD_SIGNED, 32), (O.HAD_DET, 16), (O.HAD_SIGNED, 16)]


def case(seed):
    rng = np.random.default_rng(1000 + seed)
    axis = [O.AXIS_COLS, O.AXIS_ROWS][seed % 2]
    had, had_n = MODES[rng.integers(0, len(MODES))]
    rnd = [O.RND_RTN, O.RND_SR][int(rng.integers(0, 2))]
    kc = 32 * int(rng.integers(1, 40))                   # contraction length
    m = int(rng.integers(1, 300))                        # quantized rows of operand A
    n = int(rng.integers(1, 300))                        # of operand B
    if axis == O.AXIS_ROWS:
        shape_a, shape_b = (kc, m), (kc, n)              # x[rows = contraction, cols]
    else:
        shape_a, shape_b = (m, kc), (n, kc)
    scale = 10.0 ** rng.uniform(-6, 2)
    a = bf16_bits(rng.standard_t(3, shape_a) * scale)
    b = bf16_bits(rng.standard_normal(shape_b) * scale)
    return axis, had, had_n, rnd, a, b, int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 63))


@pytest.mark.parametrize("seed", range(24))
def test_sweep_quantize_then_gemm(seed):
    need_gpu()
    axis, had, had_n, rnd, a, b, sseed, rseed = case(seed)
    say("sweep", seed, "axis", axis, "had", had, had_n, "rnd", rnd, a.shape, b.shape)
    got_a = gpu_quant(a, axis, had, had_n, rnd, sseed, rseed)
    got_b = gpu_quant(b, axis, had, had_n, rnd, sseed, rseed + 1)
    ref_a = O.quant_mx(a, axis, had_n, had, sseed, rnd, rseed)
    ref_b = O.quant_mx(b, axis, had_n, had, sseed, rnd, rseed + 1)
    for got, ref, name in ((got_a, ref_a, "A"), (got_b, ref_b, "B")):
        assert np.array_equal(got[0], ref[0]), "%s codes differ" % name
        assert np.array_equal(got[1], ref[1]), "%s scales differ" % name
    # the scaled product of the two quantized operands: C = A B^T
    aq, as_ = ref_a
    bq, bs = ref_b
    g = [to_gpu_u8(t) for t in (tile_codes(aq, 0xCD), group_scales(as_), tile_codes(bq, 0xCD), group_scales(bs))]
    out = torch.full((aq.shape[0], bq.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    F.fp4_gemm_mx(*g, out=out)
    torch.cuda.synchronize()
    c, mag = O.gemm_rows(aq, as_, bq, bs)
    gemm_check(out.cpu().numpy(), c, mag, 1e-5)
