"""GPU parity of fp4_hadamard_quantize_dual: its two outputs are byte-for-byte
the two single-axis quantizations (themselves checked against the oracle in
test_gpu_quant_mx.py), and match the oracle directly on small inputs.  The
scale padding of a partial last k-group is never written (sentinel kept)."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
from _util import bf16_bits, need_gpu, say, sentinel_u8, to_gpu_bf16, ungroup_scales, untile_codes

pytestmark = pytest.mark.gpu

SHAPES = [(64, 256), (96, 544), (1056, 288), (32, 32), (544, 1056)]
MODES = [  # (had_n, had, rnd) for the rows output, then for the cols output
    ((32, F.HAD_DET, F.RTN), (32, F.HAD_NONE, F.RTN)),
    ((16, F.HAD_SIGNED, F.SR), (32, F.HAD_DET, F.SR)),
    ((32, F.HAD_NONE, F.SR), (16, F.HAD_SIGNED, F.RTN)),
    ((32, F.HAD_SIGNED, F.RTN), (16, F.HAD_NONE, F.SR)),
]
O_HAD = {F.HAD_NONE: O.HAD_NONE, F.HAD_DET: O.HAD_DET, F.HAD_SIGNED: O.HAD_SIGNED}
O_RND = {F.RTN: O.RND_RTN, F.SR: O.RND_SR}


def single(x, axis, hn, had, rnd, sign_seed, sr_seed):
    rows, cols = x.shape
    cs, ss = F.mx_shapes(rows, cols, axis)
    codes, scales = sentinel_u8(cs), sentinel_u8(ss)
    F.fp4_hadamard_quantize(x, axis, hn, had, sign_seed, rnd, sr_seed, codes, scales)
    return codes, scales


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("mode", range(len(MODES)))
def test_dual_equals_two_single_calls(rows, cols, mode):
    need_gpu()
    (hr, ar, rr), (hc, ac, rc) = MODES[mode]
    rng = np.random.default_rng(rows + 3 * cols + mode)
    v = rng.standard_t(3, (rows, cols)) * np.exp(rng.uniform(-3, 3, (rows, 1)))
    x = to_gpu_bf16(bf16_bits(v))
    say("quant dual", rows, cols, "mode", mode)
    got = F.fp4_hadamard_quantize_dual(x, hr, ar, 11, rr, 21, hc, ac, 12, rc, 22)
    ref_r = single(x, F.AXIS_ROWS, hr, ar, rr, 11, 21)
    ref_c = single(x, F.AXIS_COLS, hc, ac, rc, 12, 22)
    torch.cuda.synchronize()
    nb_r, nb_c = rows // 32, cols // 32
    assert torch.equal(got[0], ref_r[0]), "rows codes"
    assert np.array_equal(ungroup_scales(got[1].cpu().numpy(), nb_r), ungroup_scales(ref_r[1].cpu().numpy(), nb_r))
    assert torch.equal(got[2], ref_c[0]), "cols codes"
    assert np.array_equal(ungroup_scales(got[3].cpu().numpy(), nb_c), ungroup_scales(ref_c[1].cpu().numpy(), nb_c))


@pytest.mark.parametrize("mode", [0, 1])
def test_dual_matches_oracle(mode):
    need_gpu()
    (hr, ar, rr), (hc, ac, rc) = MODES[mode]
    rows, cols = 96, 544
    rng = np.random.default_rng(40 + mode)
    bits = bf16_bits(rng.standard_normal((rows, cols)))
    say("quant dual vs oracle", mode)
    got = F.fp4_hadamard_quantize_dual(to_gpu_bf16(bits), hr, ar, 5, rr, 6, hc, ac, 7, rc, 8)
    torch.cuda.synchronize()
    want_r = O.quant_mx(bits, O.AXIS_ROWS, hr, O_HAD[ar], 5, O_RND[rr], 6)
    want_c = O.quant_mx(bits, O.AXIS_COLS, hc, O_HAD[ac], 7, O_RND[rc], 8)
    assert np.array_equal(untile_codes(got[0].cpu().numpy(), cols), want_r[0])
    assert np.array_equal(ungroup_scales(got[1].cpu().numpy(), rows // 32), want_r[1])
    assert np.array_equal(untile_codes(got[2].cpu().numpy(), rows), want_c[0])
    assert np.array_equal(ungroup_scales(got[3].cpu().numpy(), cols // 32), want_c[1])
