"""fp4_wgrad_quantize (the Wgrad operand pair in one launch) is byte-for-byte
the two fp4_hadamard_quantize calls it stands for (those are checked against
the oracle in test_gpu_quant_mx.py), including the fallback to two launches
when a column count is not a multiple of 8; directly against the oracle on
one case."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
from _util import bf16_bits, need_gpu, say, sentinel_u8, to_gpu_bf16, ungroup_scales, untile_codes

pytestmark = pytest.mark.gpu

SHAPES = [(64, 256, 128), (96, 544, 1032), (544, 1056, 40), (32, 8, 16), (64, 36, 300)]
MODES = [(32, F.HAD_DET, F.RTN), (16, F.HAD_SIGNED, F.SR), (32, F.HAD_NONE, F.SR), (32, F.HAD_SIGNED, F.RTN)]


def single(x, hn, had, seed, rnd, sr):
    rows, cols = x.shape
    cs, ss = F.mx_shapes(rows, cols, F.AXIS_ROWS)
    codes, scales = sentinel_u8(cs), sentinel_u8(ss)
    F.fp4_hadamard_quantize(x, F.AXIS_ROWS, hn, had, seed, rnd, sr, codes, scales)
    return codes, scales


@pytest.mark.parametrize("T,N,K", SHAPES)
@pytest.mark.parametrize("mode", range(len(MODES)))
def test_pair_equals_two_calls(T, N, K, mode):
    need_gpu()
    hn, had, rnd = MODES[mode]
    rng = np.random.default_rng(T + N + K + mode)
    dy = to_gpu_bf16(bf16_bits(rng.standard_t(3, (T, N)) * 1e-3))
    x = to_gpu_bf16(bf16_bits(rng.standard_normal((T, K))))
    say("wgrad quantize pair", T, N, K, "mode", mode)
    out = tuple(sentinel_u8(sh) for sh in (*F.mx_shapes(T, N, F.AXIS_ROWS), *F.mx_shapes(T, K, F.AXIS_ROWS)))
    F.fp4_wgrad_quantize(dy, x, hn, had, 99, rnd, 5, 6, out=out)
    ref_dy = single(dy, hn, had, 99, rnd, 5)
    ref_x = single(x, hn, had, 99, rnd, 6)
    torch.cuda.synchronize()
    assert torch.equal(out[0], ref_dy[0]) and torch.equal(out[2], ref_x[0])
    nb = T // 32
    assert np.array_equal(ungroup_scales(out[1].cpu().numpy(), nb), ungroup_scales(ref_dy[1].cpu().numpy(), nb))
    assert np.array_equal(ungroup_scales(out[3].cpu().numpy(), nb), ungroup_scales(ref_x[1].cpu().numpy(), nb))


def test_pair_matches_oracle():
    need_gpu()
    T, N, K = 96, 544, 128
    rng = np.random.default_rng(3)
    dyb, xb = bf16_bits(rng.standard_normal((T, N)) * 1e-4), bf16_bits(rng.standard_normal((T, K)))
    say("wgrad quantize pair vs oracle")
    got = F.fp4_wgrad_quantize(to_gpu_bf16(dyb), to_gpu_bf16(xb), 32, F.HAD_SIGNED, 7, F.SR, 8, 9)
    torch.cuda.synchronize()
    for (c, s), bits, sr in (((got[0], got[1]), dyb, 8), ((got[2], got[3]), xb, 9)):
        want = O.quant_mx(bits, O.AXIS_ROWS, 32, O.HAD_SIGNED, 7, O.RND_SR, sr)
        assert np.array_equal(untile_codes(c.cpu().numpy(), bits.shape[1]), want[0])
        assert np.array_equal(ungroup_scales(s.cpu().numpy(), T // 32), want[1])
