"""Pins of the oracle's MXFP4 quantizer: hand-worked single blocks, lossless
round trips, the per-element error bound, the layout identity between the
two axes, non-finite blocks and the unbiasedness of stochastic rounding.
CPU only."""
import numpy as np
import pytest
import torch

import oracle as O


def bf16(values) -> np.ndarray:
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def q1(block, had=O.HAD_NONE, had_n=32):
    codes, scales = O.quant_mx(bf16([block]), axis=O.AXIS_COLS, had_n=had_n, had=had)
    return scales[0, 0], bytes(codes[0])


# Hand-worked blocks.  Each expected value is derived in the comment from the
# definitions alone: scale e = floor(log2 amax) - 2 (byte e + 127), v = y / 2^e,
# nearest E2M1 with ties to the even code, |v| > 6 -> 6, low nibble first.
E1 = [.25, .75, 1.25, 1.75, 2.5, 3.5, 5, 7, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, -7,
      .5, 1, 1.5, 2, 3, 4, 6, 0, .125, .375, 2.875, 4.875, 5.125, -6.5, .625, 1.375]


def test_e1_every_midpoint_and_saturation():
    # amax 7 -> floor(log2 7) = 2 -> e = 0, byte 0x7F; v = y.
    # midpoints .25->0, .75->1(code 2), 1.25->1(2), 1.75->2(4), 2.5->2(4), 3.5->4(6), 5->4(6);
    # 7 saturates to 6 (7).  Grid points map to themselves; .125->0, .375->.5(1),
    # 2.875->3(5), 4.875->4(6), 5.125->6(7), -6.5->-6(F), .625->.5(1), 1.375->1.5(3).
    s, c = q1(E1)
    assert s == 0x7F
    assert c == bytes.fromhex("20 42 64 76 A8 CA EC FE 21 43 65 07 10 65 F7 31")


def test_e2_scale_from_largest_exponent():
    # [8, 0...]: floor(log2 8) = 3 -> e = 1 (0x80); v = 4 -> code 6
    assert q1([8] + [0] * 31) == (0x80, bytes([0x06] + [0] * 15))
    # [0.75, 0...]: floor(log2 .75) = -1 -> e = -3 (0x7C); v = 6 -> code 7
    assert q1([0.75] + [0] * 31) == (0x7C, bytes([0x07] + [0] * 15))


def test_e3_zero_block():
    assert q1([0.0] * 32) == (0x00, bytes(16))
    # negative zeros keep their sign bit (code 8), scale still e = -127
    assert q1([-0.0] * 32) == (0x00, bytes([0x88] * 16))


def test_e4_subnormal_kept():
    # bf16 0x0040 = 2^-127 (subnormal): e = floor(-127) - 2 clamped to -127 (0x00),
    # v = 2^-127 * 2^127 = 1 -> code 2.  Flushing subnormals would give code 0.
    blk = np.zeros((1, 32), np.uint16)
    blk[0, 0] = 0x0040
    codes, scales = O.quant_mx(blk)
    assert scales[0, 0] == 0 and codes[0, 0] == 0x02 and not codes[0, 1:].any()


def test_e5_constant_block_hadamard():
    # H32 of all ones: y0 = 32 * fl(1/sqrt 32) = 5.6568..., others 0.
    # amax 5.657 -> e = 0 (0x7F); 5.657 > 5 -> 6 (code 7).
    assert q1([1.0] * 32, had=O.HAD_DET) == (0x7F, bytes([0x07] + [0] * 15))


def test_e6_one_hot_hadamard_columns():
    # one-hot at 0: y_i = fl(1/sqrt 32) = 0.17677... for all i; floor(log2) = -3 ->
    # e = -5 (0x7A); v = 5.657 -> code 7 everywhere.
    assert q1([1.0] + [0] * 31, had=O.HAD_DET) == (0x7A, bytes([0x77] * 16))
    # one-hot at 1: Sylvester column 1 alternates +,-: codes 7, F, 7, F ...
    assert q1([0, 1.0] + [0] * 30, had=O.HAD_DET) == (0x7A, bytes([0xF7] * 16))


def test_lossless_round_trip():
    """Blocks of E2M1 grid values times 2^k that contain a 4 or a 6 have
    e = k and quantize exactly; dequantization returns the input."""
    rng = np.random.default_rng(5)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    rows, cols = 8, 256
    v = rng.choice(grid, (rows, cols)) * rng.choice([-1, 1], (rows, cols))
    v = v.reshape(rows, cols // 32, 32)
    v[:, :, 0] = rng.choice([4, 6, -4, -6], (rows, cols // 32))
    v *= 2.0 ** rng.integers(-20, 20, (rows, cols // 32, 1))
    v = v.reshape(rows, cols)
    codes, scales = O.quant_mx(bf16(v))
    assert np.array_equal(O.dequant_mx(codes, scales), v)


@pytest.mark.parametrize("had,had_n", [(O.HAD_NONE, 32), (O.HAD_DET, 32), (O.HAD_SIGNED, 32),
                                       (O.HAD_DET, 16)])
def test_error_bound_and_layout(had, had_n):
    rng = np.random.default_rng(6)
    x = bf16(rng.standard_t(3, (64, 96)) * 0.01)
    codes, scales = O.quant_mx(x, axis=O.AXIS_COLS, had_n=had_n, had=had, sign_seed=9)
    # the rotated values, block by block, from the oracle's own transform
    xf = bf16_to_f32(x)
    s = O.hadamard_signs(had, had_n, 9) if had else None
    y = np.stack([np.concatenate([O.fwht(r[i:i + had_n], s) if had else r[i:i + had_n]
                                  for i in range(0, r.size, had_n)]) for r in xf])
    yhat = O.dequant_mx(codes, scales)
    e = scales.astype(np.int64) - 127
    step = np.repeat(2.0 ** e, 32, axis=1)
    assert (np.abs(y - yhat) < 2 * step).all()                 # saturation bound
    small = np.abs(y) <= 4 * step
    assert (np.abs(y - yhat)[small] <= 0.5 * step[small]).all()  # half the largest step
    # blocks along rows of x are blocks along cols of x^T
    ct, st = O.quant_mx(np.ascontiguousarray(x.T), axis=O.AXIS_ROWS, had_n=had_n, had=had,
                        sign_seed=9)
    assert np.array_equal(ct, codes) and np.array_equal(st, scales)


def test_non_finite_block():
    v = np.ones((2, 64), np.float32)
    v[0, 3] = np.nan
    v[1, 40] = np.inf
    codes, scales = O.quant_mx(bf16(v))
    assert scales[0, 0] == 0xFF and not codes[0, :16].any()
    assert scales[1, 1] == 0xFF and not codes[1, 16:].any()
    assert scales[0, 1] == 0x7D and scales[1, 0] == 0x7D          # 1.0 -> e = -2
    # overflow inside the transform poisons the block the same way
    big = np.full((1, 32), 3.0e38, np.float32)
    codes, scales = O.quant_mx(bf16(big), had=O.HAD_DET)
    assert scales[0, 0] == 0xFF


def test_rows_subrange_matches_full():
    rng = np.random.default_rng(8)
    x = bf16(rng.standard_normal((96, 64)))
    full = O.quant_mx(x, axis=O.AXIS_ROWS, had=O.HAD_DET)
    part = O.quant_mx(x, axis=O.AXIS_ROWS, had=O.HAD_DET, r0=10, r1=30)
    assert np.array_equal(part[0], full[0][10:30]) and np.array_equal(part[1], full[1][10:30])


def test_sr_unbiased_and_seeded():
    """E[dequant] over seeds equals the rotated value (blocks whose maximum
    is exactly 4 * 2^e do not saturate)."""
    rng = np.random.default_rng(10)
    v = rng.uniform(-4, 4, (1, 64)).astype(np.float32)
    v[0, 0], v[0, 32] = 4.0, -4.0
    x = bf16(v)
    xf = bf16_to_f32(x).astype(np.float64)
    n = 3000
    acc = np.zeros((1, 64))
    acc2 = np.zeros((1, 64))
    for seed in range(n):
        c, s = O.quant_mx(x, rnd=O.RND_SR, sr_seed=seed)
        d = O.dequant_mx(c, s)
        acc += d
        acc2 += d * d
    mean = acc / n
    sd = np.sqrt(np.maximum(acc2 / n - mean ** 2, 1e-30) / n)
    assert (np.abs(mean - xf) <= 4.5 * sd + 1e-9).all()
    a = O.quant_mx(x, rnd=O.RND_SR, sr_seed=77)
    b = O.quant_mx(x, rnd=O.RND_SR, sr_seed=77)
    c = O.quant_mx(x, rnd=O.RND_SR, sr_seed=78)
    assert np.array_equal(a[0], b[0]) and not np.array_equal(a[0], c[0])
    assert np.array_equal(a[1], c[1])                 # scales do not depend on the SR draw


def test_sr_index_is_logical_position():
    """The SR stream index is the element's position in the quantized
    logical layout, so quantizing x^T along rows draws the same numbers as
    quantizing x along columns."""
    rng = np.random.default_rng(12)
    x = bf16(rng.standard_normal((32, 64)))
    a = O.quant_mx(x, axis=O.AXIS_COLS, rnd=O.RND_SR, sr_seed=5)
    b = O.quant_mx(np.ascontiguousarray(x.T), axis=O.AXIS_ROWS, rnd=O.RND_SR, sr_seed=5)
    assert np.array_equal(a[0], b[0])


def test_bad_arguments_rejected():
    x = bf16(np.ones((4, 48)))
    with pytest.raises(ValueError):
        O.quant_mx(x)                                  # 48 is not a multiple of 32
    with pytest.raises(ValueError):
        O.quant_mx(bf16(np.ones((4, 64))), had=O.HAD_DET, had_n=8)
