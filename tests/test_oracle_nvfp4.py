"""Pins of the oracle's NVFP4 quantizer (16-element blocks, E4M3 block scales,
fp32 tensor scale, renormalization folded into the block scales by
stochastic rounding, or stochastic rounding of every element).  CPU only.

The exact renormalization rule is a reading of the Quartet II post (which
gives the idea and the 0.94..1.06 range but no formula); its bits are
"parity unpinned" against that paper.  What is pinned here: the rotation and
tensor amax against scipy, the scale arithmetic by invariants, the
stochastic rounding of the scales by unbiasedness against an independent
binary64 computation of the renormalized scale, and the factor's range; the
element-SR mode by its neighbours and unbiasedness; and the two properties
the Quartet II post claims for the renormalized mode: averaged over random
rotations it is unbiased where round-to-nearest shrinks, and its total error
is about half that of element SR."""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O


def bf16(values) -> np.ndarray:
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def rotated64(x, had, seed):
    """Row-wise 16-block transform in binary64 via scipy's Hadamard matrix."""
    xf = f32(x).astype(np.float64)
    if had == O.HAD_NONE:
        return xf
    s = O.hadamard_signs(had, 16, seed).astype(np.float64)
    H = scipy.linalg.hadamard(16) * 0.25
    r, c = xf.shape
    return ((xf.reshape(r, c // 16, 16) * s) @ H.T).reshape(r, c)


def dequant(codes, scales, st):
    lo, hi = codes & 15, codes >> 4
    q = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    val = np.array([O.e2m1_decode(c) for c in range(16)])[q]
    sc = np.array([O.e4m3_decode(b) for b in range(256)])[scales]
    return val * np.repeat(sc, 16, axis=1) * float(st)


@pytest.fixture(scope="module")
def tdata():
    rng = np.random.default_rng(0)
    return bf16(rng.standard_t(4, (64, 256)))


@pytest.mark.parametrize("had", [O.HAD_NONE, O.HAD_SIGNED, O.HAD_DET])
def test_amax_and_tensor_scale(tdata, had):
    y = rotated64(tdata, had, 5)
    amax = O.nvfp4_amax(tdata, had, 5)
    assert abs(float(amax) - np.abs(y).max()) <= 1e-6 * np.abs(y).max()
    _, _, st = O.nvfp4_quantize(tdata, had=had, sign_seed=5, mode=O.NV_RTN)
    assert st == np.float32(amax) / np.float32(2688.0)          # 6 * 448
    _, _, st2 = O.nvfp4_quantize(tdata, had=had, sign_seed=5, mode=O.NV_RTN, amax_in=10.0)
    assert st2 == np.float32(10.0) / np.float32(2688.0)


def test_block_scale_maps_block_max_near_6(tdata):
    codes, scales, st = O.nvfp4_quantize(tdata, had=O.HAD_SIGNED, sign_seed=5, mode=O.NV_RTN)
    y = rotated64(tdata, O.HAD_SIGNED, 5)
    sb = np.array([O.e4m3_decode(b) for b in range(256)])[scales]
    mb = np.abs(y).reshape(y.shape[0], -1, 16).max(axis=2)
    ratio = mb / (sb * float(st))
    assert (ratio > 6 * 16 / 17 * (1 - 1e-6)).all() and (ratio < 6 * 16 / 15 * (1 + 1e-6)).all()
    # per-element error: half a grid step of the block, or the saturation excess
    yhat = dequant(codes, scales, st)
    unit = np.repeat(sb * float(st), 16, axis=1)
    v = np.abs(y) / unit
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    assert (np.abs(y - yhat) <= (half_step + np.maximum(v - 6, 0)) * unit * (1 + 1e-6)).all()


def test_renorm_changes_only_scales_and_is_unbiased(tdata):
    x = tdata[:4]
    c0, s0, st = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=5, mode=O.NV_RTN)
    y = rotated64(x, O.HAD_SIGNED, 5)
    sb = np.array([O.e4m3_decode(b) for b in range(256)])[s0]
    # renormalized scale in binary64: s_b * |y|^2 / <y, y_hat>
    yhat = dequant(c0, s0, st)
    yb, hb = y.reshape(4, -1, 16), yhat.reshape(4, -1, 16)
    target = sb * (yb * yb).sum(2) / (yb * hb).sum(2)
    n = 4000
    acc = np.zeros_like(target)
    acc2 = np.zeros_like(target)
    for seed in range(n):
        c1, s1, st1 = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=5, mode=O.NV_RENORM_SR, sr_seed=seed)
        assert st1 == st and np.array_equal(c1, c0)
        d = np.array([O.e4m3_decode(b) for b in range(256)])[s1]
        acc += d
        acc2 += d * d
    mean = acc / n
    sd = np.sqrt(np.maximum(acc2 / n - mean ** 2, 0) / n)
    ok = target < 448                   # above 448 the scale saturates by design
    assert ok.mean() > 0.9
    assert (np.abs(mean - target) <= 4.5 * sd + 1e-5 * target)[ok].all()
    assert (mean[~ok] == 448).all()


def test_renorm_factor_range():
    """The Quartet II post puts the renormalization factor at about
    0.94..1.06 for rotated tensors; check that the bulk lies there."""
    rng = np.random.default_rng(1)
    x = bf16(rng.standard_t(4, (128, 1024)))
    c0, s0, st = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=7, mode=O.NV_RTN)
    y = rotated64(x, O.HAD_SIGNED, 7).reshape(128, -1, 16)
    yhat = dequant(c0, s0, st).reshape(128, -1, 16)
    rho = (y * y).sum(2) / (y * yhat).sum(2)
    inside = ((rho > 0.94) & (rho < 1.06)).mean()
    assert inside > 0.9 and 0.97 < np.median(rho) < 1.03


def test_zero_tensor_and_bad_args():
    z = np.zeros((2, 32), np.uint16)
    c, s, st = O.nvfp4_quantize(z)
    assert st == 1.0 and not c.any() and not s.any()
    with pytest.raises(ValueError):
        O.nvfp4_quantize(np.zeros((2, 24), np.uint16))


E4 = np.array([O.e4m3_decode(b) for b in range(256)])


def test_element_sr_neighbours_and_scales(tdata):
    """Element SR keeps mode 0's scales and tensor scale; every code is one
    of the two E2M1 neighbours of v = y / (s_b s_t) (6 when |v| >= 6)."""
    x = tdata[:8]
    c0, s0, st = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=5, mode=O.NV_RTN)
    c2, s2, st2 = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=5, mode=O.NV_ELEMENT_SR, sr_seed=3)
    assert st2 == st and np.array_equal(s2, s0)
    assert not np.array_equal(c2, c0)
    y = rotated64(x, O.HAD_SIGNED, 5)
    unit = np.repeat(E4[s0] * float(st), 16, axis=1)
    v = np.abs(y) / unit
    got = np.abs(dequant(c2, s2, st2)) / unit
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    lo = grid[np.clip(np.searchsorted(grid, v, side="right") - 1, 0, 7)]
    hi = grid[np.clip(np.searchsorted(grid, v, side="right"), 0, 7)]
    ok = (np.abs(got - lo) < 1e-9) | (np.abs(got - hi) < 1e-9)
    assert ok[(v < 6 * (1 - 1e-6)) & (unit > 0)].all()
    assert (np.abs(got[v >= 6 * (1 + 1e-6)] - 6) < 1e-9).all()


def test_element_sr_unbiased(tdata):
    """Mean over SR seeds of each dequantized element equals y (binary64,
    independent rotation) where nothing saturates, within 4.5 standard
    errors of the two-point distribution between the element's grid
    neighbours (plus one grid step / n, the resolution of a mean of n
    samples)."""
    x = tdata[:4, :64]
    c0, s0, st = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=5, mode=O.NV_RTN)
    y = rotated64(x, O.HAD_SIGNED, 5)
    n = 3000
    acc = np.zeros_like(y)
    for seed in range(n):
        c, s, _ = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=5, mode=O.NV_ELEMENT_SR, sr_seed=seed)
        acc += dequant(c, s, st)
    mean = acc / n
    unit = np.repeat(E4[s0] * float(st), 16, axis=1)
    v = np.abs(y) / unit
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    k = np.clip(np.searchsorted(grid, v, side="right") - 1, 0, 6)
    step = grid[k + 1] - grid[k]
    p = np.clip((v - grid[k]) / step, 0, 1)
    se = step * unit * np.sqrt(p * (1 - p) / n)
    inside = v < 6 * (1 - 1e-6)
    assert inside.mean() > 0.9
    assert (np.abs(mean - y) <= 4.5 * se + step * unit / n + 1e-6 * np.abs(y))[inside].all()


def _derotated_mean_coefficient(x, mode, n):
    """<E[D H^T q(H D x)], x> / <x, x>, the expectation taken over n sign
    seeds (each with its own SR seed), in binary64."""
    H = scipy.linalg.hadamard(16) * 0.25
    xf = f32(x).astype(np.float64)
    r, c = xf.shape
    coef = []
    for seed in range(n):
        s = O.hadamard_signs(O.HAD_SIGNED, 16, seed).astype(np.float64)
        cq, sq, st = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=seed, mode=mode, sr_seed=1000 + seed)
        back = ((dequant(cq, sq, st).reshape(r, -1, 16) @ H) * s).reshape(r, c)
        coef.append((back * xf).sum() / (xf * xf).sum())
    return float(np.mean(coef))


def test_renormalized_mode_unbiased_over_rotations():
    """[QUARTET-II]: quantizing a randomly rotated tensor gives, in
    expectation, a result collinear with the original, and the per-block
    renormalization makes it unbiased.  Averaged over 1000 random-sign
    rotations, round-to-nearest shrinks the tensor by about 0.5 %
    (coefficient 0.995, standard error 1e-4); the renormalized mode's
    coefficient is within a third of that distance of 1."""
    rng = np.random.default_rng(2)
    x = bf16(rng.standard_t(4, (8, 256)))
    c_rtn = _derotated_mean_coefficient(x, O.NV_RTN, 1000)
    c_ren = _derotated_mean_coefficient(x, O.NV_RENORM_SR, 1000)
    assert c_rtn < 0.997
    assert abs(1 - c_ren) < 0.35 * abs(1 - c_rtn)


def test_total_error_half_of_element_sr():
    """[QUARTET-II]: with SR only in the FP8 scales the total error comes out
    about half that of plain (element) SR.  Mean squared error against the
    rotated tensor over 50 SR seeds on Student-t data: the ratio is 1.99
    here (accepted: 1.6 .. 2.4).  The post's other figure, a hundredfold
    smaller error from the scale SR itself, depends on what is compared and
    is not pinned (measured: the scale SR's own noise is about 1/15 of the
    element SR error)."""
    rng = np.random.default_rng(1)
    x = bf16(rng.standard_t(4, (64, 512)))
    y = rotated64(x, O.HAD_SIGNED, 7)
    _, _, st = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=7, mode=O.NV_RTN)
    me = mr = 0.0
    for seed in range(50):
        ce, se, _ = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=7, mode=O.NV_ELEMENT_SR, sr_seed=seed)
        cr, sr, _ = O.nvfp4_quantize(x, had=O.HAD_SIGNED, sign_seed=7, mode=O.NV_RENORM_SR, sr_seed=seed)
        me += np.mean((dequant(ce, se, st) - y) ** 2)
        mr += np.mean((dequant(cr, sr, st) - y) ** 2)
    assert 1.6 < me / mr < 2.4


# --- non-finite and extreme inputs (a reading: the pages are silent) --------

NAN_BITS = 0x7FC00000
MODES = [O.NV_RTN, O.NV_RENORM_SR, O.NV_ELEMENT_SR]


def _nan_tensor(c, s, st):
    return (np.float32(st).view(np.uint32) == NAN_BITS and not c.any() and (s == 0x7F).all())


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("had", [O.HAD_NONE, O.HAD_SIGNED])
@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_element_makes_computed_amax_tensor_nan(mode, had, bad):
    """A NaN or an infinity anywhere gives a non-finite tensor amax: the
    whole tensor is NaN (tensor scale NaN, every scale byte 0x7F, codes 0)."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((8, 64)).astype(np.float32)
    v[5, 17] = bad
    x = bf16(v)
    amax = O.nvfp4_amax(x, had, 2)
    assert np.isnan(amax) if np.isnan(bad) else np.isinf(amax)
    assert _nan_tensor(*O.nvfp4_quantize(x, had, 2, mode, 9))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("amax", [np.nan, np.inf, -1.0, -0.5e-30, 1e-45])
def test_invalid_amax_in_makes_tensor_nan(mode, amax):
    """A supplied amax without a finite positive tensor scale (NaN, infinite,
    negative, or so small that amax / 2688 is zero in binary32)."""
    x = bf16(np.random.default_rng(4).standard_normal((4, 32)))
    assert np.float32(np.float32(1e-45) / np.float32(2688.0)) == 0.0
    assert _nan_tensor(*O.nvfp4_quantize(x, O.HAD_SIGNED, 1, mode, 2, amax_in=amax))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("had", [O.HAD_NONE, O.HAD_DET, O.HAD_SIGNED])
def test_nonfinite_block_with_supplied_amax(mode, had):
    """With the amax supplied the blocks are independent: a block holding a
    NaN, an infinity, or values whose rotation overflows gets scale 0x7F and
    zero codes, and every other block is exactly what the same tensor with
    finite values in those blocks gives."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((6, 64)).astype(np.float32)
    bad = v.copy()
    bad[0, 3] = np.nan                    # block (0, 0)
    bad[2, 40] = -np.inf                  # block (2, 2)
    bad[4, 48:64] = 3.0e38                # block (4, 3): finite, but 16 * 3e38 overflows
    x_bad, x_ok = bf16(bad), bf16(v)
    cb, sb, tb = O.nvfp4_quantize(x_bad, had, 7, mode, 3, amax_in=5.0)
    co, so, to = O.nvfp4_quantize(x_ok, had, 7, mode, 3, amax_in=5.0)
    assert tb == to == np.float32(5.0) / np.float32(2688.0)
    bad_blocks = [(0, 0), (2, 2)] + ([(4, 3)] if had != O.HAD_NONE else [])
    keep = np.ones(sb.shape, bool)
    for r, b in bad_blocks:
        assert sb[r, b] == 0x7F and not cb[r, 8 * b:8 * b + 8].any(), (r, b)
        keep[r, b] = False
    if had == O.HAD_NONE:        # 3e38 is finite and unrotated: a saturated scale
        keep[4, 3] = False
        assert sb[4, 3] == 0x7E
    assert np.array_equal(sb[keep], so[keep])
    kc = np.repeat(keep, 8, axis=1)
    assert np.array_equal(cb[kc], co[kc])


@pytest.mark.parametrize("mode", MODES)
def test_reciprocal_scale_overflow_gives_zero_codes(mode):
    """A tensor with amax near 2^-127: for blocks whose s_b s_t is below
    about 2^-128, fl(1 / fl(s_b s_t)) is infinite in binary32 (recomputed
    here with numpy and torch's E4M3 cast); those blocks get zero codes and
    scale s_b, the others are ordinary (some nonzero code)."""
    rng = np.random.default_rng(6)
    v = (rng.uniform(0.5, 1.0, (4, 64)) * 2.0 ** -127).astype(np.float32)
    v[3] *= 2.0 ** 8                       # row 3: normal values, amax 2^-119 .. 2^-120
    x = bf16(v)
    y = f32(x)
    c, s, st = O.nvfp4_quantize(x, O.HAD_NONE, 0, mode, 5)
    A = np.float32(np.abs(y).max())
    assert st == A / np.float32(2688.0)
    hits = [0, 0]
    for r in range(4):
        for b in range(4):
            m = np.float32(np.abs(y[r, 16 * b:16 * b + 16]).max())
            sbv = torch.tensor([float(m / (np.float32(6.0) * st))]).to(torch.float8_e4m3fn).float().item()
            code = int(torch.tensor([sbv]).to(torch.float8_e4m3fn).view(torch.uint8).item())
            with np.errstate(over="ignore", divide="ignore"):
                inv = np.float32(1.0) / (np.float32(sbv) * st)
            if mode != O.NV_RENORM_SR:
                assert s[r, b] == code, (r, b)
            hits[int(np.isinf(inv))] += 1
            if np.isinf(inv):
                assert not c[r, 8 * b:8 * b + 8].any() and s[r, b] == code, (r, b)
            else:
                assert c[r, 8 * b:8 * b + 8].any(), (r, b)
    assert hits[0] > 0 and hits[1] > 0        # both kinds of block occur


def test_renorm_target_nan_keeps_block_scale():
    """Values near the binary32 limit: sum y^2 and sum y q both overflow to
    infinity, so the renormalized target is Inf / Inf; the block keeps its
    round-to-nearest scale (mode 0's byte), the other blocks still move."""
    rng = np.random.default_rng(8)
    v = rng.standard_normal((2, 32)).astype(np.float32) * np.float32(1e37)
    v[0, :16] = 3.0e38
    x = bf16(v)
    c0, s0, t0 = O.nvfp4_quantize(x, O.HAD_NONE, 0, O.NV_RTN, 1)
    c1, s1, t1 = O.nvfp4_quantize(x, O.HAD_NONE, 0, O.NV_RENORM_SR, 1)
    y = f32(x)[0, :16]
    with np.errstate(over="ignore", invalid="ignore"):
        num = np.float32(0)
        for t in y:
            num = np.float32(num + np.float32(t) * np.float32(t))
    assert np.isinf(num)
    assert s1[0, 0] == s0[0, 0] and t1 == t0
    assert np.array_equal(c1, c0)
