"""Pins of the oracle's scaled FP4 GEMM and of the three GEMM roles of a
linear layer (Fprop Y = X W^T, Dgrad dX = dY W, Wgrad dW = dY^T X).
CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O


def bf16(values) -> np.ndarray:
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


E2M1 = [0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]


def _frac_value(codes, scales, r, k):
    byte = int(codes[r, k // 2])
    code = (byte >> 4) if k & 1 else (byte & 15)
    mag = E2M1[code & 7]
    return (-mag if code & 8 else mag) * Fraction(2) ** (int(scales[r, k // 32]) - 127)


@pytest.mark.parametrize("K", [32, 64])
def test_brute_force_fraction_4x4(K):
    rng = np.random.default_rng(K)
    aq = rng.integers(0, 256, (4, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, (4, K // 2), dtype=np.uint8)
    # scales within 2^15 of each other: every partial sum fits binary64 exactly
    as_ = rng.integers(120, 135, (4, K // 32), dtype=np.uint8)
    bs = rng.integers(120, 135, (4, K // 32), dtype=np.uint8)
    c, s = O.gemm_rows(aq, as_, bq, bs)
    for m in range(4):
        for n in range(4):
            exact = sum(_frac_value(aq, as_, m, k) * _frac_value(bq, bs, n, k) for k in range(K))
            mag = sum(abs(_frac_value(aq, as_, m, k) * _frac_value(bq, bs, n, k)) for k in range(K))
            assert Fraction(c[m, n]) == exact and Fraction(s[m, n]) == mag
    # wide scale ranges: binary64 accumulation within K ulps of the magnitude
    as_ = rng.integers(60, 200, (4, K // 32), dtype=np.uint8)
    c, s = O.gemm_rows(aq, as_, bq, bs)
    for m in range(4):
        for n in range(4):
            exact = sum(_frac_value(aq, as_, m, k) * _frac_value(bq, bs, n, k) for k in range(K))
            assert abs(Fraction(c[m, n]) - exact) <= Fraction(K, 2 ** 52) * Fraction(s[m, n])
    ce, se = O.gemm_entries(aq, as_, bq, bs, [0, 3, 2], [1, 3, 0])
    assert np.array_equal(ce, c[[0, 3, 2], [1, 3, 0]]) and np.array_equal(se, s[[0, 3, 2], [1, 3, 0]])


def _lossless(rng, rows, cols, axis):
    """bf16 values that MXFP4 represents exactly when blocked along `axis`:
    E2M1 grid values times a per-block power of two, with a 4 or 6 in every
    block so that the shared exponent is that power."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    v = rng.choice(grid, (rows, cols)) * rng.choice([-1, 1], (rows, cols))
    t = v if axis == O.AXIS_COLS else v.T
    R, C = t.shape
    t = t.reshape(R, C // 32, 32).copy()
    t[:, :, 0] = rng.choice([4, 6, -6], (R, C // 32))
    t *= 2.0 ** rng.integers(-6, 6, (R, C // 32, 1))
    t = t.reshape(R, C)
    return t if axis == O.AXIS_COLS else np.ascontiguousarray(t.T)


def test_three_gemm_roles_exact_on_lossless_inputs():
    """With operands MXFP4 represents exactly, each GEMM equals the plain
    matrix product the page defines."""
    rng = np.random.default_rng(1)
    T, K, N = 64, 96, 32
    # Fprop: X blocked along K (cols), W blocked along K (cols)
    X = _lossless(rng, T, K, O.AXIS_COLS)
    W = _lossless(rng, N, K, O.AXIS_COLS)
    xq = O.quant_mx(bf16(X), axis=O.AXIS_COLS)
    wq = O.quant_mx(bf16(W), axis=O.AXIS_COLS)
    y, _ = O.gemm_rows(*xq, *wq)
    assert np.array_equal(y, X @ W.T)
    # Dgrad: dY blocked along N (cols), W blocked along N (rows of W)
    dY = _lossless(rng, T, N, O.AXIS_COLS)
    W2 = _lossless(rng, N, K, O.AXIS_ROWS)
    dyq = O.quant_mx(bf16(dY), axis=O.AXIS_COLS)
    wtq = O.quant_mx(bf16(W2), axis=O.AXIS_ROWS)
    dx, _ = O.gemm_rows(*dyq, *wtq)
    assert np.array_equal(dx, dY @ W2)
    # Wgrad: dY and X both blocked along T (rows)
    dY3 = _lossless(rng, T, N, O.AXIS_ROWS)
    X3 = _lossless(rng, T, K, O.AXIS_ROWS)
    dytq = O.quant_mx(bf16(dY3), axis=O.AXIS_ROWS)
    xtq = O.quant_mx(bf16(X3), axis=O.AXIS_ROWS)
    dw, _ = O.gemm_rows(*dytq, *xtq)
    assert np.array_equal(dw, dY3.T @ X3)


@pytest.mark.parametrize("had,seed", [(O.HAD_DET, 0), (O.HAD_SIGNED, 3)])
def test_rotated_wgrad_approximates_product(had, seed):
    """The rotation along tokens cancels in dY^T X: the quantized rotated
    Wgrad stays within the quantization error of the exact product, while a
    rotation of one operand only does not."""
    rng = np.random.default_rng(2)
    T, K, N = 512, 64, 48
    X = bf16(rng.standard_normal((T, K)))
    dY = bf16(rng.standard_normal((T, N)) * 1e-3)
    ref = f32(dY).astype(np.float64).T @ f32(X).astype(np.float64)
    mag = np.abs(f32(dY)).astype(np.float64).T @ np.abs(f32(X)).astype(np.float64)
    dytq = O.quant_mx(dY, axis=O.AXIS_ROWS, had=had, sign_seed=seed)
    xtq = O.quant_mx(X, axis=O.AXIS_ROWS, had=had, sign_seed=seed)
    dw, _ = O.gemm_rows(*dytq, *xtq)
    err = np.abs(dw - ref) / mag
    assert np.median(err) < 0.05 and err.max() < 0.5
    xt_plain = O.quant_mx(X, axis=O.AXIS_ROWS)
    bad, _ = O.gemm_rows(*dytq, *xt_plain)
    assert np.median(np.abs(bad - ref) / mag) > 5 * np.median(err)


def test_fp32_accumulation_meets_tolerance():
    """|err| <= 1e-5 * sum|a b| is reachable by binary32 accumulation at the
    longest contraction used (8192): a sequential float32 sum of the exact
    products of random MXFP4 operands stays inside it."""
    rng = np.random.default_rng(3)
    K = 8192
    aq = rng.integers(0, 256, (2, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, (3, K // 2), dtype=np.uint8)
    as_ = rng.integers(120, 135, (2, K // 32), dtype=np.uint8)
    bs = rng.integers(120, 135, (3, K // 32), dtype=np.uint8)
    c, s = O.gemm_rows(aq, as_, bq, bs)
    A, B = O.dequant_mx(aq, as_), O.dequant_mx(bq, bs)
    for m in range(2):
        for n in range(3):
            prods = (A[m] * B[n]).astype(np.float32)       # exact: few significant bits
            acc = np.float32(0)
            for p in prods:
                acc = np.float32(acc + p)
            assert abs(float(acc) - c[m, n]) <= 1e-5 * s[m, n]


def test_nan_scale_propagates():
    aq = np.full((1, 16), 0x22, np.uint8)
    bq = np.full((2, 16), 0x22, np.uint8)
    as_ = np.array([[0xFF]], np.uint8)
    bs = np.array([[127], [127]], np.uint8)
    c, _ = O.gemm_rows(aq, as_, bq, bs)
    assert np.isnan(c).all()


def test_row_and_entry_ranges_checked():
    """Rows or entries outside the product are refused before the C code
    runs (it would read past the operands)."""
    rng = np.random.default_rng(0)
    aq = rng.integers(0, 256, (4, 16), dtype=np.uint8)
    as_ = np.full((4, 1), 127, dtype=np.uint8)
    for m0, m1 in ((0, 5), (-1, 2), (3, 2)):
        with pytest.raises(ValueError):
            O.gemm_rows(aq, as_, aq, as_, m0, m1)
    for mi, ni in (([4], [0]), ([0], [-1]), ([0, 1], [0])):
        with pytest.raises(ValueError):
            O.gemm_entries(aq, as_, aq, as_, np.array(mi), np.array(ni))
    c, s = O.gemm_rows(aq, as_, aq, as_, 4, 4)
    assert c.shape == (0, 4)
