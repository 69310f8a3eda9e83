"""Pins of the oracle's scalar formats (E2M1, E4M3, E8M0) against brute force
and against torch's own float8 types.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

# E2M1 magnitudes as the OCP MX element format defines them (1 sign bit,
# 2 exponent bits with bias 1, 1 mantissa bit; exponent 0 is subnormal).
def _e2m1_by_definition(code):
    e, m = (code >> 1) & 3, code & 1
    mag = (m * 0.5) if e == 0 else (1 + m * 0.5) * 2.0 ** (e - 1)
    return -mag if code & 8 else mag


GRID = np.array([_e2m1_by_definition(c) for c in range(8)])


def _nearest_even_brute(v):
    """Nearest of the 8 magnitudes to |v|, the even code on a tie; beyond 6
    the nearest is 6 (saturation)."""
    a = Fraction(abs(float(v)))
    d = [abs(Fraction(g) - a) for g in GRID]
    best = [i for i in range(8) if d[i] == min(d)]
    code = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return code | (8 if np.signbit(v) else 0)


def test_e2m1_grid_matches_definition():
    assert list(GRID) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for c in range(16):
        assert O.e2m1_decode(c) == _e2m1_by_definition(c)


def _nearest_even_vec(w):
    """Vectorized brute force: distances to the 8 magnitudes are exact in
    binary64 for |w| < 2^20 (few significant bits); larger |w| is nearest to 6."""
    a = np.abs(w.astype(np.float64))
    d = np.abs(GRID[None, :] - np.minimum(a, 2.0 ** 20)[:, None])
    dmin = d.min(axis=1, keepdims=True)
    tie = (d == dmin)
    # among the nearest, prefer the even code (codes are column indices)
    even_first = np.where(tie & (np.arange(8)[None, :] % 2 == 0), 0, np.where(tie, 1, 2))
    code = np.argmin(even_first * 16 + np.arange(8)[None, :], axis=1)
    return code | np.where(np.signbit(w), 8, 0)


def test_e2m1_rtn_brute_force_all_bf16_times_scales():
    bits = np.arange(65536, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    with np.errstate(over="ignore"):
        for sh in range(-3, 4):
            w = (vals * np.float32(2.0 ** sh)).astype(np.float32)
            w = w[np.isfinite(w)]
            ref = _nearest_even_vec(w)
            got = np.array([O.e2m1_rtn(v) for v in w])
            bad = np.flatnonzero(got != ref)
            assert bad.size == 0, (w[bad[:5]], got[bad[:5]], ref[bad[:5]])
    # the vectorized brute force agrees with the exact-rational one on a sample
    rng = np.random.default_rng(0)
    sample = rng.choice(vals, 3000)
    assert all(_nearest_even_vec(np.array([v]))[0] == _nearest_even_brute(v) for v in sample)


def test_e2m1_rtn_ties_and_edges():
    # each midpoint goes to the even code
    for mid, code in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]:
        assert O.e2m1_rtn(mid) == code
        assert O.e2m1_rtn(-mid) == code | 8
        up = np.nextafter(np.float32(mid), np.float32(10))
        assert O.e2m1_rtn(up) == _nearest_even_brute(up)
    assert O.e2m1_rtn(7.99) == 7 and O.e2m1_rtn(-1e30) == 15
    assert O.e2m1_rtn(-0.0) == 8 and O.e2m1_rtn(0.0) == 0


def test_e2m1_sr_neighbours_and_probability():
    rng = np.random.default_rng(1)
    for v in rng.uniform(-6, 6, 2000).astype(np.float32):
        a = abs(float(v))
        lo = GRID[GRID <= a].max()
        hi = GRID[GRID > a].min() if a < 6 else 6.0
        p = (a - lo) / (hi - lo) if hi > lo else 0.0
        # u = 0 rounds up iff p > 0, u = max never rounds up unless p > 1 - 2^-24
        for u, expect_up in [(0, p > 0), (0xFFFFFFFF, p > 1 - 2 ** -24)]:
            got = abs(O.e2m1_decode(O.e2m1_sr(v, u)))
            assert got == (hi if expect_up else lo)
        # threshold: (u >> 8) * 2^-24 < p
        t = int(np.ceil(p * 2 ** 24))
        if 0 < t < 2 ** 24:
            assert abs(O.e2m1_decode(O.e2m1_sr(v, (t - 1) << 8))) == hi
            assert abs(O.e2m1_decode(O.e2m1_sr(v, t << 8))) == lo
    assert O.e2m1_sr(6.5, 0) == 7 and O.e2m1_sr(-100.0, 12345) == 15


@pytest.mark.parametrize("v", [0.3, 1.1, 2.7, 5.5, -0.9, 3.3])
def test_e2m1_sr_unbiased(v):
    n = 100_000
    draws = np.array([O.e2m1_decode(O.e2m1_sr(np.float32(v), O.stream_word(7, 0, i)))
                      for i in range(n)])
    a = abs(v)
    lo, hi = GRID[GRID <= a].max(), GRID[GRID > a].min()
    p = (a - lo) / (hi - lo)
    sigma = (hi - lo) * np.sqrt(p * (1 - p) / n)
    assert abs(draws.mean() - np.float32(v)) < 4 * sigma + 1e-12


def test_e8m0_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).double().numpy()
    codes = np.full((1, 16), 0x22, dtype=np.uint8)           # two elements of value 1
    for s in range(256):
        scales = np.array([[s]], dtype=np.uint8)
        got = O.dequant_mx(codes, scales)[0, 0]
        if s == 255:
            assert np.isnan(got) and np.isnan(ref[s])
        else:
            assert got == ref[s] == 2.0 ** (s - 127)


def test_mx_exponent_is_floor_log2_minus_2():
    import math
    rng = np.random.default_rng(2)
    mags = np.concatenate([rng.uniform(0, 10, 500), 2.0 ** rng.uniform(-140, 127, 500),
                           [2.0 ** k for k in range(-149, 128)]]).astype(np.float32)
    for m in mags:
        if m == 0:
            continue
        fr, ex = math.frexp(float(m))
        e = min(max(ex - 1 - 2, -127), 127)
        assert O.mx_exponent(m) == e
        if e > -127:
            assert 4 <= float(m) / 2.0 ** e < 8     # block maximum lands in [4, 8)
    assert O.mx_exponent(0.0) == -127


def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).double().numpy()
    for i in range(256):
        got = O.e4m3_decode(i)
        if np.isnan(ref[i]):
            assert np.isnan(got)
        else:
            assert got == ref[i], i


def test_e4m3_rne_matches_torch_cast():
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16          # all non-negative finite bf16
    vals = bits.view(np.float32)
    rng = np.random.default_rng(3)
    extra = (2.0 ** rng.uniform(-14, 8.85, 20000)).astype(np.float32)
    vals = np.concatenate([vals, extra])
    vals = vals[vals < 464]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_rne(v) for v in vals], dtype=np.uint8)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], ref[bad[:5]])
    assert O.e4m3_rne(500.0) == 0x7E and O.e4m3_rne(1e30) == 0x7E


def test_e4m3_sr_neighbours_and_unbiased():
    rng = np.random.default_rng(4)
    for x in (2.0 ** rng.uniform(-12, 8.7, 300)).astype(np.float32):
        lo = O.e4m3_decode(O.e4m3_sr(x, 0xFFFFFFFF))
        hi = O.e4m3_decode(O.e4m3_sr(x, 0))
        assert lo <= x <= hi
        if lo != hi:
            assert O.e4m3_decode(O.e4m3_rne(x)) in (lo, hi)
    x = np.float32(1.03)   # between 1.0 and 1.125
    n = 100_000
    d = np.array([O.e4m3_decode(O.e4m3_sr(x, O.stream_word(9, 2, i))) for i in range(n)])
    p = (1.03 - 1.0) / 0.125
    assert abs(d.mean() - float(x)) < 4 * 0.125 * np.sqrt(p * (1 - p) / n)
    assert O.e4m3_sr(448.0, 0) == 0x7E and O.e4m3_sr(460.0, 0) == 0x7E
