"""GPU parity of fp4_gemm_mx's output options against the oracle's binary64
product: bf16 output (the fp32 result rounded to nearest even) and
accumulation into an existing C (fp32 or bf16), on ragged shapes including
N % 4 != 0 (the element-wise store path).

Bounds.  The fp32 result r satisfies |r - ref| <= 1e-5 * S with S = sum |a b|
(the product's own bound), plus |c_old| in S when accumulating (one more
fp32 rounding, far below it).  Rounding r to bf16 moves it by at most half a
bf16 ulp, 2^-8 |r| <= 2^-8 (|ref| + 1e-5 S)."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
from _util import gemm_check, group_scales, need_gpu, say, tile_codes, to_gpu_u8

pytestmark = pytest.mark.gpu

TOL = 1e-5
SHAPES = [(64, 64, 256), (200, 136, 288), (129, 257, 96), (33, 31, 64), (300, 518, 2080), (1, 3, 32),
          (512, 384, 4096)]


def operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(112, 142, (M, K // 32), dtype=np.uint8)
    bs = rng.integers(112, 142, (N, K // 32), dtype=np.uint8)
    return rng, aq, as_, bq, bs


def run(aq, as_, bq, bs, out, dtype, acc):
    need_gpu()
    g = [to_gpu_u8(a) for a in (tile_codes(aq, 0xCD), group_scales(as_), tile_codes(bq, 0xCD), group_scales(bs))]
    F.fp4_gemm_mx(*g, out=out, out_dtype=dtype, accumulate=acc)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def bf16_check(got, ref, mag):
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "NaN pattern differs"
    g, r, s = got[~nan_ref].astype(np.float64), ref[~nan_ref], mag[~nan_ref]
    bound = TOL * s + 2.0 ** -8 * (np.abs(r) + TOL * s)
    bad = np.abs(g - r) > bound
    assert not bad.any(), "%d of %d out of bound; e.g. got %s ref %s" % (
        bad.sum(), bad.size, g[bad][:4], r[bad][:4])


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_output(M, N, K):
    rng, aq, as_, bq, bs = operands(M, N, K, M * 7 + N + K)
    say("gemm_mx bf16", M, N, K)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = run(aq, as_, bq, bs, out, F.OUT_BF16, False)
    ref, mag = O.gemm_rows(aq, as_, bq, bs)
    bf16_check(got, ref, mag)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp32_accumulate(M, N, K):
    rng, aq, as_, bq, bs = operands(M, N, K, M * 11 + N + K)
    say("gemm_mx f32 accumulate", M, N, K)
    ref, mag = O.gemm_rows(aq, as_, bq, bs)
    # an existing C of the product's own magnitude
    c_old = (rng.standard_normal((M, N)) * (np.median(np.abs(ref)) + 1e-30)).astype(np.float32)
    out = torch.from_numpy(c_old.copy()).cuda()
    got = run(aq, as_, bq, bs, out, F.OUT_F32, True)
    gemm_check(got, ref + c_old.astype(np.float64), mag + np.abs(c_old), TOL)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_accumulate(M, N, K):
    rng, aq, as_, bq, bs = operands(M, N, K, M * 13 + N + K)
    say("gemm_mx bf16 accumulate", M, N, K)
    ref, mag = O.gemm_rows(aq, as_, bq, bs)
    c_old = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)
                             * np.float32(np.median(np.abs(ref)) + 1e-30)).to(torch.bfloat16)
    old64 = c_old.float().numpy().astype(np.float64)
    got = run(aq, as_, bq, bs, c_old.cuda(), F.OUT_BF16, True)
    bf16_check(got, ref + old64, mag + np.abs(old64))


def test_nan_scale_bf16():
    """A NaN scale (0xFF) makes its row and column NaN in bf16 too."""
    M, N, K = 96, 80, 320
    rng, aq, as_, bq, bs = operands(M, N, K, 5)
    as_[3, 2] = 0xFF
    bs[10, 0] = 0xFF
    say("gemm_mx bf16 nan scales")
    out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    got = run(aq, as_, bq, bs, out, F.OUT_BF16, False)
    ref, mag = O.gemm_rows(aq, as_, bq, bs)
    bf16_check(got, ref, mag)
    assert np.isnan(got[3]).all() and np.isnan(got[:, 10]).all()


def test_role_entry_points_equal_gemm_mx():
    """Fprop through its role entry point and through fp4_gemm_mx (fp32,
    overwrite) give the same bytes."""
    M, N, K = 300, 260, 1024
    rng, aq, as_, bq, bs = operands(M, N, K, 9)
    need_gpu()
    g = [to_gpu_u8(a) for a in (tile_codes(aq, 0xCD), group_scales(as_), tile_codes(bq, 0xCD), group_scales(bs))]
    a = F.fp4_gemm_fprop(*g)
    b = F.fp4_gemm_mx(*g)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# More tiles than compute units, so each persistent workgroup runs several
# tiles: the tile-to-tile hand-over (the next tile's first stage issued during
# the current tile's epilogue, when both are full) with every tile shape and
# output mode.  (14336, 4096): 1024 full 224 x 256 tiles; (14300, 4000):
# ragged last tile row and column; (4096, 14336): 256 x 224 tiles;
# (8192, 8192): 256 x 256 tiles.
# With K a multiple of 1024 and full tiles the launches take the fast path:
# (14336, 4096, 1024) its 224 x 256 kernel, (8192, 8192, 1024) its 256 x 256
# one, in every output mode, accumulation into fp32 and bf16 included.
# (14300, 4000, 800): a contraction that is no multiple of 256 (25 blocks:
# a partial last stage and a half k-step) with ragged tiles.
MULTI_TILE = [(14336, 4096, 512), (14300, 4000, 512), (4096, 14336, 512), (8192, 8192, 512),
              (14336, 4096, 1024), (8192, 8192, 1024), (14300, 4000, 800)]


@pytest.mark.parametrize("M,N,K", MULTI_TILE)
@pytest.mark.parametrize("mode", ["f32", "bf16", "f32_acc", "bf16_acc"])
def test_multi_tile_sampled(M, N, K, mode):
    rng, aq, as_, bq, bs = operands(M, N, K, M + 3 * N + K)
    say("gemm_mx multi-tile", mode, M, N, K)
    need_gpu()
    if mode == "bf16":
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    elif mode == "f32":
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    else:
        c_old = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).cuda()
        if mode == "bf16_acc":
            c_old = c_old.to(torch.bfloat16)
        out = c_old.clone()
    got = run(aq, as_, bq, bs, out, F.OUT_BF16 if mode.startswith("bf16") else F.OUT_F32,
              mode.endswith("_acc"))
    # whole rows and columns at tile edges and in the middle, then random
    rows = [0, 223, 224, 255, 256, M // 2 + 17, M - 1]
    cols = [0, 223, 224, 255, 256, N // 2 + 5, N - 1]
    mi = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols)), rng.integers(0, M, 4000)])
    ni = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M), rng.integers(0, N, 4000)])
    ref, mag = O.gemm_entries(aq, as_, bq, bs, mi, ni)
    g = got[mi, ni]
    if mode == "bf16":
        bf16_check(g, ref, mag)
    elif mode == "f32":
        gemm_check(g, ref, mag, TOL)
    else:
        old = c_old.float().cpu().numpy()[mi, ni].astype(np.float64)
        if mode == "bf16_acc":
            bf16_check(g, ref + old, mag + np.abs(old))
        else:
            gemm_check(g, ref + old, mag + np.abs(old), TOL)
    assert np.isfinite(got).all()
