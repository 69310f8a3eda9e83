"""GPU parity of the three scaled-FP4 GEMMs against the oracle's binary64
product: |C_gpu - C_ref| <= 1e-5 * sum_k |a_mk b_nk| for every entry checked.
Operands always come from the oracle (random codes and scales, or the
oracle's quantization of workload tensors), never from the GPU path."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
import workloads as W
from _util import gemm_check, group_scales, need_gpu, say, tile_codes, to_gpu_u8

pytestmark = pytest.mark.gpu

TOL = 1e-5


def rand_operands(rng, rows, K, lo=112, hi=142):
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, (rows, K // 32), dtype=np.uint8)
    return codes, scales


def run(fn, ops, out_shape):
    """ops = (a codes, a scales, b codes, b scales) as the oracle writes them
    (codes [rows, K/2], scales [rows, K/32]); they go to the GPU in the
    library's layouts: codes 32-row tiled (padding rows 0xCD), scales
    k-grouped with NaN-scale padding."""
    need_gpu()
    aq, as_, bq, bs = ops
    g = [to_gpu_u8(a) for a in (tile_codes(aq, 0xCD), group_scales(as_), tile_codes(bq, 0xCD), group_scales(bs))]
    out = torch.full(out_shape, float("nan"), dtype=torch.float32, device="cuda")
    fn(*g, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [(64, 64, 256), (200, 136, 288), (129, 257, 96), (256, 256, 1024), (300, 520, 2080),
          (1, 1, 32), (33, 31, 64), (512, 384, 4096), (130, 66, 8192 + 32)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_random_operands(M, N, K):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    aq, as_ = rand_operands(rng, M, K)
    bq, bs = rand_operands(rng, N, K)
    say("gemm random", M, N, K)
    got = run(F.fp4_gemm_fprop, (aq, as_, bq, bs), (M, N))
    ref, mag = O.gemm_rows(aq, as_, bq, bs)
    gemm_check(got, ref, mag, TOL)


def test_gemm_uniform_and_nan_scales():
    rng = np.random.default_rng(5)
    M, N, K = 96, 80, 320
    aq, as_ = rand_operands(rng, M, K)
    bq, bs = rand_operands(rng, N, K)
    as_[3, 2] = 0xFF                     # one NaN scale: row 3 of C is NaN
    bs[10, 0] = 0xFF                     # and column 10
    as_[7, :] = 0                        # the smallest scale, 2^-127
    say("gemm nan/extreme scales")
    got = run(F.fp4_gemm_fprop, (aq, as_, bq, bs), (M, N))
    ref, mag = O.gemm_rows(aq, as_, bq, bs)
    gemm_check(got, ref, mag, TOL)
    assert np.isnan(got[3]).all() and np.isnan(got[:, 10]).all()


def _roles(w, had=O.HAD_DET, seed=0):
    X, dY = W.tensor(w, "X"), W.tensor(w, "dY")
    out = {"wgrad": (O.quant_mx(dY, O.AXIS_ROWS, 32, had, seed), O.quant_mx(X, O.AXIS_ROWS, 32, had, seed))}
    if "W" in w.dists:
        Wt = W.tensor(w, "W")
        out["fprop"] = (O.quant_mx(X, O.AXIS_COLS), O.quant_mx(Wt, O.AXIS_COLS))
        out["dgrad"] = (O.quant_mx(dY, O.AXIS_COLS), O.quant_mx(Wt, O.AXIS_ROWS))
    return out


FN = {"fprop": F.fp4_gemm_fprop, "dgrad": F.fp4_gemm_dgrad, "wgrad": F.fp4_gemm_wgrad}


def out_shape(w, role):
    return {"fprop": (w.T, w.N), "dgrad": (w.T, w.K), "wgrad": (w.N, w.K)}[role]


@pytest.mark.parametrize("w", [W.WORKLOADS["tiny_wgrad"],
                               W.scaled(W.WORKLOADS["q_proj"], 512, 384, 320),
                               W.scaled(W.WORKLOADS["gate_up"], 1024, 256, 448),
                               W.scaled(W.WORKLOADS["down_proj"], 768, 448, 256)],
                         ids=lambda w: w.name)
def test_gemm_roles_workloads(w):
    for role, ((aq, as_), (bq, bs)) in _roles(w).items():
        say("gemm", role, w.name)
        got = run(FN[role], (aq, as_, bq, bs), out_shape(w, role))
        ref, mag = O.gemm_rows(aq, as_, bq, bs)
        gemm_check(got, ref, mag, TOL)


def test_wgrad_tiny_against_unquantized_product():
    """Sanity beyond parity: the quantized rotated Wgrad of the tiny workload
    approximates dY^T X (quantization error, not a parity bound)."""
    w = W.WORKLOADS["tiny_wgrad"]
    X, dY = W.tensor(w, "X"), W.tensor(w, "dY")
    (aq, as_), (bq, bs) = _roles(w)["wgrad"]
    got = run(F.fp4_gemm_wgrad, (aq, as_, bq, bs), (w.N, w.K))
    xf = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    df = (dY.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = df.T @ xf
    mag = np.abs(df).T @ np.abs(xf)
    assert np.median(np.abs(got - exact) / mag) < 0.05


@pytest.mark.slow
@pytest.mark.parametrize("wname", ["gate_up", "q_proj", "down_proj"])
def test_gemm_full_size_sampled(wname):
    """Full Llama-3.1-8B shapes through the benchmark's launch: all three
    GEMMs on oracle-quantized operands, 1024 sampled entries each (corners,
    tile edges and random positions) recomputed by the oracle."""
    w = W.WORKLOADS[wname]
    rng = np.random.default_rng(0)
    had = O.HAD_SIGNED if wname == "down_proj" else O.HAD_DET
    roles = _roles(w, had, 77)
    for role, ((aq, as_), (bq, bs)) in roles.items():
        M, N = out_shape(w, role)
        say("full gemm", wname, role, M, N)
        got = run(FN[role], (aq, as_, bq, bs), (M, N))
        mi = np.concatenate([[0, 0, M - 1, M - 1, 255, 256], rng.integers(0, M, 1018)])
        ni = np.concatenate([[0, N - 1, 0, N - 1, 255, 256], rng.integers(0, N, 1018)])
        ref, mag = O.gemm_entries(aq, as_, bq, bs, mi, ni)
        gemm_check(got[mi, ni], ref, mag, TOL)
        assert np.isfinite(got).all()


# Shapes on which the tile-shape choice (least rounds x tile area on 256 CUs)
# takes each of the kernel's tile shapes: 256 x 256 (4096 x 4096), 224 x 256
# (14336 x 4096, the Wgrad gate/up output) and 256 x 224 (4096 x 14336), with
# ragged edges and contraction sizes with and without a partial last stage
# (640 and 384: 256 x 256 tiles with a half-empty last stage).
TILE_SHAPES = [(4096, 4096, 512), (4000, 4090, 288), (14336, 4096, 256), (14300, 4000, 320),
               (4096, 14336, 256), (4090, 14300, 96), (4096, 4090, 640), (4000, 4096, 384)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_gemm_tile_shapes_sampled(M, N, K):
    rng = np.random.default_rng(M + N + K)
    aq, as_ = rand_operands(rng, M, K)
    bq, bs = rand_operands(rng, N, K)
    say("gemm tile shapes", M, N, K)
    got = run(F.fp4_gemm_fprop, (aq, as_, bq, bs), (M, N))
    # corners, every tile edge of both tilings along a diagonal band, random
    edges = sorted({0, M - 1} | {e for t in (224, 256) for k in range(1, M // t + 1)
                                  for e in (k * t - 1, k * t) if e < M})
    mi = np.concatenate([edges, rng.integers(0, M, 2000)])
    ni = np.concatenate([[(e * 7919) % N for e in edges], rng.integers(0, N, 2000)])
    mi = np.concatenate([mi, [0, M - 1, 0, M - 1]])
    ni = np.concatenate([ni, [0, 0, N - 1, N - 1]])
    ref, mag = O.gemm_entries(aq, as_, bq, bs, mi, ni)
    gemm_check(got[mi, ni], ref, mag, TOL)
    assert np.isfinite(got).all()


@pytest.mark.slow
@pytest.mark.parametrize("K", [2 ** 24 - 256, 2 ** 24 - 32])
def test_gemm_largest_contraction(K):
    """The largest contraction the ABI accepts (K < 2^24), with and without a
    partial last stage, and M = 256 rows: the A operand is just under 2^31
    bytes, so the kernel's 32-bit buffer offsets reach their limit.  64
    entries (corners, tile edges, random) recomputed by the oracle."""
    M, N = 256, 40
    rng = np.random.default_rng(K)
    aq, as_ = rand_operands(rng, M, K)
    bq, bs = rand_operands(rng, N, K)
    assert aq.nbytes < 2 ** 31 and aq.nbytes > 2 ** 31 - 2 ** 24
    say("gemm largest contraction", M, N, K)
    got = run(F.fp4_gemm_fprop, (aq, as_, bq, bs), (M, N))
    mi = np.concatenate([[0, 0, M - 1, M - 1, 223, 224], rng.integers(0, M, 58)])
    ni = np.concatenate([[0, N - 1, 0, N - 1, 5, 39], rng.integers(0, N, 58)])
    ref, mag = O.gemm_entries(aq, as_, bq, bs, mi, ni)
    gemm_check(got[mi, ni], ref, mag, TOL)
    assert np.isfinite(got).all()
