"""GPU parity of nvfp4_quantize against the oracle: codes, E4M3 scales and
the tensor scale bit-exact, with the amax computed in the library (two
passes) or supplied (one pass), in each rounding mode (elements to nearest
with or without the renormalized scale, or every element stochastic)."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
import workloads as W
from _util import bf16_bits, need_gpu, say, sentinel_u8, to_gpu_bf16

pytestmark = pytest.mark.gpu

HD = {O.HAD_NONE: F.HAD_NONE, O.HAD_DET: F.HAD_DET, O.HAD_SIGNED: F.HAD_SIGNED}


def gpu_nv(bits, had, seed, mode, sr_seed, amax_in=None):
    need_gpu()
    x = to_gpu_bf16(bits)
    rows, cols = bits.shape
    codes, scales = sentinel_u8((rows, cols // 2)), sentinel_u8((rows, cols // 16))
    ts = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    a = None if amax_in is None else torch.tensor([amax_in], dtype=torch.float32, device="cuda")
    F.nvfp4_quantize(x, HD[had], seed, mode, sr_seed, amax_in=a, codes=codes, scales=scales,
                     tensor_scale=ts)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), np.float32(ts.item())


def check(bits, had, seed, mode, sr_seed, amax_in=None, what=""):
    say("nvfp4", what, bits.shape, had, mode, amax_in)
    gc, gs, gt = gpu_nv(bits, had, seed, mode, sr_seed, amax_in)
    rc, rs, rt = O.nvfp4_quantize(bits, had, seed, mode, sr_seed, amax_in)
    assert gt.view(np.uint32) == rt.view(np.uint32), (gt, rt)
    assert np.array_equal(gs, rs), ("scales", (gs != rs).sum(), np.argwhere(gs != rs)[:5].tolist())
    assert np.array_equal(gc, rc), ("codes", (gc != rc).sum(), np.argwhere(gc != rc)[:5].tolist())


@pytest.mark.parametrize("had", [O.HAD_NONE, O.HAD_DET, O.HAD_SIGNED])
@pytest.mark.parametrize("mode", [O.NV_RTN, O.NV_RENORM_SR, O.NV_ELEMENT_SR])
@pytest.mark.parametrize("shape", [(64, 256), (3, 16), (130, 1040), (7, 48), (5, 112)])
def test_nvfp4_parity(had, mode, shape):
    rng = np.random.default_rng(shape[0] + shape[1])
    bits = bf16_bits(rng.standard_t(4, shape))
    check(bits, had, 9, mode, 4, what="t4")
    check(bits, had, 9, mode, 4, amax_in=3.5, what="amax_in")


def test_nvfp4_edge_values():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((16, 64))
    v[0] = 0.0                                  # zero blocks -> scale 0, codes 0
    v[1, :16] = 1e-30                           # block far below the tensor scale
    v[2, 5] = 1e4                               # one outlier
    v[3, :] = -0.0
    check(bf16_bits(v), O.HAD_SIGNED, 1, 1, 2, what="edge")
    check(bf16_bits(v), O.HAD_NONE, 1, 1, 2, what="edge")
    check(bf16_bits(np.zeros((4, 32))), O.HAD_SIGNED, 1, 1, 2, what="zeros")
    check(bf16_bits(v), O.HAD_SIGNED, 1, O.NV_ELEMENT_SR, 2, what="edge element SR")


@pytest.mark.slow
def test_nvfp4_full_size():
    """The [16384 x 8192] Student-t (nu = 4) tensor, whole, as benchmarked."""
    w = W.WORKLOADS["nvfp4"]
    bits = W.tensor(w, "x")
    check(bits, O.HAD_SIGNED, 123, O.NV_RENORM_SR, 77, what="full")
    check(bits, O.HAD_SIGNED, 123, O.NV_ELEMENT_SR, 77, what="full element SR")


MODES = [O.NV_RTN, O.NV_RENORM_SR, O.NV_ELEMENT_SR]


def _edge_tensor():
    """Finite blocks, a NaN, +-Inf, a block whose 16-point rotation overflows,
    values near the binary32 limit (renorm sums overflow) and tiny ones."""
    rng = np.random.default_rng(21)
    v = rng.standard_normal((12, 96)).astype(np.float32)
    v[0, 3] = np.nan
    v[2, 40] = np.inf
    v[3, 70] = -np.inf
    v[5, 16:32] = 3.0e38                   # finite; the rotation overflows
    v[7, 48:64] = -3.0e38
    v[9, :16] = 1e-38
    return v


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("had", [O.HAD_NONE, O.HAD_SIGNED])
def test_nvfp4_nonfinite_inputs(mode, had):
    """The library's rule for non-finite values, bit-exact against the
    oracle: with the amax computed, a NaN or infinity anywhere makes the
    whole tensor NaN; with it supplied, only the affected blocks get scale
    0x7F and zero codes."""
    with np.errstate(over="ignore", invalid="ignore"):
        bits = bf16_bits(_edge_tensor())
    check(bits, had, 3, mode, 8, what="nonfinite computed amax")
    check(bits, had, 3, mode, 8, amax_in=5.0, what="nonfinite amax_in")
    check(bits, had, 3, mode, 8, amax_in=3.0e38, what="nonfinite huge amax_in")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("amax", [float("nan"), float("inf"), -1.0, 1e-45, 0.0])
def test_nvfp4_invalid_amax_in(mode, amax):
    rng = np.random.default_rng(22)
    bits = bf16_bits(rng.standard_t(4, (8, 64)))
    check(bits, O.HAD_SIGNED, 4, mode, 9, amax_in=amax, what="amax_in %r" % amax)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("had", [O.HAD_NONE, O.HAD_DET])
def test_nvfp4_tiny_and_huge_tensors(mode, had):
    """A tensor near 2^-127 (reciprocal block scales overflow) and one near
    3e38 (the renormalized target can be Inf / Inf), each whole."""
    rng = np.random.default_rng(23)
    tiny = (rng.uniform(0.5, 1.0, (8, 64)) * 2.0 ** -127).astype(np.float32)
    tiny[7] *= 2.0 ** 8
    huge = (rng.standard_normal((8, 64)) * 1e37).astype(np.float32)
    huge[0, :16] = 3.0e38
    check(bf16_bits(tiny), had, 2, mode, 6, what="tiny")
    check(bf16_bits(huge), had, 2, mode, 6, what="huge")
    check(bf16_bits(tiny), had, 2, mode, 6, amax_in=1e-40, what="tiny, small amax_in")
