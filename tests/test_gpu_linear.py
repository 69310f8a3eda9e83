"""The MXFP4 linear layer (fp4_precision_gemms_amd.linear) end to end through
torch autograd, against the oracle: Y, dX and dW each equal the oracle's
binary64 GEMM of the oracle-quantized operands (the roles and rotations of
the module's docstring) within the bf16-output bound
|got - ref| <= 1e-5 S + 2^-8 (|ref| + 1e-5 S), S = sum |a b|."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
from _util import bf16_bits, need_gpu, say, to_gpu_bf16

pytestmark = pytest.mark.gpu

TOL = 1e-5
SR_COLS_SEED_XOR = 0x9E3779B97F4A7C15        # the module's seed for the Dgrad-side SR


def check(got, ref, mag, what):
    got = got.detach().float().cpu().numpy().astype(np.float64)
    bound = TOL * mag + 2.0 ** -8 * (np.abs(ref) + TOL * mag)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), "%s: %d of %d out of bound" % (what, bad.sum(), bad.size)


@pytest.mark.parametrize("T,K,N", [(256, 128, 192), (96, 544, 64)])
@pytest.mark.parametrize("mode", ["det_rtn", "signed_sr"])
def test_linear_layer_matches_oracle(T, K, N, mode):
    need_gpu()
    rng = np.random.default_rng(T + K + N)
    xb = bf16_bits(rng.standard_normal((T, K)))
    wb = bf16_bits(rng.standard_normal((N, K)) * 0.02)
    dyb = bf16_bits(rng.standard_normal((T, N)) * 1e-3)
    had, seed, rnd, sr = ((F.HAD_DET, 0, F.RTN, 0) if mode == "det_rtn"
                          else (F.HAD_SIGNED, 1234, F.SR, 77))
    ohad, ornd = {F.HAD_DET: O.HAD_DET, F.HAD_SIGNED: O.HAD_SIGNED}[had], {F.RTN: O.RND_RTN, F.SR: O.RND_SR}[rnd]
    say("linear", T, K, N, mode)
    x = to_gpu_bf16(xb).requires_grad_(True)
    w = to_gpu_bf16(wb).requires_grad_(True)
    y = F.linear.MXFP4LinearFunction.apply(x, w, had, 32, seed, rnd, sr)
    y.backward(to_gpu_bf16(dyb))
    torch.cuda.synchronize()

    ref, mag = O.gemm_rows(*O.quant_mx(xb, O.AXIS_COLS), *O.quant_mx(wb, O.AXIS_COLS))
    check(y, ref, mag, "Y")
    dyc = O.quant_mx(dyb, O.AXIS_COLS, 32, O.HAD_NONE, 0, ornd, sr ^ SR_COLS_SEED_XOR)
    ref, mag = O.gemm_rows(*dyc, *O.quant_mx(wb, O.AXIS_ROWS))
    check(x.grad, ref, mag, "dX")
    dyt = O.quant_mx(dyb, O.AXIS_ROWS, 32, ohad, seed, ornd, sr)
    xt = O.quant_mx(xb, O.AXIS_ROWS, 32, ohad, seed)
    ref, mag = O.gemm_rows(*dyt, *xt)
    check(w.grad, ref, mag, "dW")


def test_linear_module_runs_and_approximates_the_unquantized_layer():
    """Sanity beyond parity: the MXFP4 layer's outputs approximate the
    unquantized product (quantization error, not a parity bound)."""
    need_gpu()
    torch.manual_seed(0)
    layer = F.linear.MXFP4Linear(256, 128, device="cuda")
    with torch.no_grad():
        layer.weight.copy_((torch.randn(128, 256) * 0.05).to(torch.bfloat16))
    x = torch.randn(64, 256, device="cuda").to(torch.bfloat16).requires_grad_(True)
    y = layer(x)
    y.float().square().sum().backward()
    exact = x.detach().double() @ layer.weight.detach().double().T
    rel = (y.detach().double() - exact).norm() / exact.norm()
    assert y.shape == (64, 128) and float(rel) < 0.2
    assert x.grad.shape == x.shape and layer.weight.grad.shape == layer.weight.shape
    assert torch.isfinite(x.grad.float()).all() and torch.isfinite(layer.weight.grad.float()).all()
