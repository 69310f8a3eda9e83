"""The structural-error diagnostic (fp4_precision_gemms_amd.diagnostics).

Each strategy's per-step MXFP4 Wgrad through the library equals the oracle's
(operands quantized along tokens with the strategy's transform, rounding and
per-step seeds, then the binary64 GEMM) within the GEMM bound; and the
accumulation arithmetic behaves as it must on identical steps: the
deterministic transform repeats the same error every step (|E(S)| = S |E(1)|,
slope 1), stochastic rounding adds independent zero-mean errors (slope well
below 1)."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
from _util import gemm_check, need_gpu, say

from fp4_precision_gemms_amd import diagnostics as D

HAD = {F.HAD_NONE: O.HAD_NONE, F.HAD_DET: O.HAD_DET, F.HAD_SIGNED: O.HAD_SIGNED}
RND = {F.RTN: O.RND_RTN, F.SR: O.RND_SR}


def bits(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("strategy", D.STRATEGIES)
def test_quantized_wgrad_matches_oracle(strategy):
    need_gpu()
    T, N, K = 96, 40, 72
    for step in (0, 3):
        dy, x = D.step_inputs(T, N, K, step, eps=0.5, seed=4)
        say("diagnostic wgrad", strategy, step)
        got = D.quantized_wgrad(torch.from_numpy(dy).to(torch.bfloat16).cuda(),
                                torch.from_numpy(x).to(torch.bfloat16).cuda(), strategy, step, seed=4)
        torch.cuda.synchronize()
        a = D.strategy_args(strategy, step, seed=4)
        common = dict(axis=O.AXIS_ROWS, had_n=a["had_n"], had=HAD[a["had"]],
                      sign_seed=a.get("sign_seed", 0), rnd=RND[a["rnd"]])
        aq, as_ = O.quant_mx(bits(dy), sr_seed=a.get("sr_seed_dy", 0), **common)
        bq, bs = O.quant_mx(bits(x), sr_seed=a.get("sr_seed_x", 0), **common)
        ref, mag = O.gemm_rows(aq, as_, bq, bs)
        gemm_check(got.cpu().numpy(), ref, mag, 1e-5)


def test_step_seeds_differ_only_for_random_strategies():
    assert D.strategy_args("det", 0) == D.strategy_args("det", 5)
    assert D.strategy_args("random_hadamard", 0)["sign_seed"] != D.strategy_args("random_hadamard", 1)["sign_seed"]
    a, b = D.strategy_args("sr", 2), D.strategy_args("sr", 3)
    assert len({a["sr_seed_dy"], a["sr_seed_x"], b["sr_seed_dy"], b["sr_seed_x"]}) == 4


@pytest.mark.gpu
def test_identical_steps_growth():
    need_gpu()
    say("diagnostic growth, identical steps")
    r = D.wgrad_error_growth(T=512, N=128, K=128, steps=8, eps=0.0)
    det = np.asarray(r["det"]["growth"])
    assert np.allclose(det, np.arange(1, 9), rtol=1e-9)
    assert abs(r["det"]["slope"] - 1.0) < 1e-6
    assert r["sr"]["slope"] < 0.75
    assert r["sr"]["rel_accum_err"][-1] < 0.6 * r["sr"]["rel_err_per_step"][0]
    for st in D.STRATEGIES:
        assert all(0 < e < 1 for e in r[st]["rel_err_per_step"])
