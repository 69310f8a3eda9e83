"""Structural-error diagnostic for the MXFP4 Wgrad.

[AMD-MXFP4] "Pretraining large language models with MXFP4 on Native FP4
Hardware" (htx.com news item), section "Поисковая экспериментальная работа:
корень нестабильности": with Wgrad in MXFP4, stochastic rounding and the
randomized Hadamard transform made training diverge while the deterministic
transform kept it close to FP8; the explanation offered is that the random
strategies give a different error pattern at every step and those patterns
build up along the gradient path, while the deterministic transform keeps
the pattern the same from step to step.

This module measures that on synthetic data, without training: over a
sequence of steps s = 0 .. S-1 it forms the MXFP4 Wgrad dW_q(s) of
(dY_s, X_s) through the library (the operand pair quantized along tokens by
fp4_wgrad_quantize, then fp4_gemm_wgrad) and the exact dW(s) = dY_s^T X_s
(binary64, on the host), and reports how the accumulated error
E(S) = sum_{s<S} (dW_q(s) - dW(s)) grows with S for each strategy:

    det              Hadamard-32, the same every step, round to nearest
    random_hadamard  random-sign Hadamard-32, a new sign seed every step,
                     round to nearest
    sr               no transform, stochastic rounding with new seeds every
                     step (the pages' stochastic-rounding strategy)

The inputs drift slowly: X_s = X + eps Z_s and dY_s = sigma (G + eps V_s)
with fresh Gaussian Z_s, V_s per step (eps = 0: the same tensors every step;
large eps: independent steps).  A log-log slope of |E(S)| near 1 means
errors that add up coherently, near 1/2 errors that add like independent
noise.  The reported numbers are measurements; the pages give none for this
proxy.
"""
from __future__ import annotations

import argparse
import json

import numpy as np
import torch

from . import HAD_DET, HAD_NONE, HAD_SIGNED, RTN, SR, fp4_gemm_wgrad, fp4_wgrad_quantize

STRATEGIES = ("det", "random_hadamard", "sr")


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(device)


def step_inputs(T: int, N: int, K: int, step: int, eps: float, seed: int = 0,
                dy_std: float = 1e-3):
    """The bf16 dY_s [T, N] and X_s [T, K] of one step, as float32 arrays
    holding bf16 values (rounded to nearest even)."""
    def normal(tensor_id, stream, shape):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, stream])))
        return rng.standard_normal(shape, dtype=np.float32)

    x = normal(1, 0, (T, K)) + np.float32(eps) * normal(1, step + 1, (T, K))
    dy = np.float32(dy_std) * (normal(3, 0, (T, N)) + np.float32(eps) * normal(3, step + 1, (T, N)))
    to_bf16 = lambda a: torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    return to_bf16(dy), to_bf16(x)


def strategy_args(strategy: str, step: int, seed: int = 0) -> dict:
    """Keyword arguments of fp4_wgrad_quantize for one strategy at one step:
    the sign seed and SR seeds change with the step where the strategy is
    random, and stay fixed for the deterministic transform."""
    base = (seed & 0xFFFFFFFF) << 32
    if strategy == "det":
        return dict(had_n=32, had=HAD_DET, sign_seed=0, rnd=RTN)
    if strategy == "random_hadamard":
        return dict(had_n=32, had=HAD_SIGNED, sign_seed=base | step, rnd=RTN)
    if strategy == "sr":
        return dict(had_n=32, had=HAD_NONE, rnd=SR, sr_seed_dy=base | (2 * step),
                    sr_seed_x=base | (2 * step + 1))
    raise ValueError("unknown strategy %r" % strategy)


def quantized_wgrad(dy: torch.Tensor, x: torch.Tensor, strategy: str, step: int,
                    seed: int = 0) -> torch.Tensor:
    """dW_q = MXFP4 Wgrad of bf16 dY [T, N] and X [T, K] on the GPU: both
    operands quantized along T under the strategy's settings for this step,
    then the scaled FP4 GEMM; fp32 [N, K]."""
    q = fp4_wgrad_quantize(dy, x, **strategy_args(strategy, step, seed))
    return fp4_gemm_wgrad(*q)


def _slope(values) -> float:
    s = np.log(np.arange(1, len(values) + 1, dtype=np.float64))
    v = np.log(np.maximum(np.asarray(values, dtype=np.float64), 1e-300))
    if len(values) < 2:
        return float("nan")
    return float(np.polyfit(s, v, 1)[0])


def wgrad_error_growth(T: int = 2048, N: int = 512, K: int = 512, steps: int = 16, eps: float = 0.1,
                       strategies=STRATEGIES, seed: int = 0, device="cuda") -> dict:
    """Per strategy: the relative error of each step's dW_q, the relative
    accumulated error |E(S)| / |sum dW| and the growth |E(S)| / |E(1)| for
    S = 1 .. steps (Frobenius norms, binary64), and the log-log slope of
    |E(S)| against S."""
    if T % 32:
        raise ValueError("T must be a multiple of 32")
    dev = torch.device(device)
    acc_err = {st: np.zeros((N, K)) for st in strategies}
    acc_ref = np.zeros((N, K))
    out = {st: {"rel_err_per_step": [], "rel_accum_err": [], "accum_err_norm": []} for st in strategies}
    for s in range(steps):
        dy, x = step_inputs(T, N, K, s, eps, seed)
        ref = dy.astype(np.float64).T @ x.astype(np.float64)
        acc_ref += ref
        g_dy, g_x = _bf16(dy, dev), _bf16(x, dev)
        for st in strategies:
            dwq = quantized_wgrad(g_dy, g_x, st, s, seed).double().cpu().numpy()
            err = dwq - ref
            acc_err[st] += err
            out[st]["rel_err_per_step"].append(float(np.linalg.norm(err) / np.linalg.norm(ref)))
            out[st]["accum_err_norm"].append(float(np.linalg.norm(acc_err[st])))
            out[st]["rel_accum_err"].append(float(np.linalg.norm(acc_err[st]) / np.linalg.norm(acc_ref)))
    for st in strategies:
        e = out[st]["accum_err_norm"]
        out[st]["growth"] = [v / e[0] for v in e]
        out[st]["slope"] = _slope(e)
    out["config"] = {"T": T, "N": N, "K": K, "steps": steps, "eps": eps, "seed": seed,
                     "dy_std": 1e-3, "hadamard_n": 32}
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--T", type=int, default=2048)
    ap.add_argument("--N", type=int, default=512)
    ap.add_argument("--K", type=int, default=512)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--eps", type=float, nargs="+", default=[0.0, 0.1, 1.0])
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args(argv)
    for eps in args.eps:
        r = wgrad_error_growth(args.T, args.N, args.K, args.steps, eps, seed=args.seed)
        summary = {st: {"slope": round(r[st]["slope"], 3),
                        "rel_err_step0": round(r[st]["rel_err_per_step"][0], 5),
                        "rel_accum_err_last": round(r[st]["rel_accum_err"][-1], 5),
                        "growth_last": round(r[st]["growth"][-1], 3)} for st in STRATEGIES}
        print(json.dumps({"config": r["config"], "summary": summary}), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
