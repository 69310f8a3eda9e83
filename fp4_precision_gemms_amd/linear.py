"""An MXFP4 linear layer as a torch autograd Function: Fprop, Dgrad and
Wgrad on the scaled FP4 matrix cores, wired the way the pages describe.

[AMD-MXFP4] "Pretraining large language models with MXFP4 on Native FP4
Hardware", section "Поисковая экспериментальная работа: корень
нестабильности": the three GEMMs of a linear layer run in MXFP4 --

    Fprop  Y  = X W^T      X along K, W along K      (no rotation)
    Dgrad  dX = dY W       dY along N, W^T along N   (no rotation)
    Wgrad  dW = dY^T X     dY^T, X^T along T         (block Hadamard on both)

-- and the rotation is applied only to the Wgrad operands, the same
transform on both so that it cancels in dY^T X.

Every operand is quantized once per direction by the dual quantizer (one
read of X, of W and of dY each); forward keeps only the quantized operands
backward needs (X^T and W^T codes), not the bf16 tensors.  Inputs and the
weight are bf16; Y, dX and dW are returned in bf16 (each the fp32 GEMM
result rounded to nearest even by the GEMM kernel).  This module only
sequences library calls; all arithmetic runs in libfp4.so.
"""
from __future__ import annotations

import torch

from . import HAD_DET, HAD_NONE, OUT_BF16, RTN, fp4_gemm_mx, fp4_hadamard_quantize_dual


class MXFP4LinearFunction(torch.autograd.Function):
    """y = x w^T with x [T, K], w [N, K] (both bf16, T and K multiples of 32,
    N a multiple of 32), all three GEMMs in MXFP4."""

    @staticmethod
    def forward(ctx, x, w, had: int = HAD_DET, had_n: int = 32, sign_seed: int = 0,
                grad_rounding: int = RTN, sr_seed: int = 0):
        x = x.contiguous()
        w = w.contiguous()
        # X: along rows (X^T, Wgrad, rotated) and along cols (Fprop)
        xtq, xts, xq, xs = fp4_hadamard_quantize_dual(x, had_n, had, sign_seed, RTN, 0,
                                                      32, HAD_NONE, 0, RTN, 0)
        # W [N, K]: along rows (W^T, Dgrad) and along cols (Fprop)
        wtq, wts, wq, ws = fp4_hadamard_quantize_dual(w, 32, HAD_NONE, 0, RTN, 0,
                                                      32, HAD_NONE, 0, RTN, 0)
        y = fp4_gemm_mx(xq, xs, wq, ws, out_dtype=OUT_BF16)
        ctx.save_for_backward(xtq, xts, wtq, wts)
        ctx.cfg = (had, had_n, sign_seed, grad_rounding, sr_seed)
        return y

    @staticmethod
    def backward(ctx, dy):
        xtq, xts, wtq, wts = ctx.saved_tensors
        had, had_n, sign_seed, grad_rounding, sr_seed = ctx.cfg
        dy = dy.to(torch.bfloat16).contiguous()
        # dY: along rows (dY^T, Wgrad, the same rotation as X^T) and along cols
        # (Dgrad); the gradient may be rounded stochastically
        dytq, dyts, dyq, dys = fp4_hadamard_quantize_dual(dy, had_n, had, sign_seed, grad_rounding,
                                                          sr_seed, 32, HAD_NONE, 0, grad_rounding,
                                                          sr_seed ^ 0x9E3779B97F4A7C15)
        dx = fp4_gemm_mx(dyq, dys, wtq, wts, out_dtype=OUT_BF16)       # [T, K]
        dw = fp4_gemm_mx(dytq, dyts, xtq, xts, out_dtype=OUT_BF16)     # [N, K]
        return dx, dw, None, None, None, None, None


class MXFP4Linear(torch.nn.Module):
    """A bias-free linear layer whose three GEMMs run in MXFP4.  `sign_seed`
    selects the random-sign Hadamard when had = HAD_SIGNED (change it per
    step for a per-step random rotation)."""

    def __init__(self, in_features: int, out_features: int, had: int = HAD_DET, had_n: int = 32,
                 grad_rounding: int = RTN, device=None):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features,
                                                     dtype=torch.bfloat16, device=device))
        self.had, self.had_n, self.grad_rounding = had, had_n, grad_rounding
        self.sign_seed = 0
        self.sr_seed = 0

    def forward(self, x):
        return MXFP4LinearFunction.apply(x, self.weight, self.had, self.had_n, self.sign_seed,
                                         self.grad_rounding, self.sr_seed)
