"""Seeded synthetic inputs for the block-quantized linear layer.

This module only draws random numbers and rounds them to bf16; it holds none
of the quantization or GEMM arithmetic.  Both the oracle-side tests and the
GPU path consume the same bf16 bytes produced here.

The pages measure on Llama 3.1-8B pretraining (MLPerf, C4) and on NVFP4 models
evaluated with MMLU-Pro; neither data nor weights are used.  Tensors of the
same layer shapes with Gaussian or Student-t values stand in for them.

Generator: torch's CPU generator seeded with the first 64-bit word of
numpy's SeedSequence([cfg_seed, tensor_id]); values drawn in float32 and
rounded to bf16 (round-to-nearest-even).  Student-t with an integer nu is
drawn by its definition, Z / sqrt(sum of nu squared normals / nu).
tensor_id: X = 1, W = 2, dY = 3, x (single-tensor configs) = 4.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

TENSOR_ID = {"X": 1, "W": 2, "dY": 3, "x": 4}


@dataclass(frozen=True)
class Dist:
    """A value distribution: 'normal' (std) or 'student_t' (nu, scale), with
    optional outliers: a Bernoulli(p) mask of entries multiplied by `factor`
    ('entries'), or `n_channels` seeded columns multiplied by `factor`."""
    kind: str = "normal"
    std: float = 1.0
    nu: float = 3.0
    outlier: str = ""           # "", "entries", "channels"
    p: float = 0.0
    n_channels: int = 0
    factor: float = 1.0


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                      # tokens
    K: int                      # in-features
    N: int                      # out-features
    dists: dict = field(default_factory=dict)   # tensor name -> Dist
    seed: int = 0


def _generator(seed: int, tensor_id: int) -> torch.Generator:
    word = np.random.SeedSequence([seed, tensor_id]).generate_state(1, np.uint64)[0]
    return torch.Generator().manual_seed(int(word) & 0x7FFFFFFFFFFFFFFF)


def draw(shape, dist: Dist, seed: int, tensor_id: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of a seeded tensor of `shape`."""
    g = _generator(seed, tensor_id)
    n = int(np.prod(shape))
    if dist.kind == "normal":
        v = torch.randn(n, generator=g, dtype=torch.float32).mul_(dist.std)
    elif dist.kind == "student_t":
        nu = int(dist.nu)
        if nu != dist.nu or nu < 1:
            raise ValueError("integer degrees of freedom only")
        z = torch.randn(n, generator=g, dtype=torch.float32)
        chi2 = torch.zeros(n, dtype=torch.float32)
        for _ in range(nu):
            chi2.addcmul_(*(2 * [torch.randn(n, generator=g, dtype=torch.float32)]))
        v = z.div_(chi2.div_(nu).sqrt_()).mul_(dist.std)
        del chi2
    else:
        raise ValueError(dist.kind)
    v = v.view(shape)
    if dist.outlier == "entries":
        mask = torch.rand(shape, generator=g) < dist.p
        v[mask] *= dist.factor
    elif dist.outlier == "channels":
        cols = torch.randperm(shape[1], generator=g)[:dist.n_channels]
        v[:, cols] *= dist.factor
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def tensor(w: Workload, name: str) -> np.ndarray:
    """The named tensor of workload `w`: X[T,K], W[N,K], dY[T,N] or x[T,K]."""
    shape = {"X": (w.T, w.K), "W": (w.N, w.K), "dY": (w.T, w.N), "x": (w.T, w.K)}[name]
    return draw(shape, w.dists[name], w.seed, TENSOR_ID[name])


# Distributions of the Llama-3.1-8B-shaped layers: activations N(0, 1),
# weights N(0, 0.02) (std), output gradients N(0, 1e-4) (std).
_ACT = Dist("normal", 1.0)
_WEIGHT = Dist("normal", 0.02)
_GRAD = Dist("normal", 1e-4)

WORKLOADS = {
    # tiny Wgrad: X[256x128], dY[256x64] with 1 % of entries x20
    "tiny_wgrad": Workload("tiny_wgrad", T=256, K=128, N=64, dists={
        "X": _ACT, "dY": Dist("normal", 1e-3, outlier="entries", p=0.01, factor=20.0)}),
    # Llama-3.1-8B attention q_proj, one micro-batch of 8192 tokens
    "q_proj": Workload("q_proj", T=8192, K=4096, N=4096,
                       dists={"X": _ACT, "W": _WEIGHT, "dY": _GRAD}),
    # Llama-3.1-8B MLP gate/up projection
    "gate_up": Workload("gate_up", T=8192, K=4096, N=14336,
                        dists={"X": _ACT, "W": _WEIGHT, "dY": _GRAD}),
    # Llama-3.1-8B MLP down projection, heavy-tailed activations with 0.1 %
    # of the 14336 channels (14) scaled x50
    "down_proj": Workload("down_proj", T=8192, K=14336, N=4096, dists={
        "X": Dist("student_t", 1.0, nu=3.0, outlier="channels", n_channels=14, factor=50.0),
        "W": _WEIGHT, "dY": _GRAD}),
    # NVFP4 quantize-only: one [16384 x 8192] Student-t (nu = 4) tensor
    "nvfp4": Workload("nvfp4", T=16384, K=8192, N=0,
                      dists={"x": Dist("student_t", 1.0, nu=4.0)}),
}


def scaled(w: Workload, T: int, K: int, N: int, name: str | None = None) -> Workload:
    """Same distributions at another size (parity cases the oracle finishes
    in seconds).  Channel-outlier counts scale with the column count."""
    dists = {}
    for k, d in w.dists.items():
        if d.outlier == "channels":
            cols = K if k in ("X", "W", "x") else N
            d = Dist(d.kind, d.std, d.nu, d.outlier, d.p,
                     max(1, round(0.001 * cols)) if d.n_channels else 0, d.factor)
        dists[k] = d
    return Workload(name or "%s_%dx%dx%d" % (w.name, T, K, N), T, K, N, dists, w.seed)
