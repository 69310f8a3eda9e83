"""Shared test helpers: bf16 bit patterns <-> torch tensors, GPU checks."""
import numpy as np
import pytest
import torch


def bf16_bits(values) -> np.ndarray:
    """bf16 bit patterns (uint16) of float values, rounded to nearest even."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_gpu_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*args):
    """Name the case on stdout before a GPU step (flushed, so a fault that
    ends the process still leaves the case in the log)."""
    print("[case]", *args, flush=True)


def group_scales(s: np.ndarray, pad: int = 0xFF) -> np.ndarray:
    """Row-major E8M0 scales [R, nb] -> the library's k-grouped layout
    [ceil(nb/8), R, 8] (block b of row r at [b // 8, r, b % 8]).  The unused
    tail of the last group gets `pad` (0xFF, a NaN scale, by default: a GEMM
    that read it would show NaN)."""
    R, nb = s.shape
    G = (nb + 7) // 8
    p = np.full((R, G * 8), pad, dtype=np.uint8)
    p[:, :nb] = s
    return np.ascontiguousarray(p.reshape(R, G, 8).transpose(1, 0, 2))


def ungroup_scales(g: np.ndarray, nb: int) -> np.ndarray:
    """k-grouped scales [G, R, 8] -> row-major [R, nb] (drops the tail)."""
    G, R, _ = g.shape
    return np.ascontiguousarray(g.transpose(1, 0, 2).reshape(R, G * 8)[:, :nb])


def tile_codes(c: np.ndarray, pad: int = 0) -> np.ndarray:
    """Row-major MXFP4 codes [R, C/2] -> the library's 32-row tiled layout
    [ceil(R/32), C/32, 512]: the 16 code bytes of row r, block b at
    [r // 32, b, 16 (r % 32) .. + 16].  Rows past R (the padding of the last
    row group) get `pad`."""
    R, half = c.shape
    nb = half // 16
    G = (R + 31) // 32
    p = np.full((G * 32, half), pad, dtype=np.uint8)
    p[:R] = c
    return np.ascontiguousarray(p.reshape(G, 32, nb, 16).transpose(0, 2, 1, 3).reshape(G, nb, 512))


def untile_codes(t: np.ndarray, R: int) -> np.ndarray:
    """The library's tiled codes [ceil(R/32), C/32, 512] -> row-major
    [R, C/2] (drops the padding rows)."""
    G, nb, _ = t.shape
    return np.ascontiguousarray(t.reshape(G, nb, 32, 16).transpose(0, 2, 1, 3).reshape(G * 32, nb * 16)[:R])


def sentinel_u8(shape) -> torch.Tensor:
    return torch.full(shape, 0xCD, dtype=torch.uint8, device="cuda")


def gemm_check(got: np.ndarray, ref: np.ndarray, mag: np.ndarray, tol: float = 1e-5):
    """|got - ref| <= tol * sum|a b| elementwise; NaN exactly where ref is NaN."""
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "NaN pattern differs"
    g, r, s = got[~nan_ref].astype(np.float64), ref[~nan_ref], mag[~nan_ref]
    err = np.abs(g - r)
    bad = err > tol * s
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError("%d of %d entries out of tolerance; e.g. got %s ref %s bound %s"
                             % (bad.sum(), bad.size, g[i], r[i], tol * s[i]))
    return float((err / np.maximum(s, 1e-300)).max()) if err.size else 0.0
