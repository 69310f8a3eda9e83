"""Pins of the oracle's Hadamard transform and Philox4x32-10 generator.

Hadamard: orthogonality (H H^T = n I), agreement with scipy's Sylvester
Hadamard matrix on inputs where binary32 is exact, the binary32 value of
1/sqrt(n), and cancellation of the rotation in a product along the rotated
axis.  Philox: word-for-word agreement with rocRAND's independent engine
(header-only, run on the host) and uniformity.  CPU only."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.linalg

import oracle as O


def _oracle_matrix(n, had=O.HAD_DET, seed=0):
    """Rows of the transform as the oracle applies it (columns = basis images),
    without the final normalization: apply to integer unit vectors, exact."""
    s = O.hadamard_signs(had, n, seed)
    c = float(O.hadamard_norm(n))
    cols = [O.fwht(np.eye(n, dtype=np.float32)[j], s) / c for j in range(n)]
    return np.stack(cols, axis=1).astype(np.float64)   # column j = T e_j


@pytest.mark.parametrize("n", [16, 32])
def test_fwht_is_sylvester_hadamard(n):
    M = _oracle_matrix(n)
    H = scipy.linalg.hadamard(n)
    assert np.array_equal(np.rint(M), M) or np.allclose(M, np.rint(M), atol=1e-6)
    assert np.array_equal(np.rint(M).astype(int), H)
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=int))
    # Sylvester order: row 1 alternates + - + - ...
    assert list(H[1, :4]) == [1, -1, 1, -1]


@pytest.mark.parametrize("n", [16, 32])
def test_fwht_integer_inputs_exact(n):
    rng = np.random.default_rng(n)
    H = scipy.linalg.hadamard(n).astype(np.float64)
    for _ in range(50):
        x = rng.integers(-1000, 1000, n).astype(np.float32)
        y = O.fwht(x)
        ref = (H @ x.astype(np.float64)).astype(np.float32) * O.hadamard_norm(n)
        assert np.array_equal(y, ref.astype(np.float32))


def test_norm_constants():
    assert np.float32(O.hadamard_norm(16)).view(np.uint32) == 0x3E800000
    assert np.float32(O.hadamard_norm(32)).view(np.uint32) == np.float32(1 / np.sqrt(32)).view(np.uint32)
    assert np.float32(O.hadamard_norm(32)).view(np.uint32) == 0x3E3504F3


@pytest.mark.parametrize("n", [16, 32])
def test_signed_transform_is_hadamard_times_signs(n):
    seed = 0x5EED
    s = O.hadamard_signs(O.HAD_SIGNED, n, seed)
    assert set(np.unique(s)) <= {-1.0, 1.0} and (s < 0).any()
    w = O.stream_word(seed, 1, 0)
    assert all((s[j] < 0) == bool((w >> j) & 1) for j in range(n))
    M = _oracle_matrix(n, O.HAD_SIGNED, seed)
    assert np.array_equal(np.rint(M), scipy.linalg.hadamard(n) @ np.diag(s))
    assert np.array_equal(O.hadamard_signs(O.HAD_DET, n, seed), np.ones(n, np.float32))
    assert not np.array_equal(O.hadamard_signs(O.HAD_SIGNED, n, seed + 1), s)


@pytest.mark.parametrize("had,seed", [(O.HAD_DET, 0), (O.HAD_SIGNED, 11), (O.HAD_SIGNED, 12)])
def test_rotation_cancels_in_products(had, seed):
    """(H D a)^T (H D b) = a^T b along the rotated axis: the rotation of both
    Wgrad operands along tokens leaves dY^T X unchanged up to rounding."""
    rng = np.random.default_rng(seed)
    T = 256
    a = rng.standard_normal(T).astype(np.float32)
    b = rng.standard_normal(T).astype(np.float32)
    s = O.hadamard_signs(had, 32, seed)
    ra = np.concatenate([O.fwht(a[i:i + 32], s) for i in range(0, T, 32)])
    rb = np.concatenate([O.fwht(b[i:i + 32], s) for i in range(0, T, 32)])
    lhs = ra.astype(np.float64) @ rb.astype(np.float64)
    rhs = a.astype(np.float64) @ b.astype(np.float64)
    scale = np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64)
    assert abs(lhs - rhs) < 1e-6 * scale
    # mismatched signs do not cancel
    if had == O.HAD_SIGNED:
        s2 = O.hadamard_signs(had, 32, seed + 100)
        rb2 = np.concatenate([O.fwht(b[i:i + 32], s2) for i in range(0, T, 32)])
        assert abs(ra.astype(np.float64) @ rb2.astype(np.float64) - rhs) > 1e-3 * scale


# --- Philox ------------------------------------------------------------------

def _rocrand_dump(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc / rocRAND headers not present")
    src = os.path.join(os.path.dirname(__file__), "helpers", "rocrand_philox_dump.cpp")
    exe = str(tmp_path_factory.mktemp("rocrand") / "dump")
    subprocess.check_call([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", src, "-o", exe])
    return exe


@pytest.fixture(scope="module")
def rocrand_dump(tmp_path_factory):
    return _rocrand_dump(tmp_path_factory)


@pytest.mark.parametrize("seed,sub,off", [(0, 0, 0), (1, 0, 0), (0x123456789ABCDEF, 0, 0),
                                          (0xFFFFFFFFFFFFFFFF, 3, 4 * 1000),
                                          (42, 1, 4 * (2 ** 32 - 2)), (7, 2, 0)])
def test_philox_matches_rocrand(rocrand_dump, seed, sub, off):
    """rocRAND's Philox4x32-10 engine keys with (seed low, seed high) and
    counts (offset/4 low, high, subsequence low, high): the same generator
    our streams use with purpose = subsequence."""
    calls = 64
    out = subprocess.check_output([rocrand_dump, str(seed), str(sub), str(off), str(calls)], text=True)
    rows = [[int(w, 16) for w in line.split()] for line in out.strip().splitlines()]
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for i, row in enumerate(rows):
        g = off // 4 + i
        ctr = [g & 0xFFFFFFFF, (g >> 32) & 0xFFFFFFFF, sub & 0xFFFFFFFF, sub >> 32]
        assert list(O.philox4x32_10(ctr, key)) == row, (i, row)
        for w in range(4):
            assert O.stream_word(seed, sub, 4 * g + w) == row[w]


def test_philox_uniformity():
    n = 1 << 16
    words = np.array([O.stream_word(3, 0, i) for i in range(n)], dtype=np.uint64)
    for shift in (0, 8, 24, 28):
        bins = np.bincount(((words >> shift) & 15).astype(np.int64), minlength=16)
        chi2 = ((bins - n / 16) ** 2 / (n / 16)).sum()
        assert chi2 < 50.0          # 15 dof: p < 1e-5 beyond ~44
    bits = np.unpackbits(words.astype(">u4").view(np.uint8))
    assert abs(bits.mean() - 0.5) < 4 * 0.5 / np.sqrt(bits.size)
