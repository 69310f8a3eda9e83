"""libfp4calib.so without a GPU: it loads, exports what include/fp4_calib.h
declares, counts its work as documented, and rejects bad arguments before
any HIP call (the fake pointers below are never touched)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4_calib.h")


@pytest.fixture(scope="module")
def C():
    from fp4_precision_gemms_amd import calib
    if not os.path.exists(calib.LIB_PATH):
        pytest.skip("libfp4calib.so not built")
    return calib


def declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, re.M)))


def test_declared_symbols_exported(C):
    names = declared()
    assert names == ["fp4_calib_clock_stamp", "fp4_calib_mfma", "fp4_calib_mfma_flops", "fp4_calib_mfma_src_bytes"]
    out = subprocess.check_output(["nm", "-D", "--defined-only", C.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_work_counts(C):
    L = C.lib()
    # 18 fragments of 16 bytes per lane, 256 lanes per workgroup
    assert L.fp4_calib_mfma_src_bytes(256) == 256 * 256 * 18 * 16
    assert L.fp4_calib_mfma_src_bytes(0) == 0
    # 2*32*32*64 flop per MFMA, 28 MFMAs per wave-iteration, 4 waves
    assert L.fp4_calib_mfma_flops(2, 3) == 2 * 32 * 32 * 64 * 28 * 3 * 2 * 4
    assert L.fp4_calib_mfma_flops(0, 3) == 0.0


def test_argument_errors(C):
    L = C.lib()
    A = 0x10000
    assert L.fp4_calib_mfma(0, 1, 1, A, A, None) == 1
    assert L.fp4_calib_clock_stamp(None, None) == 1
    assert L.fp4_calib_clock_stamp(A + 4, None) == 3
    assert L.fp4_calib_mfma(A, 1, 1, 0, A, None) == 1
    assert L.fp4_calib_mfma(A, 0, 1, A, A, None) == 2
    assert L.fp4_calib_mfma(A, 65537, 1, A, A, None) == 2
    assert L.fp4_calib_mfma(A, 1, 0, A, A, None) == 2
    assert L.fp4_calib_mfma(A, 1, (1 << 24) + 1, A, A, None) == 2
    assert L.fp4_calib_mfma(A + 8, 1, 1, A, A, None) == 3


def test_span_ghz_pairs_records_of_one_xcd():
    from fp4_precision_gemms_amd.calib import span_ghz
    # XCD 0 ran at 2.0 GHz, XCD 1 at 1.5 GHz (own counter origins), XCD 2
    # only in the second stamp: the median of the two pairs
    begin = [[1000, 50, 0, 0], [9_000_000, 50, 1, 0], [1001, 51, 0, 0]]
    end = [[9_000_000 + 15 * 100, 150, 1, 0], [1000 + 20 * 100, 150, 0, 0], [7, 150, 2, 0]]
    assert abs(span_ghz(begin, end) - 2.0) < 1e-12        # upper median of [1.5, 2.0]
    assert abs(span_ghz(begin[:1], end) - 2.0) < 1e-12
    assert span_ghz(begin[:1], end[:1]) != span_ghz(begin[:1], end[:1])      # NaN: no common XCD


def test_stamp_count_matches_header():
    from fp4_precision_gemms_amd.calib import STAMPS
    m = re.search(r"#define FP4_CALIB_STAMPS (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == STAMPS


def test_operand_fragments_follow_the_loop_layout():
    """Wave w's fragments f = set * 9 + i (A, i < 7) and set * 9 + 7 + j (B)
    are the 1 KB pieces 14 w + 7 set + i of A and 4 w + 2 set + j of B."""
    import torch
    from fp4_precision_gemms_amd import calib
    a = (torch.arange(40 * 1024) % 253).to(torch.uint8)        # 40 pieces
    b = (torch.arange(6 * 1024) % 241).to(torch.uint8)         # 6 pieces
    src = calib.operand_fragments(a, b, 5)
    assert src.numel() == 5 * 18 * 1024 and src.is_contiguous()
    f = src.reshape(5, 2, 9, 1024)
    pa, pb = a.reshape(-1, 1024), b.reshape(-1, 1024)
    for w in range(5):
        for s in range(2):
            for i in range(7):
                assert torch.equal(f[w, s, i], pa[(14 * w + 7 * s + i) % 40])
            for j in range(2):
                assert torch.equal(f[w, s, 7 + j], pb[(4 * w + 2 * s + j) % 6])
