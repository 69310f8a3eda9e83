"""The hand-worked MXFP4 blocks of tests/golden/mxfp4_single_blocks.txt
(derivations and citation in the file's header) against the oracle (CPU) and
against the HIP quantizers (GPU), along both block axes."""
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mxfp4_single_blocks.txt")
HAD = {"none": O.HAD_NONE, "det": O.HAD_DET}


def load_golden():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, inputs = line.split("|")
        cid, had, n, scale, codes = head.split()
        bits = np.array([int(h, 16) for h in inputs.split()], dtype=np.uint16)
        assert bits.size == 32, cid
        cases.append((cid, HAD[had], int(n), int(scale, 16), bytes.fromhex(codes), bits))
    return cases


CASES = load_golden()


def test_golden_file_has_every_case():
    assert [c[0] for c in CASES] == ["E1", "E2a", "E2b", "E3a", "E3b", "E4", "E5", "E6a", "E6b"]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_oracle_matches_golden(case):
    cid, had, n, scale, codes, bits = case
    c, s = O.quant_mx(bits[None, :], O.AXIS_COLS, n, had)
    assert s[0, 0] == scale and bytes(c[0]) == codes
    # the same block along rows (a [32, 1] column) gives the same bytes
    c, s = O.quant_mx(np.ascontiguousarray(bits[:, None]), O.AXIS_ROWS, n, had)
    assert s[0, 0] == scale and bytes(c[0]) == codes


@pytest.mark.gpu
def test_hip_quantizers_match_golden():
    """Every golden block, tiled into a [9 blocks x 8 copies] matrix along
    each axis (so the tiled kernels see them in several lanes and tiles)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_precision_gemms_amd as F
    from _util import say, sentinel_u8, to_gpu_bf16, ungroup_scales, untile_codes

    for had_name, had in HAD.items():
        sel = [c for c in CASES if c[1] == had]
        blocks = np.stack([c[5] for c in sel])                       # [nb, 32]
        reps = 8
        along_cols = np.ascontiguousarray(np.repeat(blocks, reps, axis=0))       # [nb*reps, 32]
        along_rows = np.ascontiguousarray(along_cols.T)                           # [32, nb*reps]
        for axis, x in ((F.AXIS_COLS, along_cols), (F.AXIS_ROWS, along_rows)):
            say("golden", had_name, "axis", axis, x.shape)
            cs, ss = F.mx_shapes(x.shape[0], x.shape[1], axis)
            codes, scales = sentinel_u8(cs), sentinel_u8(ss)
            F.fp4_hadamard_quantize(to_gpu_bf16(x), axis, 32, {O.HAD_NONE: F.HAD_NONE,
                                    O.HAD_DET: F.HAD_DET}[had], 0, F.RTN, 0, codes, scales)
            torch.cuda.synchronize()
            codes = untile_codes(codes.cpu().numpy(), len(sel) * reps)
            scales = ungroup_scales(scales.cpu().numpy(), 1)
            for i, (cid, _, _, scale, want, _) in enumerate(sel):
                for r in range(reps):
                    row = i * reps + r
                    assert scales[row, 0] == scale, (cid, axis, scales[row, 0], scale)
                    assert bytes(codes[row]) == want, (cid, axis)
