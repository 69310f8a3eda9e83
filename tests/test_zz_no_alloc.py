"""nvfp4_quantize_noalloc (the allocation-free NVFP4 entry point, whose
in-library amax lives in the library's per-device scratch array) against
nvfp4_quantize with a caller workspace: codes, scales and tensor scale equal
byte for byte on two calls in a row, the second on a smaller input with a
smaller amax (a stale amax left in the shared scratch would change its
tensor scale), in every mode, with the amax computed and supplied."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
from _util import bf16_bits, need_gpu, say, to_gpu_bf16

pytestmark = pytest.mark.gpu

MODES = [F.NV_RTN, F.NV_RENORM_SR, F.NV_ELEMENT_SR]


def outputs(rows, cols, fill):
    dev = "cuda"
    return (torch.full((rows, cols // 2), fill, dtype=torch.uint8, device=dev),
            torch.full((rows, cols // 16), fill, dtype=torch.uint8, device=dev),
            torch.full((1,), float("nan"), dtype=torch.float32, device=dev))


def both(x, had, mode, amax_in):
    rows, cols = x.shape
    ref = outputs(rows, cols, 0xCD)
    ws = torch.zeros(F.nvfp4_workspace_bytes(rows, cols), dtype=torch.uint8, device=x.device)
    F.nvfp4_quantize(x, had, 5, mode, 7, amax_in=amax_in, codes=ref[0], scales=ref[1],
                     tensor_scale=ref[2], workspace=None if amax_in is not None else ws)
    got = outputs(rows, cols, 0xAB)
    F.nvfp4_quantize_noalloc(x, *got, had=had, sign_seed=5, mode=mode, sr_seed=7, amax_in=amax_in)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("supplied", [False, True])
def test_noalloc_equals_workspace_entry_point(mode, supplied):
    need_gpu()
    rng = np.random.default_rng(11 + mode)
    big = to_gpu_bf16(bf16_bits(rng.standard_t(4, (1024, 4096)) * 8.0))
    small = to_gpu_bf16(bf16_bits(rng.standard_t(4, (64, 256)) * 0.5))
    for name, x in (("first", big), ("second, smaller", small)):
        amax = None
        if supplied:
            amax = torch.tensor([float(x.float().abs().max()) * 1.25], dtype=torch.float32, device="cuda")
        say("nvfp4 noalloc", name, tuple(x.shape), "mode", mode, "amax supplied", supplied)
        ref, got = both(x, F.HAD_SIGNED, mode, amax)
        assert torch.equal(got[2].view(torch.int32), ref[2].view(torch.int32)), (name, got[2], ref[2])
        assert torch.equal(got[1], ref[1]), name
        assert torch.equal(got[0], ref[0]), name
    # the second call's tensor scale is its own amax's, not the first one's
    assert float(got[2]) < float(F.nvfp4_quantize(big, F.HAD_SIGNED, 5, mode, 7)[2])
