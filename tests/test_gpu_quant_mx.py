"""GPU parity of fp4_hadamard_quantize against the oracle: codes and scales
bit-exact, on ragged small shapes, edge-case blocks, the workload
distributions, and the full Llama-3.1-8B-shaped operands (sampled rows).
Outputs are pre-filled with 0xCD so an unwritten byte shows as a mismatch."""
import numpy as np
import pytest
import torch

import fp4_precision_gemms_amd as F
import oracle as O
import workloads as W
from _util import bf16_bits, need_gpu, say, sentinel_u8, to_gpu_bf16, ungroup_scales, untile_codes

pytestmark = pytest.mark.gpu

HADS = [(O.HAD_NONE, 32), (O.HAD_DET, 32), (O.HAD_SIGNED, 32), (O.HAD_DET, 16), (O.HAD_SIGNED, 16)]
# oracle enum -> library enum (values happen to coincide; mapped explicitly)
AX = {O.AXIS_COLS: F.AXIS_COLS, O.AXIS_ROWS: F.AXIS_ROWS}
HD = {O.HAD_NONE: F.HAD_NONE, O.HAD_DET: F.HAD_DET, O.HAD_SIGNED: F.HAD_SIGNED}
RN = {O.RND_RTN: F.RTN, O.RND_SR: F.SR}


def gpu_quant(bits, axis, had, had_n, rnd, sign_seed=0, sr_seed=0):
    need_gpu()
    x = to_gpu_bf16(bits)
    rows, cols = bits.shape
    cs, ss = F.mx_shapes(rows, cols, AX[axis])
    codes, scales = sentinel_u8(cs), sentinel_u8(ss)
    F.fp4_hadamard_quantize(x, AX[axis], had_n, HD[had], sign_seed, RN[rnd], sr_seed, codes, scales)
    torch.cuda.synchronize()
    g = scales.cpu().numpy()
    nb = (cols if axis == O.AXIS_COLS else rows) // 32
    # the padding of the last k-group is never written
    tail = g[-1, :, nb - 8 * (g.shape[0] - 1):]
    assert (tail == 0xCD).all(), "quantizer wrote the scale padding"
    R = rows if axis == O.AXIS_COLS else cols
    return untile_codes(codes.cpu().numpy(), R), ungroup_scales(g, nb)


def assert_same(got, ref, what):
    gc, gs = got
    rc, rs = ref
    if not np.array_equal(gs, rs):
        i = np.argwhere(gs != rs)[:5]
        raise AssertionError("%s: %d scale bytes differ, first at %s: gpu %s oracle %s"
                             % (what, (gs != rs).sum(), i.tolist(), gs[tuple(i.T)], rs[tuple(i.T)]))
    if not np.array_equal(gc, rc):
        i = np.argwhere(gc != rc)[:5]
        raise AssertionError("%s: %d code bytes differ, first at %s: gpu %s oracle %s"
                             % (what, (gc != rc).sum(), i.tolist(), gc[tuple(i.T)], rc[tuple(i.T)]))


def check(bits, axis, had, had_n, rnd, sign_seed=0, sr_seed=0, what=""):
    say("quant", what, bits.shape, "axis", axis, "had", had, had_n, "rnd", rnd)
    got = gpu_quant(bits, axis, had, had_n, rnd, sign_seed, sr_seed)
    ref = O.quant_mx(bits, axis, had_n, had, sign_seed, rnd, sr_seed)
    assert_same(got, ref, what)


SHAPES = [
    (O.AXIS_COLS, 96, 160), (O.AXIS_COLS, 5, 32), (O.AXIS_COLS, 333, 1024),
    (O.AXIS_ROWS, 96, 37), (O.AXIS_ROWS, 96, 38), (O.AXIS_ROWS, 160, 100),
    (O.AXIS_ROWS, 32, 1), (O.AXIS_ROWS, 1056, 300), (O.AXIS_ROWS, 544, 1032),
]


@pytest.mark.parametrize("axis,rows,cols", SHAPES)
@pytest.mark.parametrize("had,had_n", HADS)
@pytest.mark.parametrize("rnd", [O.RND_RTN, O.RND_SR])
def test_quant_parity_shapes(axis, rows, cols, had, had_n, rnd):
    rng = np.random.default_rng(rows * 7 + cols)
    v = rng.standard_t(3, (rows, cols)) * np.exp(rng.uniform(-4, 4, (rows, 1)))
    check(bf16_bits(v), axis, had, had_n, rnd, sign_seed=1234, sr_seed=99,
          what="shape %s" % ((rows, cols),))


def edge_matrix():
    """Rows of 32-element blocks with the cases the method has: zeros, -0,
    subnormals, every rounding midpoint at several exponents, values that
    saturate, NaN, infinities, transform overflow, huge and tiny scales."""
    mids = [.25, .75, 1.25, 1.75, 2.5, 3.5, 5, 7, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, -7,
            .5, 1, 1.5, 2, 3, 4, 6, 0, .125, .375, 2.875, 4.875, 5.125, -6.5, .625, 1.375]
    blocks = [np.zeros(32), -np.zeros(32), np.full(32, 1.0), np.eye(32)[0], np.eye(32)[1]]
    for k in (-130, -126, -100, -3, 0, 5, 60, 120, 126):
        blocks.append(np.array(mids) * 2.0 ** k)
    sub = np.zeros(32)
    sub[0] = 2.0 ** -127
    sub[5] = -2.0 ** -133
    blocks.append(sub)
    sat = np.linspace(-7.9, 7.9, 32)
    sat[0] = 4.0
    blocks.append(sat)
    nanb = np.ones(32)
    nanb[7] = np.nan
    blocks.append(nanb)
    infb = np.ones(32)
    infb[30] = -np.inf
    blocks.append(infb)
    blocks.append(np.full(32, 3.0e38))                  # overflows inside the transform
    blocks.append(np.array([3.0e38, -3.0e38] * 16))
    blocks.append(np.full(32, 1e-38))
    rng = np.random.default_rng(0)
    blocks.append(rng.standard_normal(32) * 1e-40)
    m = np.stack(blocks)                                # [nblocks, 32]
    return m


@pytest.mark.parametrize("had,had_n", HADS)
@pytest.mark.parametrize("rnd", [O.RND_RTN, O.RND_SR])
def test_quant_parity_edge_blocks(had, had_n, rnd):
    m = edge_matrix()
    with np.errstate(over="ignore", invalid="ignore"):
        bits = bf16_bits(m)
    # along cols: each row a block; along rows: the transpose, each column a block
    check(bits, O.AXIS_COLS, had, had_n, rnd, 7, 3, what="edge cols")
    check(np.ascontiguousarray(bits.T), O.AXIS_ROWS, had, had_n, rnd, 7, 3, what="edge rows")
    # several blocks per row, ragged number of rows
    wide = np.ascontiguousarray(bits[: bits.shape[0] // 3 * 3].reshape(-1, 96))
    check(wide, O.AXIS_COLS, had, had_n, rnd, 7, 3, what="edge wide")


def test_determinism_and_seeds():
    rng = np.random.default_rng(1)
    bits = bf16_bits(rng.standard_normal((256, 512)))
    a = gpu_quant(bits, O.AXIS_ROWS, O.HAD_SIGNED, 32, O.RND_SR, 5, 6)
    b = gpu_quant(bits, O.AXIS_ROWS, O.HAD_SIGNED, 32, O.RND_SR, 5, 6)
    c = gpu_quant(bits, O.AXIS_ROWS, O.HAD_SIGNED, 32, O.RND_SR, 5, 7)
    d = gpu_quant(bits, O.AXIS_ROWS, O.HAD_SIGNED, 32, O.RND_SR, 8, 6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    assert not np.array_equal(a[0], d[0])


SCALED = [W.scaled(W.WORKLOADS["q_proj"], 512, 384, 320),
          W.scaled(W.WORKLOADS["gate_up"], 544, 256, 448),
          W.scaled(W.WORKLOADS["down_proj"], 512, 448, 256)]


@pytest.mark.parametrize("w", [W.WORKLOADS["tiny_wgrad"]] + SCALED, ids=lambda w: w.name)
def test_quant_parity_workloads(w):
    # Wgrad operands: along tokens, the same rotation on both
    for name in ("dY", "X"):
        bits = W.tensor(w, name)
        check(bits, O.AXIS_ROWS, O.HAD_DET, 32, O.RND_RTN, what=w.name + " " + name)
        check(bits, O.AXIS_ROWS, O.HAD_SIGNED, 32, O.RND_RTN, 17, what=w.name + " " + name)
        check(bits, O.AXIS_ROWS, O.HAD_NONE, 32, O.RND_SR, 0, 31, what=w.name + " " + name)
    if "W" in w.dists:
        Wb = W.tensor(w, "W")
        check(W.tensor(w, "X"), O.AXIS_COLS, O.HAD_NONE, 32, O.RND_RTN, what=w.name + " X fprop")
        check(Wb, O.AXIS_COLS, O.HAD_NONE, 32, O.RND_RTN, what=w.name + " W fprop")
        check(W.tensor(w, "dY"), O.AXIS_COLS, O.HAD_NONE, 32, O.RND_RTN, what=w.name + " dY dgrad")
        check(Wb, O.AXIS_ROWS, O.HAD_NONE, 32, O.RND_RTN, what=w.name + " W dgrad")


FULL = [("gate_up", "dY", O.AXIS_ROWS, O.HAD_DET, O.RND_RTN),
        ("gate_up", "X", O.AXIS_ROWS, O.HAD_DET, O.RND_RTN),
        ("gate_up", "X", O.AXIS_COLS, O.HAD_NONE, O.RND_RTN),
        ("gate_up", "W", O.AXIS_ROWS, O.HAD_NONE, O.RND_RTN),
        ("down_proj", "X", O.AXIS_ROWS, O.HAD_SIGNED, O.RND_RTN),
        ("down_proj", "X", O.AXIS_ROWS, O.HAD_NONE, O.RND_SR)]


@pytest.mark.slow
@pytest.mark.parametrize("wname,tname,axis,had,rnd", FULL)
def test_quant_parity_full_size_sampled_rows(wname, tname, axis, had, rnd):
    """Full Llama-3.1-8B shapes through fp4_hadamard_quantize, the
    single-tensor entry point (the benchmark times fp4_wgrad_quantize, the
    pair launch, which test_gpu_full_size.py checks whole); the oracle
    recomputes three ranges of 64 logical rows (first, middle, last)."""
    w = W.WORKLOADS[wname]
    bits = W.tensor(w, tname)
    say("full quant", wname, tname, bits.shape)
    gc, gs = gpu_quant(bits, axis, had, 32, rnd, sign_seed=2024, sr_seed=11)
    R = gc.shape[0]
    for r0 in (0, R // 2 - 32, R - 64):
        rc, rs = O.quant_mx(bits, axis, 32, had, 2024, rnd, 11, r0=r0, r1=r0 + 64)
        assert_same((gc[r0:r0 + 64], gs[r0:r0 + 64]), (rc, rs), "%s %s rows %d" % (wname, tname, r0))


@pytest.mark.slow
def test_quant_input_over_2gib():
    """An input of 2^31 bytes or more: x[33024, 32768] bf16 (2.16 GB).  The
    transposed quantizer takes its 64-bit-indexed kernel and the dual entry
    point its two-launch fallback; three ranges of 32 logical rows of every
    output are recomputed by the oracle."""
    need_gpu()
    rows, cols = 33024, 32768
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((rows, cols), generator=g, device="cuda").to(torch.bfloat16)
    bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    assert bits.nbytes >= 2 ** 31
    say("quant over 2 GiB", rows, cols)
    codes, scales = F.fp4_hadamard_quantize(x, F.AXIS_ROWS, 32, F.HAD_DET, 0, F.RTN, 0)
    rq, rs, cq, cs = F.fp4_hadamard_quantize_dual(x, 32, F.HAD_SIGNED, 9, F.RTN, 0, 32, F.HAD_NONE)
    torch.cuda.synchronize()
    got = {
        "rows": (untile_codes(codes.cpu().numpy(), cols), ungroup_scales(scales.cpu().numpy(), rows // 32),
                 (O.AXIS_ROWS, O.HAD_DET, 0)),
        "dual rows": (untile_codes(rq.cpu().numpy(), cols), ungroup_scales(rs.cpu().numpy(), rows // 32),
                      (O.AXIS_ROWS, O.HAD_SIGNED, 9)),
        "dual cols": (untile_codes(cq.cpu().numpy(), rows), ungroup_scales(cs.cpu().numpy(), cols // 32),
                      (O.AXIS_COLS, O.HAD_NONE, 0)),
    }
    for what, (gc, gs, (axis, had, seed)) in got.items():
        R = gc.shape[0]
        for r0 in (0, R // 2 - 16, R - 32):
            rc, rsc = O.quant_mx(bits, axis, 32, had, seed, O.RND_RTN, 0, r0=r0, r1=r0 + 32)
            assert_same((gc[r0:r0 + 32], gs[r0:r0 + 32]), (rc, rsc), "%s rows %d" % (what, r0))
