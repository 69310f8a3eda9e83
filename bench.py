"""Benchmark: MXFP4 Wgrad including the Hadamard rotation and quantization of
both operands, on the Llama-3.1-8B MLP gate/up layer (T = 8192 tokens,
N = 14336 out-features, K = 4096 in-features), on one MI355X.

A step is the whole hot path over one batch: rotate (deterministic
Hadamard-32 along tokens) and quantize dY[T, N] and X[T, K] to MXFP4 (RTN;
both operands in one fp4_wgrad_quantize launch), then dW[N, K] = dY^T X on
the scaled FP4 matrix cores, fp32 output.  Inputs
are synthetic bf16 tensors resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--settle-ms MS] [--flush]
                    [--workload gate_up|q_proj|down_proj]
                    [--variant det-rtn|signed-rtn|signed-rtn-perstep|sr]
                    [--no-cpu-baseline] [--no-mfma-ceiling] [--copy-calibration]
    python bench.py --counters FETCH_DIR WRITE_DIR     (no GPU: writes the summary)
    python bench.py --nvfp4                            (the secondary NVFP4 quantizer)
    python bench.py --layer [--workload W]             (the whole linear layer: three GEMMs)
    python bench.py --autograd [--workload W]          (MXFP4LinearFunction forward + backward, bf16)
    python bench.py --mfma-ceiling                     (only the MFMA-rate measurement aid)

Procedure: W warm-up steps and a 10-step probe, a host synchronization, then
with no host synchronization in between (the card must not idle before the
measured windows): back-to-back steps for --settle-ms of GPU time whatever W
is (reported as "settle"), the K timed steps between two events holding
nothing but their launches, with a clock-stamp kernel on either side
(timed_clock), and the per-kernel windows: K launches of each kernel back
to back between two events.  Prints one JSON line.
`value` is Wgrad TFLOP/s including quantization (2 T N K flops per step);
the roofline object describes the dominant kernel (the GEMM) from its
window (an event record between two launches opens a gap of about 5 us
before the second, so events around every launch would count that gap as
the kernel's); breakdown holds both kernels' windows, what the timed step
spends beyond them, and the card's device-to-device copy rate; --flush adds
passes with a 1 GiB write before each step, then before each kernel alone
(cold L2 and memory-side cache; median and minimum); cpu_baseline times the plain CPU oracle on a bounded sample of
the same workload and checks the last timed step's outputs against it
(timed_run_parity); mfma_ceiling is the scaled FP4 MFMA rate the card
sustains on random operands with no memory traffic at all
(libfp4calib.so), measured after the timed steps, and the shader clock it
ran at -- the bound the card's power limit puts on any GEMM on such data.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MXFP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 matrix peak
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "MXFP4 Wgrad TFLOPS incl. Hadamard+quantize (8192×14336×4096); quantizer GB/s"
COUNTERS = os.path.join(ROOT, "profiles", "gemm_mx_wgrad_gate_up_counters.json")
GEMM_SRC = os.path.join(ROOT, "fp4_precision_gemms_amd", "csrc", "gemm_mx.hip")


# Rotation and rounding of the Wgrad operands (the down_proj workload is
# specified under three of them): (hadamard, per-step sign seed, rounding,
# per-step SR seeds).  Per-step seeds change with the step index, as a
# training loop would pass them.
VARIANTS = {
    "det-rtn": ("deterministic-32", False, "rtn"),
    "signed-rtn": ("random-sign-32, fixed seed", False, "rtn"),
    "signed-rtn-perstep": ("random-sign-32, seed = step", True, "rtn"),
    "sr": ("none", False, "sr, seeds = step"),
}


def quant_bytes(elems: int) -> float:
    """Algorithmic bytes of one MXFP4 quantization: 2 B bf16 read, 0.5 B of
    codes and 1/32 B of scale written per element."""
    return elems * (2.0 + 0.5 + 1.0 / 32.0)


def traffic_per_launch(workload="gate_up", path=None):
    """HBM bytes per GEMM launch from the committed counter summary (taken
    on the gate/up Wgrad; `path` defaults to it), if it was taken on the
    current kernel source and `workload` is that shape; else None."""
    if workload != "gate_up":
        return None
    try:
        with open(path or COUNTERS) as f:
            rec = json.load(f)
        src = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
        if rec.get("gemm_source_sha256") == src:
            return float(rec["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def gapless_window(torch, dev, step, steps, settle_ms, after=None):
    """Times `steps` calls of `step` (warm-up already done): a 10-call probe
    of the call's duration and a host synchronization, then -- enqueued with
    no host synchronization between them, so the card does not idle before
    the window -- settle calls for about `settle_ms` of GPU time, the timed
    calls between two events on the current stream, and `after()` (another
    measured pass) if given; then a synchronization.  Returns (ms per timed
    call, settle calls, settle ms)."""
    t = time.perf_counter()
    for _ in range(10):
        step()
    torch.cuda.synchronize(dev)
    per = (time.perf_counter() - t) / 10
    n = int(settle_ms * 1e-3 / per) if settle_ms > 0 else 0
    s0, e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    s0.record()
    for _ in range(n):
        step()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    if after is not None:
        after()
    torch.cuda.synchronize(dev)
    return e0.elapsed_time(e1) / steps, n, s0.elapsed_time(e0)


COPY_BYTES = 256 << 20           # the calibration copy reads and writes this many bytes


def copy_calibration(torch, dev):
    """A plain elementwise copy of known size (float32 negation, 256 MiB read
    and 256 MiB written), launched a few times so that a counter run over
    this program sees it next to the GEMM: its FETCH_SIZE / WRITE_SIZE
    readings give the bytes-per-count factors of the two counters."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize(dev)


def counter_summary(fetch_dir, write_dir, out=None):
    """Reads the rocprofv3 counter CSVs of two runs of
        rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d DIR -o run --
            python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline
                --copy-calibration --no-mfma-ceiling
    and writes the calibrated HBM traffic per GEMM launch, with the GEMM
    source's hash, to `out` (default: the summary bench.py reads beside the
    kernel traces; the Markdown next to it is written by hand).  The copy
    kernel's readings (COPY_BYTES each way) give each counter's bytes per
    counted KiB."""
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter CSV under %s" % d)
        disp = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], f, r["Dispatch_Id"])
                disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"])
        out = {}
        for (k, _, _), v in disp.items():
            out.setdefault(k, []).append(v)
        return out

    def pick(table, needle):
        hits = {k: v for k, v in table.items() if needle in k}
        if len(hits) != 1:
            raise SystemExit("expected one kernel matching %r, found %s" % (needle, list(hits)))
        (name, vals), = hits.items()
        return name, sum(vals) / len(vals), len(vals)

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    gname, g_fetch, nf = pick(fetch, "gemm_mx_tn")
    _, g_write, nw = pick(write, "gemm_mx_tn")
    cname, c_fetch, _ = pick(fetch, "neg")
    _, c_write, _ = pick(write, "neg")
    f_fetch = COPY_BYTES / (c_fetch * 1024.0)        # counters are in KiB
    f_write = COPY_BYTES / (c_write * 1024.0)
    rd, wr = g_fetch * 1024.0 * f_fetch, g_write * 1024.0 * f_write
    rec = {"kernel": gname, "dispatches": [nf, nw],
           "gemm_fetch_kib": g_fetch, "gemm_write_kib": g_write,
           "copy_kernel": cname, "copy_bytes_each_way": COPY_BYTES,
           "copy_fetch_kib": c_fetch, "copy_write_kib": c_write,
           "fetch_factor": f_fetch, "write_factor": f_write,
           "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
           "hbm_bytes_per_launch": rd + wr,
           "gemm_source_sha256": hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()}
    with open(out or COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    return 0


def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def untile_codes(t, R):
    """The library's 32-row tiled MXFP4 codes [ceil(R/32), C/32, 512] ->
    row-major [R, C/2] (layout only)."""
    G, nb, _ = t.shape
    return t.reshape(G, nb, 32, 16).transpose(0, 2, 1, 3).reshape(G * 32, nb * 16)[:R]


def ungroup_scales(g, nb):
    """k-grouped scales [ceil(nb/8), R, 8] -> row-major [R, nb] (layout only)."""
    G, R, _ = g.shape
    return g.transpose(1, 0, 2).reshape(R, G * 8)[:, :nb]


def step_settings(variant, i):
    """(hadamard name, sign seed, rounding name, SR seeds) of step i."""
    had_name, per_step_sign, rnd_name = VARIANTS[variant]
    sign_seed = 1000 + i if per_step_sign else 7
    seeds = (2 * i + 1, 2 * i + 2) if rnd_name.startswith("sr") else (0, 0)
    return had_name, sign_seed, rnd_name, seeds


def cpu_baseline(w, dY, X, variant="det-rtn", timed=None):
    """The oracle, untuned, on a bounded sample of the same Wgrad: the full
    rotation + MXFP4 quantization of dY and X along tokens (the variant's
    transform and rounding, step 0's seeds), then as many of dW's rows by
    the binary64 oracle GEMM as about 10 s allow (256 at a time), scaled to
    all rows.  Returns the JSON object.

    `timed` = (step index, dY^T codes, dY^T scales, X^T codes, X^T scales,
    dW) copied to the host right after the timed steps: its codes and scales
    are compared whole with the oracle's quantization under that step's
    seeds, and 4096 entries of dW (corners, every 224/256-row tile edge,
    random) with the oracle's binary64 product (|err| <= 1e-5 sum |a b|),
    reported as "timed_run_parity"."""
    import numpy as np
    import oracle as O

    def settings(i):
        had_name, sign_seed, rnd_name, seeds = step_settings(variant, i)
        had = {"deterministic-32": O.HAD_DET, "none": O.HAD_NONE}.get(had_name, O.HAD_SIGNED)
        rnd = O.RND_SR if rnd_name.startswith("sr") else O.RND_RTN
        return had_name, had, sign_seed, rnd_name, rnd, seeds

    had_name, had, sign_seed, rnd_name, rnd, seeds = settings(0)
    t0 = time.perf_counter()
    aq, as_ = O.quant_mx(dY, O.AXIS_ROWS, 32, had, sign_seed, rnd, seeds[0])
    bq, bs = O.quant_mx(X, O.AXIS_ROWS, 32, had, sign_seed, rnd, seeds[1])
    t1 = time.perf_counter()
    # dW rows in chunks of 256 until about 10 s of GEMM work
    n = 0
    while n < w.N and time.perf_counter() - t1 < 10.0:
        O.gemm_rows(aq, as_, bq, bs, n, min(n + 256, w.N))
        n = min(n + 256, w.N)
    t2 = time.perf_counter()
    t_full = (t1 - t0) + (t2 - t1) * w.N / n
    flops = 2.0 * w.T * w.N * w.K
    out = {"value": flops / t_full / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(),
           "cpu_model": cpu_model(), "kind": "oracle",
           "sample": "rotation (%s) + MXFP4 quantization (%s) of all of dY[%d x %d] and X[%d x %d] "
                     "along tokens (%.1f s), then %d of %d dW rows by the binary64 oracle GEMM "
                     "(%.1f s), GEMM time scaled by rows to the full layer (%.0f s total)"
                     % (had_name, rnd_name, w.T, w.N, w.T, w.K, t1 - t0, n, w.N, t2 - t1, t_full)}
    if timed is not None:
        i, gq_dy, gs_dy, gq_x, gs_x, gdw = timed
        _, had_i, sign_i, _, rnd_i, seeds_i = settings(i)
        if (had_i, sign_i, rnd_i, seeds_i) != (had, sign_seed, rnd, seeds):
            aq, as_ = O.quant_mx(dY, O.AXIS_ROWS, 32, had_i, sign_i, rnd_i, seeds_i[0])
            bq, bs = O.quant_mx(X, O.AXIS_ROWS, 32, had_i, sign_i, rnd_i, seeds_i[1])
        nb = w.T // 32
        codes_ok = bool(np.array_equal(untile_codes(gq_dy, w.N), aq) and
                        np.array_equal(untile_codes(gq_x, w.K), bq))
        scales_ok = bool(np.array_equal(ungroup_scales(gs_dy, nb), as_) and
                         np.array_equal(ungroup_scales(gs_x, nb), bs))
        rng = np.random.default_rng(1)
        M, N = w.N, w.K

        def edges(n):
            # both sides of every 224- and 256-wide tile boundary, and the ends
            return np.array(sorted({0, n - 1} | {e for t in (224, 256) for k in range(1, n // t + 1)
                                                 for e in (k * t - 1, k * t) if e < n}))

        em, en = edges(M), edges(N)
        nr = 4096 - em.size - en.size - 4
        mi = np.concatenate([em, rng.integers(0, M, en.size), rng.integers(0, M, nr), [0, 0, M - 1, M - 1]])
        ni = np.concatenate([rng.integers(0, N, em.size), en, rng.integers(0, N, nr), [0, N - 1, 0, N - 1]])
        ref, mag = O.gemm_entries(aq, as_, bq, bs, mi, ni)
        err = np.abs(gdw[mi, ni].astype(np.float64) - ref)
        out["timed_run_parity"] = {
            "step": i, "codes_bitexact": codes_ok, "scales_bitexact": scales_ok,
            "dw_entries": int(mi.size), "dw_within_1e-5_sum_abs": bool((err <= 1e-5 * mag).all()),
            "dw_max_err_over_sum_abs": float((err / np.maximum(mag, 1e-300)).max()),
            "what": "the last timed step's dY^T and X^T codes and scales, whole, against the oracle "
                    "under that step's seeds; 4096 dW entries against the binary64 oracle product"}
    return out


def nvfp4_bench(args) -> int:
    """The secondary kernel: NVFP4 quantization of the [16384 x 8192]
    Student-t (nu = 4) tensor with the random-sign Hadamard-16 and the renorm
    folded into the E4M3 scales by SR, the tensor amax computed in-library
    (two passes) and supplied (one pass); beside it the element-SR mode (one
    pass).  One JSON line; HBM roofline over algorithmic bytes (2.5625
    B/element, +2 B/element for the amax pass)."""
    import numpy as np
    import torch

    import fp4_precision_gemms_amd as F
    import workloads as W

    w = W.WORKLOADS["nvfp4"]
    rows, cols = w.T, w.K
    dev = torch.device("cuda:0")
    bits = W.tensor(w, "x")
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(F.nvfp4_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
    F.nvfp4_quantize(x, F.HAD_SIGNED, 7, F.NV_RENORM_SR, 11, codes=codes, scales=scales, tensor_scale=ts,
                     workspace=ws)
    amax = (ts * 2688.0).contiguous()          # the amax the first call found, for the one-pass run

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize(dev)
        return gapless_window(torch, dev, fn, args.steps, args.settle_ms)[0]

    el = rows * cols
    t2 = timed(lambda: F.nvfp4_quantize(x, F.HAD_SIGNED, 7, F.NV_RENORM_SR, 11, codes=codes, scales=scales,
                                        tensor_scale=ts, workspace=ws))
    t1 = timed(lambda: F.nvfp4_quantize(x, F.HAD_SIGNED, 7, F.NV_RENORM_SR, 11, amax_in=amax, codes=codes,
                                        scales=scales, tensor_scale=ts))
    te = timed(lambda: F.nvfp4_quantize(x, F.HAD_SIGNED, 7, F.NV_ELEMENT_SR, 11, amax_in=amax,
                                        codes=codes, scales=scales, tensor_scale=ts))
    b1, b2 = el * (2 + 0.5 + 1 / 16), el * (2 + 0.5 + 1 / 16 + 2)
    g2, g1, ge = b2 / (t2 * 1e-3) / 1e9, b1 / (t1 * 1e-3) / 1e9, b1 / (te * 1e-3) / 1e9
    print(json.dumps({
        "metric": "NVFP4 quantize GB/s (16384x8192, SIGNED-16, renorm by SR, amax in-library)",
        "value": g2, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t2, "higher_is_better": True, "dtype": "bf16->nvfp4", "data": "synthetic",
        "config": {"workload": "nvfp4 [16384x8192] Student-t nu=4", "had": "signed-16", "renorm": 1},
        "roofline": {"bound": "hbm", "achieved": g2, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": g2 / HBM_PEAK_GBS, "traffic": None},
        "one_pass_amax_in": {"ms": t1, "GBps": g1, "frac_hbm": g1 / HBM_PEAK_GBS},
        "element_sr_one_pass": {"ms": te, "GBps": ge, "frac_hbm": ge / HBM_PEAK_GBS}}), flush=True)
    return 0


def layer_bench(args) -> int:
    """The whole MXFP4 linear layer on the gate/up shape: X[T, K], W[N, K]
    and dY[T, N] each quantized once per direction by the dual quantizer
    (rows: along the first axis, Hadamard-32 on the Wgrad operands X and dY;
    cols: along the second axis, no rotation), then Fprop Y = X W^T, Dgrad
    dX = dY W and Wgrad dW = dY^T X through the role entry points (fp32
    outputs).  One JSON line: 3 * 2 T N K flops over the step, and each
    launch's average time over K launches of it back to back between two
    HIP events."""
    import numpy as np
    import torch

    import fp4_precision_gemms_amd as F
    import workloads as W

    w = W.WORKLOADS[args.workload]
    T, N, K = w.T, w.N, w.K
    dev = torch.device("cuda:0")
    up = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    X, Wt, dY = up(W.tensor(w, "X")), up(W.tensor(w, "W")), up(W.tensor(w, "dY"))

    def bufs(rows, cols):
        shapes = F.mx_shapes(rows, cols, F.AXIS_ROWS) + F.mx_shapes(rows, cols, F.AXIS_COLS)
        return [torch.empty(sh, dtype=torch.uint8, device=dev) for sh in shapes]

    qx, qw, qdy = bufs(T, K), bufs(N, K), bufs(T, N)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    dx = torch.empty((T, K), dtype=torch.float32, device=dev)
    dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    launches = [
        ("quant_X_dual", lambda: F.fp4_hadamard_quantize_dual(X, 32, F.HAD_DET, out=qx)),
        ("quant_W_dual", lambda: F.fp4_hadamard_quantize_dual(Wt, 32, F.HAD_NONE, out=qw)),
        ("quant_dY_dual", lambda: F.fp4_hadamard_quantize_dual(dY, 32, F.HAD_DET, out=qdy)),
        ("fprop", lambda: F.fp4_gemm_fprop(qx[2], qx[3], qw[2], qw[3], out=y)),
        ("dgrad", lambda: F.fp4_gemm_dgrad(qdy[2], qdy[3], qw[0], qw[1], out=dx)),
        ("wgrad", lambda: F.fp4_gemm_wgrad(qdy[0], qdy[1], qx[0], qx[1], out=dw)),
    ]

    def step():
        for _, fn in launches:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    # per-launch times: each launch K times back to back between two events,
    # right behind the timed steps (events around every launch would count
    # the gap an event record opens before the next launch)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]

    def windows():
        for (a, b), (_, fn) in zip(ev, launches):
            a.record()
            for _ in range(args.steps):
                fn()
            b.record()

    ms, settle_steps, settle_ms = gapless_window(torch, dev, step, args.steps, args.settle_ms, windows)
    per = {name: 1e3 * ev[j][0].elapsed_time(ev[j][1]) / args.steps for j, (name, _) in enumerate(launches)}
    flop = 2.0 * T * N * K
    qbytes = {"quant_X_dual": T * K * (2 + 1 + 1 / 16), "quant_W_dual": N * K * (2 + 1 + 1 / 16),
              "quant_dY_dual": T * N * (2 + 1 + 1 / 16)}
    breakdown = {}
    for name, us in per.items():
        breakdown[name + "_us"] = us
        if name in qbytes:
            breakdown[name + "_GBps"] = qbytes[name] / (us * 1e-6) / 1e9
        else:
            breakdown[name + "_TFLOPs"] = flop / (us * 1e-6) / 1e12
    gemm_us = min(per["fprop"], per["dgrad"], per["wgrad"])
    print(json.dumps({
        "metric": "MXFP4 linear layer TFLOP/s (Fprop + Dgrad + Wgrad incl. dual quantization, %dx%dx%d)" % (T, N, K),
        "value": 3 * flop / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "%s linear layer, all three GEMMs" % w.name, "T": T, "N": N, "K": K,
                   "hadamard": "deterministic-32 on the Wgrad operands", "rounding": "rtn",
                   "outputs": "fp32"},
        "roofline": {"bound": "mfma", "kernel": "gemm_mx_tn (fastest of the three roles)",
                     "achieved": flop / (gemm_us * 1e-6) / 1e12, "peak": MXFP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flop / (gemm_us * 1e-6) / 1e12 / MXFP4_PEAK_TFLOPS,
                     "traffic": None},
        "settle": {"steps": settle_steps, "ms": settle_ms},
        "step_minus_launches_us": ms * 1e3 - sum(per.values()),
        "breakdown": breakdown}), flush=True)
    return 0


def autograd_bench(args) -> int:
    """The linear layer as training uses it: MXFP4LinearFunction forward
    (Y = X W^T) and backward (dX, dW) through torch autograd on the
    workload's shapes, bf16 inputs and outputs, deterministic Hadamard-32 on
    the Wgrad operands, RTN.  A step = forward + backward with a fixed
    upstream gradient dY; 3 * 2 T N K flops per step.  One JSON line."""
    import numpy as np
    import torch

    from fp4_precision_gemms_amd.linear import MXFP4LinearFunction
    import fp4_precision_gemms_amd as F
    import workloads as W

    w = W.WORKLOADS[args.workload]
    T, N, K = w.T, w.N, w.K
    dev = torch.device("cuda:0")
    up = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    x = up(W.tensor(w, "X")).requires_grad_(True)
    wt = up(W.tensor(w, "W")).requires_grad_(True)
    dy = up(W.tensor(w, "dY"))

    def step():
        y = MXFP4LinearFunction.apply(x, wt, F.HAD_DET, 32, 0, F.RTN, 0)
        x.grad = None
        wt.grad = None
        y.backward(dy)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    ms, settle_steps, settle_ms = gapless_window(torch, dev, step, args.steps, args.settle_ms)
    flop = 3 * 2.0 * T * N * K
    print(json.dumps({
        "metric": "MXFP4 linear layer training step TFLOP/s (autograd forward + backward, %dx%dx%d)" % (T, N, K),
        "value": flop / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "%s MXFP4LinearFunction forward + backward" % w.name, "T": T, "N": N, "K": K,
                   "hadamard": "deterministic-32 on the Wgrad operands", "rounding": "rtn",
                   "outputs": "bf16 Y, dX, dW"},
        "settle": {"steps": settle_steps, "ms": settle_ms}}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 warm-up steps, the settle stretch, then 100 timed steps (about 30 ms)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="gate_up", choices=["gate_up", "q_proj", "down_proj"])
    ap.add_argument("--variant", default="det-rtn", choices=sorted(VARIANTS),
                    help="rotation and rounding of the Wgrad operands")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="steps run back to back before timing, whatever --warmup is, until this many "
                         "milliseconds have passed (the card's clocks settle under sustained load)")
    ap.add_argument("--flush", action="store_true",
                    help="also time each step after a 1 GiB write that flushes L2 and the memory-side "
                         "cache; reports the median and minimum")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB copy kernel (counter calibration)")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 counter runs and exit")
    ap.add_argument("--nvfp4", action="store_true", help="time the NVFP4 quantizer instead")
    ap.add_argument("--layer", action="store_true", help="time the whole linear layer instead")
    ap.add_argument("--autograd", action="store_true",
                    help="time MXFP4LinearFunction forward + backward instead")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the MFMA-only rate on random operands (libfp4calib.so)")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="leave the MFMA-only measurement out of the default run")
    args = ap.parse_args()
    if args.counters:
        return counter_summary(*args.counters)
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    if args.nvfp4:
        return nvfp4_bench(args)
    if args.layer:
        return layer_bench(args)
    if args.autograd:
        return autograd_bench(args)
    if args.mfma_ceiling:
        import torch
        from fp4_precision_gemms_amd import calib
        print(json.dumps({"mfma_ceiling": calib.mfma_ceiling(torch.device("cuda:0")),
                          "peak_TFLOPs": MXFP4_PEAK_TFLOPS}), flush=True)
        return 0

    import numpy as np
    import torch

    import fp4_precision_gemms_amd as F
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    F.lib()
    w = W.WORKLOADS[args.workload]
    T, N, K = w.T, w.N, w.K
    dev = torch.device("cuda:0")
    dY_np, X_np = W.tensor(w, "dY"), W.tensor(w, "X")

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    dY, X = up(dY_np), up(X_np)
    (cq, cs) = F.mx_shapes(T, N, F.AXIS_ROWS)
    dytq = torch.empty(cq, dtype=torch.uint8, device=dev)
    dyts = torch.empty(cs, dtype=torch.uint8, device=dev)
    (cq, cs) = F.mx_shapes(T, K, F.AXIS_ROWS)
    xtq = torch.empty(cq, dtype=torch.uint8, device=dev)
    xts = torch.empty(cs, dtype=torch.uint8, device=dev)
    dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    had_name, per_step_sign, rnd_name = VARIANTS[args.variant]
    had = {"deterministic-32": F.HAD_DET, "none": F.HAD_NONE}.get(had_name, F.HAD_SIGNED)
    rnd = F.SR if rnd_name.startswith("sr") else F.RTN
    counter = [0]

    def step():
        # both Wgrad operands (one rotation, one launch), then the GEMM
        i = counter[0]
        counter[0] += 1
        _, sign_seed, _, (sr_dy, sr_x) = step_settings(args.variant, i)
        F.fp4_wgrad_quantize(dY, X, 32, had, sign_seed, rnd, sr_dy, sr_x, out=(dytq, dyts, xtq, xts))
        F.fp4_gemm_wgrad(dytq, dyts, xtq, xts, out=dw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    # settle: back-to-back steps for a fixed stretch of GPU time, whatever
    # --warmup is (the first tens of milliseconds of load run at other
    # clocks).  The step count comes from a short probe; the settle steps,
    # the timed steps and the per-kernel windows are then enqueued with no host
    # synchronization between them, so the card never idles before or
    # between the measured windows (after even a short idle the next few
    # milliseconds run slower, which a 20-step window would measure).
    t_probe = time.perf_counter()
    for _ in range(10):
        step()
    torch.cuda.synchronize(dev)
    per_step_s = (time.perf_counter() - t_probe) / 10
    settle_steps = int(args.settle_ms * 1e-3 / per_step_s) if args.settle_ms > 0 else 0
    from fp4_precision_gemms_amd import calib
    span = calib.ClockSpan(dev, stream)
    # everything the measured sequence uses is allocated before it starts
    snap = None
    if not args.no_cpu_baseline:
        snap = [torch.empty_like(t) for t in (dytq, dyts, xtq, xts, dw)]
    # each kernel's window: its launch K times back to back (the quantizer
    # with the first step's seeds, the GEMM on the last step's operands)
    _, q_sign, _, (q_sr_dy, q_sr_x) = step_settings(args.variant, 0)
    kernels = [("quant", lambda: F.fp4_wgrad_quantize(dY, X, 32, had, q_sign, rnd, q_sr_dy, q_sr_x,
                                                      out=(dytq, dyts, xtq, xts))),
               ("gemm", lambda: F.fp4_gemm_wgrad(dytq, dyts, xtq, xts, out=dw))]
    win = {name: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for name, _ in kernels}
    s0 = torch.cuda.Event(enable_timing=True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(settle_steps):
        step()
    # the timed steps: nothing but the two launches per step (an event record
    # between launches costs about 3 % of the step); one clock-stamp kernel
    # before and after, outside the events
    span.begin()
    start.record(stream)
    for i in range(args.steps):
        step()
    stop.record(stream)
    span.end()
    last_timed = counter[0] - 1
    # the last timed step's outputs, kept on the device for the parity check
    if snap is not None:
        for d, t in zip(snap, (dytq, dyts, xtq, xts, dw)):
            d.copy_(t)
    # per-kernel launch durations: K launches of each back to back between
    # two events on the launch stream, still without a host synchronization
    for name, fn in kernels:
        win[name][0].record(stream)
        for _ in range(args.steps):
            fn()
        win[name][1].record(stream)
    torch.cuda.synchronize(dev)
    settle_ms = s0.elapsed_time(start)
    ms_step = start.elapsed_time(stop) / args.steps
    sclk = span.ghz()
    timed = None
    if snap is not None:
        timed = (last_timed, *(t.cpu().numpy() for t in snap))
        del snap

    t_q, t_gemm = (win[name][0].elapsed_time(win[name][1]) / args.steps for name, _ in kernels)
    flops = 2.0 * T * N * K
    gemm_tflops = flops / (t_gemm * 1e-3) / 1e12
    q_bytes = quant_bytes(T * N) + quant_bytes(T * K)
    q_gbs = q_bytes / (t_q * 1e-3) / 1e9

    # the box's device-to-device copy rate (512 MiB each way), the practical
    # ceiling of a read-once write-once kernel
    csrc = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    for _ in range(3):
        cdst.copy_(csrc)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize(dev)
    copy_gbs = 2.0 * csrc.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst
    flushed = None
    if args.flush:
        # each measured call after a 1 GiB write (evicts L2 and the 256 MB
        # memory-side cache), HIP events at its two ends only: the whole
        # step, then each kernel in a loop of its own
        fbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        import statistics

        def cold(fn):
            times = []
            for _ in range(args.steps):
                fbuf.zero_()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize(dev)
                times.append(e0.elapsed_time(e1))
            return statistics.median(times), min(times)

        st_med, st_min = cold(step)
        q_med, q_min = cold(kernels[0][1])
        g_med, g_min = cold(kernels[1][1])
        del fbuf
        flushed = {"steps": args.steps, "flush_bytes": 1 << 30,
                   "step_ms_median": st_med, "step_ms_min": st_min,
                   "quant_ms_median": q_med, "quant_ms_min": q_min,
                   "gemm_ms_median": g_med, "gemm_ms_min": g_min}
    traffic = traffic_per_launch(w.name)
    out = {
        "metric": METRIC if (w.name, args.variant) == ("gate_up", "det-rtn") else
                  "MXFP4 Wgrad TFLOPS incl. rotation+quantize (%dx%dx%d, %s)" % (T, N, K, args.variant),
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "%s Wgrad incl. rotation + MXFP4 quantize" % w.name,
                   "T": T, "N": N, "K": K, "hadamard": had_name + " along tokens",
                   "rounding": rnd_name, "output": "fp32 dW[N,K]"},
        "roofline": {"bound": "mfma", "kernel": "gemm_mx_tn (Wgrad)",
                     "achieved": gemm_tflops, "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": gemm_tflops / MXFP4_PEAK_TFLOPS, "traffic": traffic},
        "settle": {"steps": settle_steps, "ms": settle_ms,
                   "what": "back-to-back steps right before the timed ones (GPU time), whatever --warmup is; "
                           "settle, timed steps and the per-kernel windows run with no host synchronization "
                           "between them"},
        "timed_clock": {"sclk_GHz": sclk,
                        "what": "shader clock counter (s_memtime) against the 100 MHz reference "
                                "(s_memrealtime) between clock-stamp launches on either side of the "
                                "timed steps, median over the XCDs; under the power limit the matrix "
                                "cores' rate is not proportional to it (measured: equal kernel times "
                                "at rates 13 % apart)"},
        "breakdown": {"quant_dY_X_ms": t_q, "gemm_ms": t_gemm,
                      "step_minus_kernels_ms": ms_step - t_q - t_gemm,
                      "what": "each kernel's average launch time over K launches of it back to back "
                              "between two events on the launch stream, right after the timed steps; "
                              "step_minus_kernels: what a timed step takes beyond the two",
                      "quantizer_GBps": q_gbs, "quantizer_frac_hbm": q_gbs / HBM_PEAK_GBS,
                      "d2d_copy_GBps": copy_gbs, "quantizer_frac_copy": q_gbs / copy_gbs,
                      "gemm_TFLOPs": gemm_tflops,
                      "gemm_frac_of_peak_at_timed_sclk": gemm_tflops / (MXFP4_PEAK_TFLOPS * sclk / 2.4)},
    }
    if flushed is not None:
        out["flushed"] = flushed
    if not args.no_mfma_ceiling:
        from fp4_precision_gemms_amd import calib
        ceil = calib.mfma_ceiling(dev)
        ceil["frac_of_peak"] = ceil["value"] / MXFP4_PEAK_TFLOPS
        ceil["gemm_frac_of_ceiling"] = gemm_tflops / ceil["value"]
        # the same loop on this product's own quantized operands (fragments of
        # dY^T and X^T as the GEMM reads them): the matrix cores' power, hence
        # their rate under the power limit, depends on the operand bits
        own = calib.mfma_ceiling(dev, operands=(dytq, xtq))
        ceil["on_operands"] = {"value": own["value"], "sclk_GHz": own["sclk_GHz"],
                               "frac_of_peak": own["value"] / MXFP4_PEAK_TFLOPS,
                               "gemm_frac_of_ceiling": gemm_tflops / own["value"],
                               "what": own["what"]}
        out["mfma_ceiling"] = ceil
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, dY_np, X_np, args.variant, timed)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
