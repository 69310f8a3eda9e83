"""CPU test of bench.py's HBM-traffic bookkeeping: the two counter runs'
CSVs are reduced per kernel, scaled by the copy kernel's readings, stored
with the GEMM source's hash, and reported only while that hash matches."""
import csv
import json
import os

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
GEMM = "void fp4dev::(anonymous namespace)::gemm_mx_tn<7, 4, true, false, false, false>(unsigned char const*)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"
QUANT = "void fp4dev::(anonymous namespace)::quant_mx_along_rows_lds<32, false, 2, -1>(unsigned short const*)"


def _write_run(d, counter, rows):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, value in rows:
            # each dispatch's value arrives split over two XCD rows, summed by the reader
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value / 2})
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value / 2})
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": "OTHER",
                        "Counter_Value": 1e9})


def test_counter_summary_scales_by_the_copy_kernel(tmp_path):
    kib = bench.COPY_BYTES / 1024.0
    # FETCH_SIZE counts half the bytes (factor 2), WRITE_SIZE all of them
    _write_run(str(tmp_path / "f"), "FETCH_SIZE",
               [(1, GEMM, 1000.0), (2, GEMM, 1200.0), (3, COPY, kib / 2), (4, QUANT, 5.0)])
    _write_run(str(tmp_path / "w"), "WRITE_SIZE",
               [(1, GEMM, 300.0), (2, GEMM, 300.0), (3, COPY, kib), (4, QUANT, 5.0)])
    out = str(tmp_path / "c.json")
    assert bench.counter_summary(str(tmp_path / "f"), str(tmp_path / "w"), out=out) == 0
    rec = json.load(open(out))
    assert rec["dispatches"] == [2, 2]
    assert abs(rec["fetch_factor"] - 2.0) < 1e-12 and abs(rec["write_factor"] - 1.0) < 1e-12
    assert abs(rec["hbm_read_bytes_per_launch"] - 1100.0 * 1024 * 2) < 1e-6
    assert abs(rec["hbm_write_bytes_per_launch"] - 300.0 * 1024) < 1e-6
    assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    # reported while the recorded hash is the current source's, and only for gate/up
    assert bench.traffic_per_launch("gate_up", out) == rec["hbm_bytes_per_launch"]
    assert bench.traffic_per_launch("q_proj", out) is None
    rec["gemm_source_sha256"] = "0" * 64
    json.dump(rec, open(out, "w"))
    assert bench.traffic_per_launch("gate_up", out) is None
    assert bench.traffic_per_launch("gate_up", str(tmp_path / "missing.json")) is None


def test_counter_summary_needs_exactly_one_gemm_kernel(tmp_path):
    kib = bench.COPY_BYTES / 1024.0
    _write_run(str(tmp_path / "f"), "FETCH_SIZE", [(1, COPY, kib)])
    _write_run(str(tmp_path / "w"), "WRITE_SIZE", [(1, COPY, kib)])
    try:
        bench.counter_summary(str(tmp_path / "f"), str(tmp_path / "w"), out=str(tmp_path / "c.json"))
    except SystemExit as e:
        assert "gemm_mx_tn" in str(e)
    else:
        raise AssertionError("a run without the GEMM was accepted")
    assert not (tmp_path / "c.json").exists()
