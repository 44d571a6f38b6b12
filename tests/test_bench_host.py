"""Host-side logic of bench.py (no GPU): the per-path summary and the HBM
traffic record built from rocprofv3 counter CSV files."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_summary_rates_and_ratios():
    # 1 TFLOP and 1 GB in 1 ms: 1000 TFLOP/s and 1000 GB/s
    s = bench._summary(1e12, 1e9, {"overlap": 1.0, "serial": 1.5, "compute_only": 0.8, "comm_only": 0.5})
    assert s["tflops"] == 1000.0
    assert s["pct_bf16_peak"] == 40.0
    assert s["hbm_GBps_algorithmic"] == 1000.0
    assert s["pct_hbm_peak"] == 12.5
    assert s["speedup_vs_serial"] == 1.5
    assert s["overlap_vs_compute_only"] == 1.25
    # (compute + comm - overlap) / comm
    assert s["overlap_ratio"] == pytest.approx((0.8 + 0.5 - 1.0) / 0.5)
    s2 = bench._summary(1e12, 1e9, {"overlap": 1.0, "serial": 1.0, "compute_only": 1.0, "comm_only": None})
    assert "overlap_ratio" not in s2


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_counters_scales_by_the_plain_copy(tmp_path):
    # the calibration copy moves 1 GiB each way; FETCH_SIZE reads half of it
    # (factor 2), WRITE_SIZE all of it (factor 1); values are KiB per dispatch
    gib_kib = (1 << 30) / 1024
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _write_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", gib_kib / 2), ("__amd_rocclr_copyBuffer", 10.0),
                                     ("void ag_gemm_kernel<...>(Args)", 1000.0), ("void ag_gemm_kernel<...>(Args)", 3000.0),
                                     ("ag_copy_kernel(CopyArgs)", 500.0)])
    _write_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib_kib),
                                     ("void ag_gemm_kernel<...>(Args)", 100.0), ("void ag_gemm_kernel<...>(Args)", 300.0),
                                     ("ag_copy_kernel(CopyArgs)", 700.0)])
    out = tmp_path / "traffic.json"
    rec = bench.summarize_counters(str(fetch), str(write), str(out))
    assert rec["FETCH_SIZE_scale"] == pytest.approx(2.0)
    assert rec["WRITE_SIZE_scale"] == pytest.approx(1.0)
    g = rec["kernels"]["ag_gemm_kernel"]
    assert g["fetch_bytes"] == int(2000.0 * 1024 * 2)     # mean of 1000 and 3000 KiB, times 2
    assert g["write_bytes"] == int(200.0 * 1024)
    assert g["bytes_per_launch"] == g["fetch_bytes"] + g["write_bytes"]
    assert g["launches"] == 2
    c = rec["kernels"]["ag_copy_kernel"]
    assert c["fetch_bytes"] == int(500.0 * 1024 * 2) and c["write_bytes"] == int(700.0 * 1024)
    assert json.load(open(out))["source_hash"] == bench.source_hash()


def test_traffic_record_applies_only_to_current_sources(tmp_path, monkeypatch):
    rec = {"source_hash": "not-the-current-sources", "kernels": {"ag_gemm_kernel": {"bytes_per_launch": 5}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC", str(path))
    assert bench._traffic("ag_gemm_kernel") is None
    rec["source_hash"] = bench.source_hash()
    path.write_text(json.dumps(rec))
    assert bench._traffic("ag_gemm_kernel") == 5
    assert bench._traffic("missing_kernel") is None


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU only" in capsys.readouterr().err
