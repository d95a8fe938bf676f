"""Host logic of bench.py (no GPU): peak derivation from rocminfo text, the HBM
byte calibration behind the roofline's "traffic" figure and its source-digest
check, the rocprofv3 CSV summary, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_peaks_from_rocminfo_text(monkeypatch):
    text = ("*******\nAgent 1\n  Name: AMD EPYC\n  Compute Unit: 128\n  Max Clock Freq. (MHz): 3700\n"
            "*******\nAgent 2\n  Name: gfx950\n  Compute Unit: 256\n  Max Clock Freq. (MHz): 2400\n")

    class R:
        stdout = text

    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: R())
    pk = bench.peaks()
    assert pk["compute_units"] == 256 and pk["max_clock_mhz"] == 2400
    assert pk["source"].startswith("rocminfo")
    # 256 CUs x 4096 flop/clk (v_mfma_f32_32x32x16: 32768 flop per 32 cycles on each of 4 SIMDs) x 2.4 GHz
    assert abs(pk["mfma_bf16_tflops"] - 2516.5824) < 1e-6
    assert pk["mfma_fp8_tflops"] == 2 * pk["mfma_bf16_tflops"]
    assert pk["hbm_gbs"] == 8000.0


def test_peaks_without_rocminfo(monkeypatch):
    def boom(*a, **k):
        raise FileNotFoundError("rocminfo")

    monkeypatch.setattr(bench.subprocess, "run", boom)
    pk = bench.peaks()
    assert pk["source"].startswith("published") and abs(pk["mfma_bf16_tflops"] - 2516.5824) < 1e-6


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_record_traffic_calibration_and_digest(tmp_path, monkeypatch):
    # a fake repository: the sources the digest covers, and profiles/
    for p in set(p for _, srcs in bench.DOMINANT.values() for p in srcs):
        os.makedirs(os.path.dirname(tmp_path / p), exist_ok=True)
        (tmp_path / p).write_text("// " + p + "\n")
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    neg = "void at::native::vectorized_elementwise_kernel<8, at::native::neg_kernel_cuda()>"
    c5 = "void attn::tile_attn_kernel<attn::BF16, 192, 128, true, false, 1, 4, 1, 64, true, true, 2, false, false>(a)"
    # the copy pass of 16 MiB reads and writes 16384 KiB; FETCH_SIZE reports half of it, WRITE_SIZE all of it
    _counter_csv(tmp_path / "f", [(neg, "FETCH_SIZE", 8192.0), (neg, "FETCH_SIZE", 8192.0),
                                  (c5, "FETCH_SIZE", 1000.0), (c5, "FETCH_SIZE", 1200.0)])
    _counter_csv(tmp_path / "w", [(neg, "WRITE_SIZE", 16384.0), (c5, "WRITE_SIZE", 300.0)])
    bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), 16)
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))
    assert rec["_calibration"] == {"copy_mib": 16, "fetch_scale": 2.0, "write_scale": 1.0}
    c = rec["C5_fwd_asym_b2h16s4096_causal"]
    assert c["kernel"] == c5
    assert c["fetch_kib_per_dispatch"] == 1100.0          # mean over dispatches
    assert c["hbm_bytes_per_launch"] == 1024.0 * (1100.0 * 2.0 + 300.0 * 1.0)
    assert "C3_decode_gqa" not in rec                     # no matching kernel in the runs
    # the figure is reported while the kernel's sources are unchanged, and not after an edit
    assert bench.traffic_entry("C5_fwd_asym_b2h16s4096_causal") == c["hbm_bytes_per_launch"]
    (tmp_path / bench.TILE_SRCS[0]).write_text("// edited\n")
    assert bench.traffic_entry("C5_fwd_asym_b2h16s4096_causal") is None


def test_committed_traffic_matches_committed_sources():
    # profiles/traffic.json was recorded from the kernels as they are in the tree
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    names = [k for k in rec if not k.startswith("_")]
    assert set(names) == set(bench.DOMINANT)
    for name in names:
        assert bench.traffic_entry(name) is not None, name


def test_summarize_kernel_stats(tmp_path, capsys):
    d = tmp_path / "trace"
    os.makedirs(d)
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "void attn::decode_attn_kernel<x>", "Calls": 10, "AverageNs": 34170.0,
                    "MinNs": 28000.0, "MaxNs": 40000.0})
    bench.summarize(str(d))
    out = capsys.readouterr().out
    assert "decode_attn_kernel" in out and "34.17" in out and "28.00" in out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
