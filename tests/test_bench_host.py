"""Host-side parts of the benchmark (no GPU): the algorithmic counts its rates are built on,
the bookkeeping of counter-derived HBM traffic, and its refusal of more than one GPU."""
from __future__ import annotations

import argparse
import csv
import json
import subprocess
import sys
from pathlib import Path

import pytest

import bench
import workloads as wl

ROOT = Path(__file__).resolve().parents[1]


def test_algorithmic_counts_by_hand():
    """Tiny workload shape: L = {64, 200}, s_q = 1, h_q = 16, every token visible."""
    nbytes, flops = wl.algorithmic_counts([64, 200], 1, 16, True)
    rows = 2 * 16
    assert nbytes == (64 + 200) * 1152 + rows * (1152 + 1024 + 4) + 4 * (1 + 4) + 4 * 2
    assert flops == (64 + 200) * 16 * 2 * (576 + 512)


def test_algorithmic_counts_causal_and_empty():
    """Two new tokens see L - 1 and L tokens; an empty sequence moves only its q/out/lse and length."""
    nbytes, flops = wl.algorithmic_counts([10, 0], 2, 16, True)
    assert flops == (9 + 10) * 16 * 2 * 1088
    assert nbytes == 10 * 1152 + 2 * 2 * 16 * 2180 + 4 * 1 + 4 * 2
    _, flops_nc = wl.algorithmic_counts([10, 0], 2, 16, False)
    assert flops_nc == 20 * 16 * 2 * 1088


def test_fp8_counts_bytes_per_row():
    b16, f16 = wl.algorithmic_counts([100, 300], 1, 16, True)
    b8, f8 = wl.fp8_counts([100, 300], 1, 16, True)
    assert f8 == f16
    assert b16 - b8 == 400 * (1152 - 580)


@pytest.mark.parametrize("op,workload,key,kernel", [
    ("decode", "memory_bound", "memory_bound", "decode_stream_kernel<1, false>"),
    ("decode", "long", "long", "decode_stream_kernel<1, false>"),
    ("decode", "compute_bound", "compute_bound", "decode_wide_kernel"),
    ("decode", "mixed", "mixed", "decode_wide_kernel"),
    ("fp8", "memory_bound", "fp8_memory_bound", "decode_stream_fp8_kernel"),
    ("fp8", "mixed", "fp8_mixed", "decode_wide_fp8_kernel"),
    ("sparse", "memory_bound", "sparse", "decode_stream_kernel<1, true>"),
    ("append", "memory_bound", "append", "append_kernel"),
    ("append_fp8", "memory_bound", "append_fp8", "append_fp8_kernel"),
])
def test_traffic_keys_and_kernels(op, workload, key, kernel):
    assert bench.traffic_key(op, workload) == key
    assert bench.traffic_kernel(key) == kernel


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("long") is None                      # no file
    f.write_text(json.dumps({"long": {"hbm_bytes_per_launch": 123, "kernel_source_sha": "0" * 16}}))
    assert bench.measured_traffic("long") is None                      # taken on other sources
    f.write_text(json.dumps({"long": {"hbm_bytes_per_launch": 123,
                                      "kernel_source_sha": bench.kernel_source_digest("long")}}))
    assert bench.measured_traffic("long") == 123
    assert bench.measured_traffic("mixed") is None                     # no entry


def _counter_csv(path: Path, rows):
    path.mkdir(parents=True)
    with open(path / "p_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, counter, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    """HBM bytes = FETCH_SIZE x (copy bytes / copy FETCH_SIZE) + WRITE_SIZE x (copy bytes / copy WRITE_SIZE),
    counters in KiB per dispatch, averaged over the dispatches of the case's kernel only."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kname = "void mla::decode_stream_kernel<1, false>(mla::DecodeParams)"
    _counter_csv(tmp_path / "fetch", [(kname, "FETCH_SIZE", 1000.0), (kname, "FETCH_SIZE", 3000.0),
                                      ("mla::combine_kernel", "FETCH_SIZE", 99999.0)])
    _counter_csv(tmp_path / "write", [(kname, "WRITE_SIZE", 500.0)])
    copy = 256 * 2 ** 20
    _counter_csv(tmp_path / "cfetch", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy / 1024 / 2)])
    _counter_csv(tmp_path / "cwrite", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy / 1024)])
    args = argparse.Namespace(
        pmc_summary=[str(tmp_path / d) for d in ("fetch", "write", "cfetch", "cwrite")],
        op="decode", workload="memory_bound", copy_bytes=copy)
    assert bench.pmc_summary(args) == 0
    ent = json.loads((tmp_path / "traffic.json").read_text())["memory_bound"]
    assert ent["factor_fetch"] == 2.0 and ent["factor_write"] == 1.0
    assert ent["dispatches"] == [2, 1]
    assert ent["hbm_bytes_per_launch"] == int(2000 * 1024 * 2.0 + 500 * 1024 * 1.0)
    assert ent["kernel_source_sha"] == bench.kernel_source_digest("memory_bound")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=str(ROOT), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_spread_sample_keeps_the_ends_and_is_bounded():
    assert bench.spread_sample(128, 5) == [0, 32, 64, 95, 127]
    assert bench.spread_sample(16, 40) == list(range(16))
    assert bench.spread_sample(7, 0) == [0]


def test_median_rate_arithmetic():
    med, gbs, tf = bench.median_rate([3.0, 1.0, 2.0], 4e9, 6e12)
    assert med == 2.0 and gbs == 2.0 and tf == 3.0


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
