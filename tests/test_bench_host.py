"""Host-side parts of bench.py (no GPU): the one-GPU guard, the traffic
record's tie to the GEMM sources, and the CPU-oracle baseline leg."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_matches_the_gemm_sources():
    """The committed HBM byte counters were taken on the current GEMM
    sources; after a kernel change they must be taken again (until then the
    bench reports traffic as null)."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert rec["kernel_source_sha"] == bench.kernel_source_hash(bench.GEMM_SOURCES), \
        "GEMM sources changed since the traffic counters were taken"
    assert bench.measured_traffic() == rec["bytes_per_launch"]
    scaled = round(rec["fetch_size_kib_per_launch_raw"] * 1024 * rec["fetch_scale"]
                   + rec["write_size_kib_per_launch_raw"] * 1024 * rec["write_scale"])
    assert scaled == rec["bytes_per_launch"]
    assert rec["bytes_per_launch"] >= rec["algorithmic_bytes_per_launch"]


def test_cpu_baseline_leg_reports_the_contract_fields():
    gen = torch.Generator().manual_seed(5)
    x = torch.randn((8, 64), generator=gen).to(torch.bfloat16)
    w = torch.randn((32, 64), generator=gen).to(torch.bfloat16)
    out = bench.cpu_baseline(x, w, rows=4, min_seconds=0.01)
    assert set(out) >= {"value", "unit", "cores", "kind", "sample"}
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "4 of 8 rows" in out["sample"]
