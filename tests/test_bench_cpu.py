"""bench.py's host logic on the CPU (no GPU needed): the one-GPU guard, the
algorithmic byte count behind the roofline, the recorded-traffic guard, and
the shape of the CPU-baseline record."""

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_grouped_gemm_route_amd.synth import make_config  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_count_active_experts_and_unique_rows():
    p = make_config(1)      # 8 experts, expert 7 empty, gathered token rows
    active = len(set(p["topk_ids"].reshape(-1).tolist()))
    assert active == 7
    nbytes, got_active = bench.algorithmic_bytes(p, "mxfp4")
    # codes: half a byte per weight; E8M0 scales: one byte per 32 weights;
    # activations: every token row once (gathered), bf16
    assert got_active == active
    assert nbytes == active * p["N"] * p["K"] // 2 + active * p["N"] * p["K"] // 32 + p["T"] * p["K"] * 2
    nv, _ = bench.algorithmic_bytes(p, "nvfp4")
    assert nv == active * p["N"] * p["K"] // 2 + active * p["N"] * p["K"] // 16 + 4 * active + p["T"] * p["K"] * 2


def test_recorded_traffic_needs_the_current_kernel_source(monkeypatch):
    rec = json.load(open(bench.TRAFFIC_FILE))
    entry = rec["w13_decode"]
    monkeypatch.setattr(bench, "gmm_source_hash", lambda: entry["gmm_source_sha256_16"])
    assert bench.recorded_traffic("w13_decode") == entry["bytes_per_launch"]
    monkeypatch.setattr(bench, "gmm_source_hash", lambda: "0" * 16)
    assert bench.recorded_traffic("w13_decode") is None
    assert bench.recorded_traffic("no_such_workload") is None


def test_cpu_baseline_record():
    p = make_config(1)
    out = bench.cpu_baseline(p, "mxfp4", "GB/s", target_s=0.2)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "active experts" in out["sample"]
    assert np.isfinite(out["value"])
