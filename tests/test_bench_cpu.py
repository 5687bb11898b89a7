"""bench.py's host logic on the CPU (no GPU needed): the one-GPU guard, the
algorithmic byte count behind the roofline, the recorded-traffic guard and the
code hash it keys on, and the shape of the CPU-baseline record."""

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


def test_code_hash_ignores_comments_and_blank_space_only():
    src = "int f(int a) {\n  // the sum\n  return a + 1;  /* one */\n}\n"
    same = "int f(int a) {   return a + 1; }  // edited comment\n/* a new\n block */\n"
    changed = "int f(int a) {\n  return a + 2;\n}\n"
    assert bench.code_hash(src) == bench.code_hash(same)
    assert bench.code_hash(src) != bench.code_hash(changed)
    assert bench.gmm_source_hash() == bench.code_hash(open(bench.GMM_SOURCE, encoding="utf-8").read())


def test_cpu_baseline_record():
    p = make_config(1)
    out = bench.cpu_baseline(p, "mxfp4", "GB/s", target_s=0.2)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "active experts" in out["sample"]
    assert np.isfinite(out["value"])


def test_roofline_picks_the_longer_roof_and_reports_against_its_own_peak():
    # HBM roof time 1e9 B / 8 TB/s = 125 us; bf16 MFMA roof of 1e11 FLOP at
    # 2.5 PFLOP/s = 40 us: HBM-bound
    r = bench.roofline(1e9, 1e11, 250e-6)
    assert r["bound"] == "hbm" and r["peak"] == bench.HBM_PEAK_GBS
    assert abs(r["achieved"] - 4000.0) < 0.1 and abs(r["frac"] - 0.5) < 1e-4
    # 1e12 FLOP: 400 us on bf16 MFMA, the longer roof
    r = bench.roofline(1e9, 1e12, 1e-3)
    assert r["bound"] == "mfma" and r["peak"] == bench.BF16_PEAK_TFLOPS
    assert abs(r["frac"] - 1000.0 / bench.BF16_PEAK_TFLOPS) < 1e-4
    # a W4A4 shape bound by the FP4 matrix unit (5e12 FLOP: 495 us at 10.1
    # PFLOP/s) is reported against the FP4 peak, not the bf16 one
    r = bench.roofline(1e9, 5e12, 1e-3, bench.FP4_PEAK_TFLOPS)
    assert r["bound"] == "mfma" and r["peak"] == bench.FP4_PEAK_TFLOPS
    assert abs(r["frac"] - 5000.0 / bench.FP4_PEAK_TFLOPS) < 1e-4
    # 1e12 FLOP at FP4 speed is 99 us, shorter than the 125 us of HBM
    assert bench.roofline(1e9, 1e12, 1e-3, bench.FP4_PEAK_TFLOPS)["bound"] == "hbm"


def test_tokens_flag_is_refused_for_layer_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "layer_prefill",
                        "--tokens", "512"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--tokens" in r.stderr
