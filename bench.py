"""Benchmark of the routed-expert W4A16 grouped matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input with the
expert weights already packed and resident in HBM (the one-time load-time
repack is excluded, as the grouped-matmul timings of "Running DeepSeek V4
Flash on TPU v6", section "Grouped matmul performance vs bf16", exclude it):
  route-sort of the top-k ids -> grouped matmul (-> top-k combine for the
  down-projection workload, whose router weights are given).
The default workload is the gate/up (w13) decode: 64 tokens, hidden 4096,
256 experts, top-6 uniform routing, fused gate+up weight K = N = 4096 in
MXFP4, bf16 output.  The layer_decode workload runs one whole routed-expert
layer on the same tokens: route-sort -> w13 with the SiLU-gated gate/up
activation fused (bf16 [384, 2048]) -> w2 (K = 2048, N = 4096, f32) ->
top-k combine; layer_prefill runs the same layer on config 4's 4,096
tokens (both matmuls on the LDS-tiled kernel), and w4a4_layer_prefill runs it
W4A4 (x and the activation h quantized to MXFP4 inside the step).  The bf16_w13_decode, bf16_w2_decode and bf16_w13_prefill
workloads time the bf16-weight comparison arm on the decoded weights of
configs 2, 3 and 4 (the same values, four times the bytes) next to the MXFP4
kernel on the same inputs, and report the MXFP4 speedup.  The w4a4_w13_prefill workload runs
the 4,096-token w13 prefill W4A4: the activations are quantized to MXFP4
inside the step and the matmul runs on the scaled FP4 matrix instructions.

One JSON line is printed.  value is the whole step's throughput in the
algorithmic bytes of the matmul (codes + scales of the experts that received
tokens, plus the activations read) per second; roofline.achieved is the same
bytes over the grouped-matmul kernel's own average duration, timed with HIP
events on the stream it runs on (gmm_us; the median and minimum are reported
beside it).  The CPU baseline times the float64 oracle on a bounded sample of
the same workload on the host cores; gpu_over_cpu is value over its value.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 MFMA, published

WORKLOADS = {
    "tiny": 1, "w13_decode": 2, "w2_decode": 3, "w13_prefill": 4, "nvfp4_w13": 5,
    "layer_decode": 0, "layer_prefill": 0, "w4a4_layer_prefill": 0, "bf16_w13_decode": 2, "bf16_w2_decode": 3, "bf16_w13_prefill": 4,
    "w4a4_w13_prefill": 4,
}
KERNELS = {"auto": 0, "stream": 1, "tiled": 2}
GMM_SOURCE = os.path.join(ROOT, "moe_grouped_gemm_route_amd", "csrc", "gmm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")


def gmm_source_hash():
    with open(GMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(p, fmt):
    """Codes + scales (or bf16 weights) of every expert with a non-empty band,
    plus the activation bytes the matmul reads (unique token rows when
    gathering)."""
    counts = np.bincount(p["topk_ids"].reshape(-1), minlength=p["E"])
    active = int(np.count_nonzero(counts))
    per_weight = {"mxfp4": 0.5 + 1.0 / 32, "nvfp4": 0.5 + 1.0 / 16, "bf16": 2.0}[fmt]
    w_bytes = active * p["N"] * p["K"] * per_weight + (active * 4 if fmt == "nvfp4" else 0)
    x_rows = p["T"] if p["gather"] else p["T"] * p["k"]
    return w_bytes + x_rows * p["K"] * 2, active


def cpu_baseline(p, fmt, unit, target_s=15.0):
    """The float64 oracle on the host: route-sort of the whole batch, then the
    grouped matmul of as many expert bands (in expert order) as fit in about
    target_s seconds.  Reported as the same algorithmic bytes per second."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    if fmt == "nvfp4":
        bs, ts = oracle.mxfp4_to_nvfp4(p["scales"])
        w = {"fmt": "nvfp4", "codes": p["codes"], "block_scales": bs, "tensor_scale": ts}
    else:
        w = {"fmt": "mxfp4", "codes": p["codes"], "scales": p["scales"]}
    t0 = time.perf_counter()
    r = oracle.route_sort(p["topk_ids"], p["E"])
    off = r["group_offsets"]
    active = [e for e in range(p["E"]) if off[e + 1] > off[e]]
    done, nbytes = 0, 0.0
    per_weight = 0.5 + (1.0 / 32 if fmt == "mxfp4" else 1.0 / 16)
    rows_done = 0
    while done < len(active) and time.perf_counter() - t0 < target_s:
        e = active[done]
        sub_off = np.array([off[e], off[e + 1]], dtype=np.int32)
        sub = dict(w)
        sub["codes"] = w["codes"][e:e + 1]
        if fmt == "mxfp4":
            sub["scales"] = w["scales"][e:e + 1]
        else:
            sub["block_scales"] = w["block_scales"][e:e + 1]
            sub["tensor_scale"] = w["tensor_scale"][e:e + 1]
        ri = r["sorted_token"] if p["gather"] else None
        oracle.gmm(p["x"], ri, sub_off, sub)
        nbytes += p["N"] * p["K"] * per_weight
        rows_done += int(off[e + 1] - off[e])
        done += 1
    elapsed = time.perf_counter() - t0
    x_rows = (p["T"] * rows_done / (p["T"] * p["k"])) if p["gather"] else rows_done
    nbytes += x_rows * p["K"] * 2
    if unit == "TFLOP/s":
        value = 2.0 * rows_done * p["K"] * p["N"] / elapsed / 1e12
    else:
        value = nbytes / elapsed / 1e9
    return {
        "value": round(value, 6), "unit": unit, "cores": int(threads),
        "kind": "oracle",
        "sample": "float64 numpy oracle on %s: route-sort of all %d pairs + grouped matmul of "
                  "the first %d of %d active experts' bands (%d rows), %.1f s"
                  % (cpu_model(), p["T"] * p["k"], done, len(active), rows_done, elapsed),
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def layer_cpu_baseline(p, unit="GB/s", target_s=15.0):
    """The float64 oracle for one layer on the host: route-sort, then for as
    many active experts (in expert order) as fit in about target_s seconds,
    the w13 band matmul, the gate/up activation and the w2 band matmul."""
    import oracle
    from moe_grouped_gemm_route_amd.synth import f32_to_bf16_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    r = oracle.route_sort(p["topk_ids"], p["E"])
    off = r["group_offsets"]
    active = [e for e in range(p["E"]) if off[e + 1] > off[e]]
    per13 = p["N"] * p["K"] * (0.5 + 1.0 / 32)
    per2 = p["K"] * (p["N"] // 2) * (0.5 + 1.0 / 32)
    done, rows_done, nbytes = 0, 0, 0.0
    while done < len(active) and time.perf_counter() - t0 < target_s:
        e = active[done]
        sub_off = np.array([0, off[e + 1] - off[e]], dtype=np.int32)
        w13 = {"fmt": "mxfp4", "codes": p["codes"][e:e + 1], "scales": p["scales"][e:e + 1]}
        w2 = {"fmt": "mxfp4", "codes": p["w2_codes"][e:e + 1], "scales": p["w2_scales"][e:e + 1]}
        rows = r["sorted_token"][off[e]:off[e + 1]]
        y13 = oracle.gmm(p["x"], rows, sub_off, w13)
        h = oracle.silu_mul(y13)
        oracle.gmm(f32_to_bf16_bits(h.astype(np.float32)), None, sub_off, w2)   # w2 reads bf16
        nbytes += per13 + per2
        rows_done += int(off[e + 1] - off[e])
        done += 1
    elapsed = time.perf_counter() - t0
    nbytes += (p["T"] * rows_done / (p["T"] * p["k"])) * p["K"] * 2 + rows_done * (p["N"] // 2) * 2
    flops = 2.0 * rows_done * p["K"] * (p["N"] + p["N"] // 2)
    rate = flops / elapsed / 1e12 if unit == "TFLOP/s" else nbytes / elapsed / 1e9
    return {
        "value": round(rate, 6), "unit": unit, "cores": int(threads),
        "kind": "oracle",
        "sample": "float64 numpy oracle on %s: route-sort of all %d pairs + w13, gate/up "
                  "activation and w2 of the first %d of %d active experts' bands (%d rows), %.1f s"
                  % (cpu_model(), p["T"] * p["k"], done, len(active), rows_done, elapsed),
    }


def route_workspace(T, k, E, dev):
    """The route sort's device workspace, allocated once outside the timed
    steps (None when the sort needs none)."""
    import torch
    import moe_grouped_gemm_route_amd as moe
    need = moe.route_sort_workspace_bytes(T, k, E)
    return torch.empty((need + 3) // 4, dtype=torch.int32, device=dev) if need else None


def run_layer(args):
    """One routed-expert layer (the layer_decode and layer_prefill workloads)."""
    import torch
    import moe_grouped_gemm_route_amd as moe
    from moe_grouped_gemm_route_amd.synth import make_layer_decode, make_layer_prefill

    prefill = args.workload in ("layer_prefill", "w4a4_layer_prefill")
    w4a4 = args.workload == "w4a4_layer_prefill"
    p = make_layer_prefill() if prefill else make_layer_decode()
    E, K, N, T, k = p["E"], p["K"], p["N"], p["T"], p["k"]
    M, H = T * k, N // 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    ids, x, tw = d(p["topk_ids"]), d(p["x"]), d(p["topk_weights"])
    codes = d(p["codes"])
    w13 = moe.mxfp4_encode(codes, d(p["scales"]), None, moe.MXFP4)
    del codes
    codes = d(p["w2_codes"])
    w2 = moe.mxfp4_encode(codes, d(p["w2_scales"]), None, moe.MXFP4)
    del codes
    h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((M, K), dtype=torch.float32, device=dev)
    ws = route_workspace(T, k, E, dev)
    torch.cuda.synchronize()
    ev = []

    def step(timed):
        # events around each matmul kernel (the W4A4 quantizations fall between)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        r = moe.route_sort(ids, E, ws=ws)
        if w4a4:
            qc, qs = moe.mxfp4_quantize(x)
            if timed:
                e[0].record()
            moe.moe_gmm_w4a4(w13, E, N, K, qc, qs, r["group_offsets"], M, row_index=r["sorted_token"],
                             out_dtype=moe.BF16, act=moe.ACT_SILU_MUL, out=h)
            if timed:
                e[1].record()
            qc, qs = moe.mxfp4_quantize(h)
            if timed:
                e[2].record()
            moe.moe_gmm_w4a4(w2, E, K, H, qc, qs, r["group_offsets"], M, out_dtype=moe.F32, out=y2)
        else:
            if timed:
                e[0].record()
            moe.moe_gmm(w13, moe.MXFP4, E, N, K, x, r["group_offsets"], M, row_index=r["sorted_token"],
                        out_dtype=moe.BF16, act=moe.ACT_SILU_MUL, out=h)
            if timed:
                e[1].record()
                e[2].record()
            moe.moe_gmm(w2, moe.MXFP4, E, K, H, h, r["group_offsets"], M, out_dtype=moe.F32, out=y2)
        if timed:
            e[3].record()
            ev.append(e)
        return moe.moe_combine(y2, tw, r["pair_row"])

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t13 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / 1e3
    t2 = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) / 1e3
    counts = np.bincount(p["topk_ids"].reshape(-1), minlength=E)
    active = int(np.count_nonzero(counts))
    b13 = active * N * K * (0.5 + 1.0 / 32) + T * K * 2
    b2 = active * K * H * (0.5 + 1.0 / 32) + M * H * 2
    step_s = wall / args.steps
    flops = 2.0 * M * K * (N + H)
    if w4a4:
        # quantized activations: K/2 + K/32 bytes per row instead of 2K
        b13 = active * N * K * (0.5 + 1.0 / 32) + T * (K // 2 + K // 32)
        b2 = active * K * H * (0.5 + 1.0 / 32) + M * (H // 2 + H // 32)
    # matrix-unit bound when its roof time is the longer one (bf16 prefill)
    peak_flops = (FP4_PEAK_TFLOPS if w4a4 else BF16_PEAK_TFLOPS) * 1e12
    mfma_bound = flops / peak_flops > (b13 + b2) / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved = flops / (t13 + t2) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
        value, unit = flops / step_s / 1e12, "TFLOP/s"
    else:
        achieved = (b13 + b2) / (t13 + t2) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
        value, unit = (b13 + b2) / step_s / 1e9, "GB/s"
        if prefill:
            value, unit = flops / step_s / 1e12, "TFLOP/s"
    if w4a4:
        roof["fp4_mfma_frac"] = round(flops / (t13 + t2) / peak_flops, 4)
    calib = mfma_calibration(roof["achieved"]) if mfma_bound else None
    out = {
        "metric": "moe_gmm TFLOP/s and HBM GB/s (% roofline), w13/w2, 256 experts top-6",
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4" if w4a4 else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "top_k": k, "experts": E,
                   "w13": [K, N], "w2": [H, K], "routed_rows": M, "weights": "mxfp4",
                   "activations": "mxfp4 (quantized in the step)" if w4a4 else "bf16",
                   "gate_up": "silu(gate) * up fused into the w13 epilogue",
                   "step": ("route_sort + mxfp4_quantize(x) + moe_gmm_w4a4(w13, act) + mxfp4_quantize(h) "
                            "+ moe_gmm_w4a4(w2) + moe_combine") if w4a4 else
                           "route_sort + moe_gmm(w13, act) + moe_gmm(w2) + moe_combine"},
        "w13_us": round(t13 * 1e6, 2),
        "w2_us": round(t2 * 1e6, 2),
        "active_experts": active,
        "algorithmic_bytes": int(b13 + b2),
        "layer_tflops": round(flops / (t13 + t2) / 1e12, 2),
        "roofline": roof,
    }
    if calib is not None:
        out["mfma_calibration"] = calib
    if not args.no_cpu_baseline and not w4a4:
        out["cpu_baseline"] = layer_cpu_baseline(p, unit)
        out["gpu_over_cpu"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


CALIB_BLOCKS, CALIB_ITERS = 512, 12800     # two workgroups per CU, about 25 ms per launch


def mfma_calibration(achieved_tflops):
    """The bf16 matrix-unit rate this part sustains with no memory traffic
    (moe_calib_mfma_bf16: the tiled kernel's 128 x 64 wave tile of 16x16x32
    MFMAs on register-resident N(0,1) activations and decoded MXFP4 weights),
    the median of 3 launches after one warm-up, with the matmul's achieved
    rate as a fraction of it.  Measured after the timed steps; the roofline
    fraction stays the one against the published peak."""
    import torch
    import moe_grouped_gemm_route_amd as moe
    from moe_grouped_gemm_route_amd.synth import make_problem

    q = make_problem(T=2048, k=1, E=1, K=4096, N=1024, seed=41)
    dev = torch.device("cuda", 0)
    a = torch.from_numpy(q["x"].view(np.int16)).to(dev)
    packed = moe.mxfp4_encode(torch.from_numpy(q["codes"]).to(dev), torch.from_numpy(q["scales"]).to(dev),
                              None, moe.MXFP4)
    b = moe.debug_decode(packed, moe.MXFP4, 1, 1024, 4096)
    moe.calib_mfma_bf16(a, b, CALIB_BLOCKS, CALIB_ITERS)
    ms = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.calib_mfma_bf16(a, b, CALIB_BLOCKS, CALIB_ITERS)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    flops = CALIB_BLOCKS * 4.0 * CALIB_ITERS * 128 * 16384
    sustained = flops / (float(np.median(ms)) / 1e3) / 1e12
    return {"sustained_tflops": round(sustained, 1),
            "kernel_frac_of_sustained": round(achieved_tflops / sustained, 4),
            "loop": "bf16 16x16x32 MFMAs over a 128 x 64 wave tile, operands in registers, "
                    "%d workgroups of 4 waves, %.1f ms per launch" % (CALIB_BLOCKS, float(np.median(ms)))}


def recorded_traffic(workload):
    """HBM bytes per launch of the workload's matmul kernel from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated on a copy kernel),
    or None when there is none or the kernel source has changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        entry = json.load(open(TRAFFIC_FILE)).get(workload, {})
    except (OSError, ValueError):
        return None
    if entry.get("gmm_source_sha256_16") != gmm_source_hash():
        return None
    return entry.get("bytes_per_launch")


def run_w4a4(args):
    """The W4A4 prefill workload: route-sort, MXFP4 activation quantization and
    the grouped matmul on the scaled FP4 MFMA, over config 4's problem."""
    import torch
    import moe_grouped_gemm_route_amd as moe
    from moe_grouped_gemm_route_amd.synth import make_config

    p = make_config(4)
    E, K, N, T, k = p["E"], p["K"], p["N"], p["T"], p["k"]
    M = T * k
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    ids, x = d(p["topk_ids"]), d(p["x"])
    codes = d(p["codes"])
    packed = moe.mxfp4_encode(codes, d(p["scales"]), None, moe.MXFP4)
    del codes
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = route_workspace(T, k, E, dev)
    torch.cuda.synchronize()
    ev = []

    def step(timed):
        r = moe.route_sort(ids, E, ws=ws)
        qc, qs = moe.mxfp4_quantize(x)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        moe.moe_gmm_w4a4(packed, E, N, K, qc, qs, r["group_offsets"], M, row_index=r["sorted_token"], out=y)
        if timed:
            e1.record()
            ev.append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gmm_ms = [a.elapsed_time(b) for a, b in ev]
    gmm_s = float(np.mean(gmm_ms)) / 1e3
    flops = 2.0 * M * K * N
    counts = np.bincount(p["topk_ids"].reshape(-1), minlength=E)
    active = int(np.count_nonzero(counts))
    nbytes = active * N * K * (0.5 + 1.0 / 32) + T * (K // 2 + K // 32)
    achieved = nbytes / gmm_s / 1e9
    step_s = wall / args.steps
    out = {
        "metric": "moe_gmm TFLOP/s and HBM GB/s (% roofline), w13/w2, 256 experts top-6",
        "value": round(flops / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": "w4a4_w13_prefill", "tokens": T, "top_k": k, "experts": E, "K": K,
                   "N": N, "routed_rows": M, "weights": "mxfp4", "activations": "mxfp4 (quantized in the step)",
                   "output": "f32", "step": "route_sort + mxfp4_quantize + moe_gmm_w4a4"},
        "gmm_us": round(gmm_s * 1e6, 2),
        "gmm_us_median": round(float(np.median(gmm_ms)) * 1e3, 2),
        "gmm_us_min": round(float(np.min(gmm_ms)) * 1e3, 2),
        "gmm_tflops": round(flops / gmm_s / 1e12, 2),
        "active_experts": active,
        "algorithmic_bytes": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(args.workload),
                     "fp4_mfma_frac": round(flops / gmm_s / 1e12 / FP4_PEAK_TFLOPS, 4)},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="w13_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--kernel", default="auto", choices=sorted(KERNELS))
    ap.add_argument("--out-dtype", default=None, choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer --steps times (a plain copy "
                         "kernel of known size, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the routed-expert matmul would shard by experts, 32 per GPU on 8 GPUs)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload in ("layer_decode", "layer_prefill", "w4a4_layer_prefill") and not args.copy_calibration:
        run_layer(args)
        return
    if args.workload == "w4a4_w13_prefill" and not args.copy_calibration:
        run_w4a4(args)
        return

    import torch
    import moe_grouped_gemm_route_amd as moe
    from moe_grouped_gemm_route_amd.synth import make_config

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps}), flush=True)
        return

    cfg = WORKLOADS[args.workload]
    p = make_config(cfg)
    bf16_arm = args.workload.startswith("bf16_")
    fmt = "nvfp4" if cfg == 5 else "mxfp4"
    out_dtype = args.out_dtype or p["out"]
    odt = moe.BF16 if out_dtype == "bf16" else moe.F32
    E, K, N, T, k = p["E"], p["K"], p["N"], p["T"], p["k"]
    M = T * k
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    ids = d(p["topk_ids"])
    x = d(p["x"])
    codes = d(p["codes"])
    if fmt == "mxfp4":
        packed = moe.mxfp4_encode(codes, d(p["scales"]), None, moe.MXFP4)
        wf = moe.MXFP4
    else:
        bs, ts, err = moe.mxfp4_to_nvfp4(d(p["scales"]))
        packed = moe.mxfp4_encode(codes, bs, ts, moe.NVFP4)
        wf = moe.NVFP4
        assert err.item() == 0
    del codes
    packed_mx = None
    if bf16_arm:
        # the comparison arm streams the decoded weights as bf16
        dense = moe.debug_decode(packed, wf, E, N, K)
        packed_mx, packed = packed, moe.bf16_encode(dense)
        del dense
        fmt, wf = "bf16", moe.W_BF16
    tw = d(p["topk_weights"])
    combine = cfg == 3
    y = torch.empty((M, N), dtype=torch.bfloat16 if odt == moe.BF16 else torch.float32, device=dev)
    kernel = KERNELS[args.kernel]
    ws = route_workspace(T, k, E, dev)
    torch.cuda.synchronize()

    ev = []

    def step(timed):
        r = moe.route_sort(ids, E, ws=ws)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        moe.moe_gmm(packed, wf, E, N, K, x, r["group_offsets"], M,
                    row_index=r["sorted_token"] if p["gather"] else None,
                    out_dtype=odt, kernel=kernel, out=y)
        if timed:
            e1.record()
            ev.append((e0, e1))
        if combine:
            moe.moe_combine(y, tw, r["pair_row"])

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    mx_ms = None
    if bf16_arm:
        # the MXFP4 kernel on the same inputs, for the speedup
        r = moe.route_sort(ids, E, ws=ws)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        for i in range(args.warmup):
            moe.moe_gmm(packed_mx, moe.MXFP4, E, N, K, x, r["group_offsets"], M,
                        row_index=r["sorted_token"] if p["gather"] else None,
                        out_dtype=odt, kernel=kernel, out=y)
        e[0].record()
        for i in range(args.steps):
            moe.moe_gmm(packed_mx, moe.MXFP4, E, N, K, x, r["group_offsets"], M,
                        row_index=r["sorted_token"] if p["gather"] else None,
                        out_dtype=odt, kernel=kernel, out=y)
            e[i + 1].record()
        torch.cuda.synchronize()
        mx_ms = [e[i].elapsed_time(e[i + 1]) for i in range(args.steps)]

    gmm_ms = [a.elapsed_time(b) for a, b in ev]
    gmm_avg_s = float(np.mean(gmm_ms)) / 1e3
    gmm_med_s = float(np.median(gmm_ms)) / 1e3
    gmm_min_s = float(np.min(gmm_ms)) / 1e3
    nbytes, active = algorithmic_bytes(p, fmt)
    flops = 2.0 * M * K * N
    step_s = wall / args.steps
    # the roof is whichever bound takes longer at peak: the matrix unit for
    # MXFP4 prefill, HBM for decode and for bf16 weights at prefill
    prefill = flops / (BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9)
    if prefill:
        achieved = flops / gmm_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
        value, unit = flops / step_s / 1e12, "TFLOP/s"
    else:
        achieved = nbytes / gmm_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        value, unit = nbytes / step_s / 1e9, "GB/s"
    roof["traffic"] = recorded_traffic(args.workload)

    out = {
        "metric": "moe_gmm TFLOP/s and HBM GB/s (% roofline), w13/w2, 256 experts top-6",
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "top_k": k, "experts": E, "K": K,
                   "N": N, "routed_rows": M,
                   "weights": fmt + (" (decoded MXFP4 weights)" if bf16_arm else ""),
                   "activations": "bf16",
                   "output": out_dtype, "kernel": args.kernel,
                   "step": "route_sort + moe_gmm" + (" + moe_combine" if combine else "")},
        "gmm_us": round(gmm_avg_s * 1e6, 2),
        "gmm_us_median": round(gmm_med_s * 1e6, 2),
        "gmm_us_min": round(gmm_min_s * 1e6, 2),
        "gmm_tflops": round(flops / gmm_avg_s / 1e12, 2),
        "gmm_gbs": round(nbytes / gmm_avg_s / 1e9, 1),
        "active_experts": active,
        "algorithmic_bytes": int(nbytes),
        # + the output written and the index arrays read (band offsets, row index)
        "algorithmic_bytes_all": int(nbytes + M * N * (2 if odt == moe.BF16 else 4)
                                     + 4 * (E + 1) + (4 * M if p["gather"] else 0)),
        "roofline": roof,
    }
    if prefill:
        out["mfma_calibration"] = mfma_calibration(roof["achieved"])
    if mx_ms is not None:
        mx_s = float(np.mean(mx_ms)) / 1e3
        out["mxfp4_us"] = round(mx_s * 1e6, 2)
        out["mxfp4_speedup_over_bf16"] = round(gmm_avg_s / mx_s, 3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, "mxfp4" if bf16_arm else fmt, unit)
        out["gpu_over_cpu"] = round(value / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
