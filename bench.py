"""Benchmark of the routed-expert W4A16 grouped matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--tokens T] [--kernel auto|stream|tiled] [--only]

A step is one pass of the hot path over one batch of synthetic input with the
expert weights already packed and resident in HBM (the one-time load-time
repack is excluded, as the grouped-matmul timings of "Running DeepSeek V4
Flash on TPU v6", section "Grouped matmul performance vs bf16", exclude it):
  route-sort of the top-k ids -> grouped matmul (-> top-k combine for the
  down-projection workload, whose router weights are given).

The default workload is the gate/up (w13) decode: 64 tokens, hidden 4096,
256 experts, top-6 uniform routing, fused gate+up weight K = N = 4096 in
MXFP4, bf16 output.  Its line is the headline, timed over exactly --steps
steps.  Unless --only is given, the default run then times every other
benchmark workload (fewer steps each, and a shorter CPU-baseline sample) and
reports them in the same line under "workloads": tiny (64 tokens, 8 experts),
w2_decode (256 tokens, Zipf routing, K = 2048, with the combine), w13_prefill
(4,096 tokens), nvfp4_w13 (256 tokens, NVFP4 weights from the lossless cast),
nvfp4_w13_prefill, the whole routed-expert layer at decode and at prefill
(layer_decode, layer_prefill), the W4A4 w13 prefill and layer
(w4a4_w13_prefill, w4a4_layer_prefill), and one GPU's share of the w13 and
w2 decode under expert parallelism over 8 GPUs (ep8_w13_decode,
ep8_w2_decode: experts dealt round-robin, e on GPU e % 8; GPU 0's 32 experts,
the Zipf head among them, and one top-1 row per token-expert pair routed to
them, as the dispatch would deliver them; no combine in the share's step).

Other workloads, run alone with --workload:
  layer_decode / layer_prefill: route-sort -> w13 with the SiLU-gated gate/up
    activation fused (bf16 [M, 2048]) -> w2 (K = 2048, N = 4096, f32) ->
    top-k combine, on config 2's 64 or config 4's 4,096 tokens;
  w4a4_layer_prefill: the same layer W4A4 (x and h quantized to MXFP4 inside
    the step); w4a4_w13_prefill: the 4,096-token w13 W4A4, with MXFP4
    weights, or with NVFP4 ones from the lossless cast (w4a4_nvfp4_w13_prefill);
    w4a4_nvfp4_w13: config 5's 256 tokens, W4A4 with its NVFP4 weights;
  bf16_w13_decode, bf16_w2_decode, bf16_w13_prefill: the bf16-weight
    comparison arm on the decoded weights of configs 2, 3 and 4 (the same
    values, four times the bytes) next to the MXFP4 kernel on the same inputs;
  nvfp4_w13_prefill (also in the default run): the 4,096-token w13 with NVFP4
    weights from the lossless cast, next to the MXFP4 kernel on the same inputs;
  route_sort_decode / route_sort_prefill: the route sort alone on config 2's
    384 or config 4's 24,576 token-expert pairs (Mpairs/s).
--tokens T replaces a workload's token count (the weights stay the config's;
x and the routing are redrawn the same way), for the kernel-choice sweep.

value is the whole step's throughput: the algorithmic bytes of the matmul
(codes + scales of the experts that received tokens, plus the activations
read) per second for HBM-bound shapes, 2 M K N FLOP per second for the
MFMA-bound prefill.  roofline.achieved is the same quantity over the
grouped-matmul kernel's own average duration, timed with HIP events on the
stream it runs on (gmm_us; median and minimum beside it).  hbm_calibration
and mfma_calibration report the read rate and the matrix-unit rate this part
sustains on plain loops, with the kernel's fraction of them
(--mixed-calibration prints, alone, what plain PyTorch copy and row-sum
kernels reach when reads and writes mix, the regime of the combine;
--prefill-breakdown prints the matrix-unit rate of the tiled kernel's wave
tile with each part of its data movement added, and the rate of a plain bf16
library matmul of the prefill shape).  The CPU
baseline times the float64 oracle on a bounded sample of the same workload on
the host cores; gpu_over_cpu is value over its value.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 MFMA, published
METRIC = "moe_gmm TFLOP/s and HBM GB/s (% roofline), w13/w2, 256 experts top-6"

GMM_WORKLOADS = {
    "tiny": 1, "w13_decode": 2, "w2_decode": 3, "w13_prefill": 4, "nvfp4_w13": 5, "nvfp4_w13_prefill": 4,
    "bf16_w13_decode": 2, "bf16_w2_decode": 3, "bf16_w13_prefill": 4,
    # one GPU's share under expert parallelism over 8 GPUs (experts dealt
    # round-robin; rank 0, which holds the Zipf head expert)
    "ep8_w13_decode": 2, "ep8_w2_decode": 3,
}
NVFP4_GMM = ("nvfp4_w13", "nvfp4_w13_prefill")   # NVFP4 weights from the lossless cast
LAYER_WORKLOADS = ("layer_decode", "layer_prefill", "w4a4_layer_prefill")
# W4A4 grouped matmul: config, weight format
W4A4_WORKLOADS = {"w4a4_w13_prefill": (4, "mxfp4"), "w4a4_nvfp4_w13_prefill": (4, "nvfp4"),
                  "w4a4_nvfp4_w13": (5, "nvfp4")}
ROUTE_WORKLOADS = {"route_sort_decode": 2, "route_sort_prefill": 4}   # the route sort alone, on a config's routing
WORKLOADS = sorted(list(GMM_WORKLOADS) + list(LAYER_WORKLOADS) + list(W4A4_WORKLOADS) + list(ROUTE_WORKLOADS))
# timed after the headline in the default run
EXTRA_WORKLOADS = ("tiny", "w2_decode", "w13_prefill", "nvfp4_w13", "nvfp4_w13_prefill", "layer_decode",
                   "layer_prefill", "w4a4_w13_prefill", "w4a4_layer_prefill", "ep8_w13_decode", "ep8_w2_decode")
KERNELS = {"auto": 0, "stream": 1, "tiled": 2}
GMM_SOURCE = os.path.join(ROOT, "moe_grouped_gemm_route_amd", "csrc", "gmm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")


def code_hash(text):
    """sha256 prefix of C++ source with its comments and blank space removed,
    so that an edit of the comments keeps the hash of the code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def gmm_source_hash():
    with open(GMM_SOURCE, encoding="utf-8") as f:
        return code_hash(f.read())


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


def roofline(nbytes, flops, kernel_s, peak_tflops=BF16_PEAK_TFLOPS):
    """The roof whose time at peak is the longer one (the matrix unit for the
    MXFP4 prefill, HBM for decode shapes and bf16 weights), and the kernel's
    achieved rate against it."""
    peak_flops = peak_tflops * 1e12
    if flops / peak_flops > nbytes / (HBM_PEAK_GBS * 1e9):
        achieved = flops / kernel_s / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tflops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tflops, 4)}
    achieved = nbytes / kernel_s / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(p, fmt, unit, target_s=15.0):
    """The float64 oracle on the host: route-sort of the whole batch, then the
    grouped matmul of as many expert bands (in expert order) as fit in about
    target_s seconds.  Reported as the same algorithmic bytes (or FLOPs) per
    second."""
    import oracle
    threads = _threads()
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


def layer_cpu_baseline(p, unit="GB/s", target_s=15.0):
    """The float64 oracle for one layer on the host: route-sort, then for as
    many active experts (in expert order) as fit in about target_s seconds,
    the w13 band matmul, the gate/up activation and the w2 band matmul."""
    import oracle
    from moe_grouped_gemm_route_amd.synth import f32_to_bf16_bits
    threads = _threads()
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


# ---------------------------------------------------------------- GPU side --

class Gpu:
    """torch, the binding and device 0, imported on first use."""

    def __init__(self):
        import torch
        import moe_grouped_gemm_route_amd as moe
        self.torch, self.moe = torch, moe
        self.dev = torch.device("cuda", 0)
        torch.cuda.set_device(self.dev)
        # warm-up floor in seconds of device time, besides the step count;
        # warmup_done is the number of warm-up steps the last run took
        self.min_warmup_s = 0.0
        self.warmup_done = 0

    def put(self, a):
        a = np.ascontiguousarray(a)
        return self.torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(self.dev)

    def route_workspace(self, T, k, E):
        """The route sort's device workspace, allocated once outside the
        timed steps (None when the sort needs none)."""
        need = self.moe.route_sort_workspace_bytes(T, k, E)
        return self.torch.empty((need + 3) // 4, dtype=self.torch.int32, device=self.dev) if need else None

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def timed_steps(self, step, steps, warmup):
        """warmup untimed steps (and more until min_warmup_s has passed, for
        the shader clock to settle under sustained matrix work), then exactly
        `steps` steps between two device synchronisations; step(timed)
        returns its kernel events or None.  Returns (wall seconds, list of
        event tuples)."""
        n, t0 = 0, time.perf_counter()
        while n < warmup or time.perf_counter() - t0 < self.min_warmup_s:
            step(False)
            n += 1
            if n % 8 == 0:
                self.torch.cuda.synchronize()
        self.torch.cuda.synchronize()
        self.warmup_done = n
        ev = []
        t0 = time.perf_counter()
        for _ in range(steps):
            ev.append(step(True))
        self.torch.cuda.synchronize()
        return time.perf_counter() - t0, ev


def base_line(workload, steps, warmup, step_s, value, unit, dtype, config):
    cfg = {"workload": workload}
    cfg.update(config)
    return {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic", "config": cfg,
    }


def run_gmm(gpu, workload, steps, warmup, cpu_s, kernel="auto", out_dtype=None, tokens=None):
    """One grouped-matmul workload: route_sort + moe_gmm (+ moe_combine for
    the down projection) per step."""
    torch, moe = gpu.torch, gpu.moe
    from moe_grouped_gemm_route_amd.synth import make_config, make_ep_share, make_tokens_problem

    cfg = GMM_WORKLOADS[workload]
    ep = workload.startswith("ep8_")
    if ep:
        p = make_ep_share(cfg, gpus=8, rank=0)
    else:
        p = make_config(cfg) if tokens is None else make_tokens_problem(cfg, tokens)
    bf16_arm = workload.startswith("bf16_")
    fmt = "nvfp4" if workload in NVFP4_GMM else "mxfp4"
    out_dtype = out_dtype or p["out"]
    odt = moe.BF16 if out_dtype == "bf16" else moe.F32
    E, K, N, T, k = p["E"], p["K"], p["N"], p["T"], p["k"]
    M = T * k

    ids, x = gpu.put(p["topk_ids"]), gpu.put(p["x"])
    codes = gpu.put(p["codes"])
    packed = moe.mxfp4_encode(codes, gpu.put(p["scales"]), None, moe.MXFP4)
    wf = moe.MXFP4
    packed_mx = None
    if fmt == "nvfp4":
        # the same weights through the lossless cast; the MXFP4 kernel on the
        # MXFP4 pack is timed beside them
        bs, ts, err = moe.mxfp4_to_nvfp4(gpu.put(p["scales"]))
        assert err.item() == 0
        packed_mx, packed = packed, moe.mxfp4_encode(codes, bs, ts, moe.NVFP4)
        wf = moe.NVFP4
    del codes
    if bf16_arm:
        # the comparison arm streams the decoded weights as bf16
        dense = moe.debug_decode(packed, wf, E, N, K)
        packed_mx, packed = packed, moe.bf16_encode(dense)
        del dense
        fmt, wf = "bf16", moe.W_BF16
    tw = gpu.put(p["topk_weights"])
    # the down matmul's step ends with the combine; under expert parallelism
    # that runs on the tokens' own GPUs after the return exchange
    combine = cfg == 3 and not ep
    y = torch.empty((M, N), dtype=torch.bfloat16 if odt == moe.BF16 else torch.float32, device=gpu.dev)
    kern = KERNELS[kernel]
    ws = gpu.route_workspace(T, k, E)
    torch.cuda.synchronize()

    def gmm(pk, f, r):
        moe.moe_gmm(pk, f, E, N, K, x, r["group_offsets"], M,
                    row_index=r["sorted_token"] if p["gather"] else None,
                    out_dtype=odt, kernel=kern, out=y)

    def step(timed):
        r = moe.route_sort(ids, E, ws=ws)
        e = (gpu.event(), gpu.event()) if timed else None
        if timed:
            e[0].record()
        gmm(packed, wf, r)
        if timed:
            e[1].record()
        if combine:
            moe.moe_combine(y, tw, r["pair_row"])
        return e

    wall, ev = gpu.timed_steps(step, steps, warmup)

    mx_ms = None
    if packed_mx is not None:
        # the MXFP4 kernel on the same inputs, for the comparison
        r = moe.route_sort(ids, E, ws=ws)
        for _ in range(warmup):
            gmm(packed_mx, moe.MXFP4, r)
        e = [gpu.event() for _ in range(steps + 1)]
        e[0].record()
        for i in range(steps):
            gmm(packed_mx, moe.MXFP4, r)
            e[i + 1].record()
        torch.cuda.synchronize()
        mx_ms = [e[i].elapsed_time(e[i + 1]) for i in range(steps)]

    gmm_ms = [a.elapsed_time(b) for a, b in ev]
    gmm_s = float(np.mean(gmm_ms)) / 1e3
    nbytes, active = algorithmic_bytes(p, fmt)
    flops = 2.0 * M * K * N
    step_s = wall / steps
    roof = roofline(nbytes, flops, gmm_s)
    roof["traffic"] = recorded_traffic(workload) if tokens is None else None
    if roof["bound"] == "mfma":
        value, unit = flops / step_s / 1e12, "TFLOP/s"
    else:
        value, unit = nbytes / step_s / 1e9, "GB/s"
    config = {"tokens": T, "top_k": k, "experts": E, "K": K, "N": N, "routed_rows": M,
              "weights": fmt + (" (decoded MXFP4 weights)" if bf16_arm else ""),
              "activations": "bf16", "output": out_dtype, "kernel": kernel,
              "step": "route_sort + moe_gmm" + (" + moe_combine" if combine else "")}
    if ep:
        config["ep_share"] = ("GPU 0 of 8 after the dispatch: experts e % 8 == 0 of the 256, one top-1 row "
                              "per (token, slot) pair routed to them")
    out = base_line(workload, steps, gpu.warmup_done, step_s, value, unit, "bf16", config)
    out.update({
        "gmm_us": round(gmm_s * 1e6, 2),
        "gmm_us_median": round(float(np.median(gmm_ms)) * 1e3, 2),
        "gmm_us_min": round(float(np.min(gmm_ms)) * 1e3, 2),
        "gmm_tflops": round(flops / gmm_s / 1e12, 2),
        "gmm_gbs": round(nbytes / gmm_s / 1e9, 1),
        "active_experts": active,
        "algorithmic_bytes": int(nbytes),
        # + the output written and the index arrays read (band offsets, row index)
        "algorithmic_bytes_all": int(nbytes + M * N * (2 if odt == moe.BF16 else 4)
                                     + 4 * (E + 1) + (4 * M if p["gather"] else 0)),
        "roofline": roof,
    })
    if roof["bound"] == "mfma":
        out["mfma_calibration"] = mfma_calibration(gpu, roof["achieved"])
    if mx_ms is not None:
        mx_s = float(np.mean(mx_ms)) / 1e3
        out["mxfp4_us"] = round(mx_s * 1e6, 2)
        out["mxfp4_speedup_over_" + fmt] = round(gmm_s / mx_s, 3)
    if cpu_s > 0:
        out["cpu_baseline"] = cpu_baseline(p, "mxfp4" if bf16_arm else fmt, unit, target_s=cpu_s)
        out["gpu_over_cpu"] = round(value / out["cpu_baseline"]["value"], 1)
    return out


def run_layer(gpu, workload, steps, warmup, cpu_s):
    """One routed-expert layer (layer_decode, layer_prefill and its W4A4
    form)."""
    torch, moe = gpu.torch, gpu.moe
    from moe_grouped_gemm_route_amd.synth import make_layer_decode, make_layer_prefill

    prefill = workload in ("layer_prefill", "w4a4_layer_prefill")
    w4a4 = workload == "w4a4_layer_prefill"
    p = make_layer_prefill() if prefill else make_layer_decode()
    E, K, N, T, k = p["E"], p["K"], p["N"], p["T"], p["k"]
    M, H = T * k, N // 2
    ids, x, tw = gpu.put(p["topk_ids"]), gpu.put(p["x"]), gpu.put(p["topk_weights"])
    codes = gpu.put(p["codes"])
    w13 = moe.mxfp4_encode(codes, gpu.put(p["scales"]), None, moe.MXFP4)
    del codes
    codes = gpu.put(p["w2_codes"])
    w2 = moe.mxfp4_encode(codes, gpu.put(p["w2_scales"]), None, moe.MXFP4)
    del codes
    h = torch.empty((M, H), dtype=torch.bfloat16, device=gpu.dev)
    y2 = torch.empty((M, K), dtype=torch.float32, device=gpu.dev)
    ws = gpu.route_workspace(T, k, E)
    torch.cuda.synchronize()

    def step(timed):
        # events around each matmul kernel (the W4A4 quantizations fall between)
        e = [gpu.event() for _ in range(4)] if timed else None
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
        moe.moe_combine(y2, tw, r["pair_row"])
        return e

    wall, ev = gpu.timed_steps(step, steps, warmup)
    t13 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / 1e3
    t2 = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) / 1e3
    counts = np.bincount(p["topk_ids"].reshape(-1), minlength=E)
    active = int(np.count_nonzero(counts))
    if w4a4:
        # quantized activations: K/2 + K/32 bytes per row instead of 2K
        b13 = active * N * K * (0.5 + 1.0 / 32) + T * (K // 2 + K // 32)
        b2 = active * K * H * (0.5 + 1.0 / 32) + M * (H // 2 + H // 32)
    else:
        b13 = active * N * K * (0.5 + 1.0 / 32) + T * K * 2
        b2 = active * K * H * (0.5 + 1.0 / 32) + M * H * 2
    step_s = wall / steps
    flops = 2.0 * M * K * (N + H)
    roof = roofline(b13 + b2, flops, t13 + t2, FP4_PEAK_TFLOPS if w4a4 else BF16_PEAK_TFLOPS)
    roof["traffic"] = None
    if w4a4:
        roof["fp4_mfma_frac"] = round(flops / (t13 + t2) / (FP4_PEAK_TFLOPS * 1e12), 4)
    if roof["bound"] == "mfma" or prefill:
        value, unit = flops / step_s / 1e12, "TFLOP/s"
    else:
        value, unit = (b13 + b2) / step_s / 1e9, "GB/s"
    config = {"tokens": T, "top_k": k, "experts": E, "w13": [K, N], "w2": [H, K], "routed_rows": M,
              "weights": "mxfp4", "activations": "mxfp4 (quantized in the step)" if w4a4 else "bf16",
              "gate_up": "silu(gate) * up fused into the w13 epilogue",
              "step": ("route_sort + mxfp4_quantize(x) + moe_gmm_w4a4(w13, act) + mxfp4_quantize(h) "
                       "+ moe_gmm_w4a4(w2) + moe_combine") if w4a4 else
                      "route_sort + moe_gmm(w13, act) + moe_gmm(w2) + moe_combine"}
    out = base_line(workload, steps, gpu.warmup_done, step_s, value, unit, "fp4" if w4a4 else "bf16", config)
    out.update({
        "w13_us": round(t13 * 1e6, 2),
        "w2_us": round(t2 * 1e6, 2),
        "active_experts": active,
        "algorithmic_bytes": int(b13 + b2),
        "layer_tflops": round(flops / (t13 + t2) / 1e12, 2),
        "roofline": roof,
    })
    if roof["bound"] == "mfma" and not w4a4:
        out["mfma_calibration"] = mfma_calibration(gpu, roof["achieved"])
    if cpu_s > 0 and not w4a4:
        out["cpu_baseline"] = layer_cpu_baseline(p, unit, target_s=cpu_s)
        out["gpu_over_cpu"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    return out


def run_route(gpu, workload, steps, warmup):
    """The route sort alone, back to back on one routing (its workspace
    allocated once): token-expert pairs sorted per second."""
    moe = gpu.moe
    from moe_grouped_gemm_route_amd.synth import make_config

    p = make_config(ROUTE_WORKLOADS[workload])
    E, T, k = p["E"], p["T"], p["k"]
    ids = gpu.put(p["topk_ids"])
    ws = gpu.route_workspace(T, k, E)

    def step(timed):
        e = (gpu.event(), gpu.event()) if timed else None
        if timed:
            e[0].record()
        moe.route_sort(ids, E, ws=ws)
        if timed:
            e[1].record()
        return e

    wall, ev = gpu.timed_steps(step, steps, warmup)
    sort_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    step_s = wall / steps
    config = {"tokens": T, "top_k": k, "experts": E, "pairs": T * k,
              "workspace_bytes": moe.route_sort_workspace_bytes(T, k, E), "step": "route_sort"}
    out = base_line(workload, steps, gpu.warmup_done, step_s, T * k / step_s / 1e6, "Mpairs/s", "int32", config)
    out["route_sort_us"] = round(sort_s * 1e6, 2)
    return out


def run_w4a4(gpu, workload, steps, warmup):
    """The W4A4 workloads: route-sort, MXFP4 activation quantization and the
    grouped matmul on the scaled FP4 MFMA, over config 4's problem (MXFP4
    weights, or NVFP4 ones from the library's lossless cast) or config 5's
    (NVFP4 by the cast)."""
    torch, moe = gpu.torch, gpu.moe
    from moe_grouped_gemm_route_amd.synth import make_config

    cfg, wfmt = W4A4_WORKLOADS[workload]
    p = make_config(cfg)
    E, K, N, T, k = p["E"], p["K"], p["N"], p["T"], p["k"]
    M = T * k
    ids, x = gpu.put(p["topk_ids"]), gpu.put(p["x"])
    codes = gpu.put(p["codes"])
    if wfmt == "mxfp4":
        packed = moe.mxfp4_encode(codes, gpu.put(p["scales"]), None, moe.MXFP4)
        wf = moe.MXFP4
    else:
        bs, ts, err = moe.mxfp4_to_nvfp4(gpu.put(p["scales"]))
        assert err.item() == 0
        packed = moe.mxfp4_encode(codes, bs, ts, moe.NVFP4)
        wf = moe.NVFP4
    del codes
    y = torch.empty((M, N), dtype=torch.float32, device=gpu.dev)
    ws = gpu.route_workspace(T, k, E)
    bad = torch.zeros(1, dtype=torch.int32, device=gpu.dev)
    torch.cuda.synchronize()

    def step(timed):
        r = moe.route_sort(ids, E, ws=ws)
        qc, qs = moe.mxfp4_quantize(x)
        e = (gpu.event(), gpu.event()) if timed else None
        if timed:
            e[0].record()
        moe.moe_gmm_w4a4(packed, E, N, K, qc, qs, r["group_offsets"], M, row_index=r["sorted_token"], out=y,
                         fmt=wf, err_count=bad if wf == moe.NVFP4 else None)
        if timed:
            e[1].record()
        return e

    wall, ev = gpu.timed_steps(step, steps, warmup)
    gmm_ms = [a.elapsed_time(b) for a, b in ev]
    gmm_s = float(np.mean(gmm_ms)) / 1e3
    flops = 2.0 * M * K * N
    assert bad.item() == 0
    counts = np.bincount(p["topk_ids"].reshape(-1), minlength=E)
    active = int(np.count_nonzero(counts))
    per_weight = 0.5 + (1.0 / 32 if wfmt == "mxfp4" else 1.0 / 16)
    nbytes = active * N * K * per_weight + (active * 4 if wfmt == "nvfp4" else 0) + T * (K // 2 + K // 32)
    step_s = wall / steps
    roof = roofline(nbytes, flops, gmm_s, FP4_PEAK_TFLOPS)
    roof["traffic"] = recorded_traffic(workload)
    roof["fp4_mfma_frac"] = round(flops / gmm_s / 1e12 / FP4_PEAK_TFLOPS, 4)
    config = {"tokens": T, "top_k": k, "experts": E, "K": K, "N": N, "routed_rows": M,
              "weights": wfmt + (" (from the lossless cast)" if wfmt == "nvfp4" else ""),
              "activations": "mxfp4 (quantized in the step)", "output": "f32",
              "step": "route_sort + mxfp4_quantize + moe_gmm_w4a4"}
    rate, unit = (flops / step_s / 1e12, "TFLOP/s") if roof["bound"] == "mfma" or cfg == 4 else \
        (nbytes / step_s / 1e9, "GB/s")
    out = base_line(workload, steps, gpu.warmup_done, step_s, rate, unit, "fp4", config)
    out.update({
        "gmm_us": round(gmm_s * 1e6, 2),
        "gmm_us_median": round(float(np.median(gmm_ms)) * 1e3, 2),
        "gmm_us_min": round(float(np.min(gmm_ms)) * 1e3, 2),
        "gmm_tflops": round(flops / gmm_s / 1e12, 2),
        "active_experts": active,
        "algorithmic_bytes": int(nbytes),
        "roofline": roof,
    })
    return out


CALIB_BLOCKS, CALIB_ITERS = 512, 12800     # two workgroups per CU, about 25 ms per launch
HBM_CALIB_BYTES, HBM_CALIB_BLOCKS = 2 << 30, 1536   # regions of 341 KiB per wave: not a power of two


def mfma_calibration(gpu, achieved_tflops):
    """The bf16 matrix-unit rate this part sustains with no memory traffic
    (moe_calib_mfma_bf16: the tiled kernel's 128 x 64 wave tile of 16x16x32
    MFMAs on register-resident N(0,1) activations and decoded MXFP4 weights),
    the median of 3 launches after one warm-up, with the matmul's achieved
    rate as a fraction of it.  Measured after the timed steps; the roofline
    fraction stays the one against the published peak."""
    torch, moe = gpu.torch, gpu.moe
    from moe_grouped_gemm_route_amd.synth import make_problem

    q = make_problem(T=2048, k=1, E=1, K=4096, N=1024, seed=41)
    a = gpu.put(q["x"])
    packed = moe.mxfp4_encode(gpu.put(q["codes"]), gpu.put(q["scales"]), None, moe.MXFP4)
    b = moe.debug_decode(packed, moe.MXFP4, 1, 1024, 4096)
    moe.calib_mfma_bf16(a, b, CALIB_BLOCKS, CALIB_ITERS)
    ms = []
    for _ in range(3):
        e0, e1 = gpu.event(), gpu.event()
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


def prefill_breakdown(gpu):
    """The tiled kernel's wave tile built up from the matrix unit alone
    (moe_calib_mfma_parts), one part of its data movement at a time, then all
    of it, then all of it at 6 of 8 row subtiles (bands of about 96 rows).
    Operands as in mfma_calibration; 512 workgroups of 4 waves over 8,000
    chunks per wave (about 20-40 ms per launch); codes from a 2 GiB buffer,
    staging from 1 MiB (L2 hits) or 32 MiB (misses).  Best and median of 4
    launches after one warm-up."""
    torch, moe = gpu.torch, gpu.moe
    from moe_grouped_gemm_route_amd.synth import make_problem

    q = make_problem(T=2048, k=1, E=1, K=4096, N=1024, seed=41)
    a = gpu.put(q["x"])
    packed = moe.mxfp4_encode(gpu.put(q["codes"]), gpu.put(q["scales"]), None, moe.MXFP4)
    b = moe.debug_decode(packed, moe.MXFP4, 1, 1024, 4096)
    del packed
    g = torch.Generator(device=gpu.dev)
    g.manual_seed(43)
    codes = torch.randint(0, 256, (2 << 30,), dtype=torch.uint8, device=gpu.dev, generator=g)
    x = torch.randn(16 << 20, dtype=torch.float32, device=gpu.dev, generator=g).to(torch.bfloat16)
    blocks, chunks = CALIB_BLOCKS, 8000
    P = moe
    rows = [
        ("operands in registers", 0, 8, 0),
        ("a barrier per chunk", P.PARTS_BARRIER, 8, 0),
        ("decode of register-held codes that change every chunk", P.PARTS_REG_DECODE, 8, 0),
        ("A fragments read from LDS", P.PARTS_LDS_A, 8, 0),
        ("activation chunks staged to LDS from 1 MiB (L2 hits), wait and barrier", P.PARTS_STAGE, 8, 1),
        ("the same staging from 32 MiB (L2 misses)", P.PARTS_STAGE, 8, 32),
        ("codes streamed from HBM, only XOR-ed", P.PARTS_CODES_XOR, 8, 0),
        ("codes streamed from HBM and decoded", P.PARTS_CODES, 8, 0),
        ("all: LDS A reads, code stream and decode, staging from 1 MiB",
         P.PARTS_LDS_A | P.PARTS_CODES | P.PARTS_STAGE, 8, 1),
        ("all, staging from 32 MiB", P.PARTS_LDS_A | P.PARTS_CODES | P.PARTS_STAGE, 8, 32),
        ("all at 6 of 8 row subtiles, staging from 1 MiB", P.PARTS_LDS_A | P.PARTS_CODES | P.PARTS_STAGE, 6, 1),
        ("all at 6 of 8 row subtiles, staging from 32 MiB", P.PARTS_LDS_A | P.PARTS_CODES | P.PARTS_STAGE, 6, 32),
    ]
    out = []
    for label, parts, rows16, xmib in rows:
        xs = x[: (max(xmib, 1) << 20) // 2]
        run = lambda: moe.calib_mfma_parts(parts, rows16, a, b, codes, xs, 2.0 ** -5, blocks, chunks)
        run()
        ms = []
        for _ in range(4):
            e0, e1 = gpu.event(), gpu.event()
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        flops = blocks * 4.0 * chunks * 4 * rows16 * 4 * 16384
        rec = {"label": label, "parts": parts, "rows16": rows16,
               "pflops_best": round(flops / (min(ms) / 1e3) / 1e15, 3),
               "pflops_median": round(flops / (float(np.median(ms)) / 1e3) / 1e15, 3),
               "ms_median": round(float(np.median(ms)), 2)}
        if parts & (P.PARTS_CODES | P.PARTS_CODES_XOR):
            rec["codes_tbs"] = round(blocks * 4.0 * chunks * 4096 / (float(np.median(ms)) / 1e3) / 1e12, 2)
        out.append(rec)
        print("bench: %s %.3f PFLOP/s" % (label, rec["pflops_median"]), file=sys.stderr, flush=True)
    return {"blocks": blocks, "chunks": chunks, "rows": out}


def library_matmul(gpu):
    """A plain bf16 torch.matmul (hipBLASLt) of the 4,096-token w13 prefill's
    shape, [24,576 x 4,096] x [4,096 x 4,096], N(0,1) operands: warmed up for
    half a second (the shader clock settles under sustained matrix work),
    then 20 launches timed with HIP events; median and best."""
    torch = gpu.torch
    g = torch.Generator(device=gpu.dev)
    g.manual_seed(44)
    M, K, N = 24576, 4096, 4096
    A = torch.randn((M, K), dtype=torch.float32, device=gpu.dev, generator=g).to(torch.bfloat16)
    B = torch.randn((K, N), dtype=torch.float32, device=gpu.dev, generator=g).to(torch.bfloat16).contiguous()
    C = torch.empty((M, N), dtype=torch.bfloat16, device=gpu.dev)
    t0 = time.time()
    while time.time() - t0 < 0.5:
        for _ in range(8):
            torch.matmul(A, B, out=C)
        torch.cuda.synchronize()
    ev = [gpu.event() for _ in range(21)]
    ev[0].record()
    for i in range(20):
        torch.matmul(A, B, out=C)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(20)]
    flops = 2.0 * M * K * N
    return {"shape": [M, K, N], "us_median": round(float(np.median(ms)) * 1e3, 1),
            "us_min": round(min(ms) * 1e3, 1),
            "pflops_median": round(flops / (float(np.median(ms)) / 1e3) / 1e15, 3)}


def hbm_calibration(gpu):
    """The HBM read rate this part sustains (moe_calib_hbm_read: 16-byte
    non-temporal loads, each wave reading contiguous 1 KiB runs, over a 2 GiB
    buffer, eight times the last-level cache), median of 5 launches after
    one warm-up."""
    torch, moe = gpu.torch, gpu.moe
    buf = torch.ones(HBM_CALIB_BYTES // 4, dtype=torch.int32, device=gpu.dev)
    moe.calib_hbm_read(buf, HBM_CALIB_BLOCKS)
    ms = []
    for _ in range(5):
        e0, e1 = gpu.event(), gpu.event()
        e0.record()
        moe.calib_hbm_read(buf, HBM_CALIB_BLOCKS)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del buf
    gbs = HBM_CALIB_BYTES / (float(np.median(ms)) / 1e3) / 1e9
    return {"read_gbs": round(gbs, 1),
            "loop": "%d MiB read with 16-byte loads, %d workgroups of 256 threads, %.3f ms per launch"
                    % (HBM_CALIB_BYTES >> 20, HBM_CALIB_BLOCKS, float(np.median(ms)))}


def mixed_calibration(gpu):
    """HBM rates of plain PyTorch kernels whose reads and writes come in a
    fixed ratio (f32): a copy (1:1) and sums over the leading dimension of
    [2, n] and [6, n] tensors (2:1, 6:1).  Reference figures for the kernels
    that also write what they read (the combine reads six rows per row
    written); medians of 20 launches after 3 warm-up launches."""
    torch = gpu.torch

    def rate(fn, nbytes):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [gpu.event() for _ in range(21)]
        ev[0].record()
        for i in range(20):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        s = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(20)])) / 1e3
        return {"us": round(s * 1e6, 1), "gbs": round(nbytes / s / 1e9, 1)}

    out = {}
    n = 256 << 20
    src = torch.ones(n, dtype=torch.float32, device=gpu.dev)
    dst = torch.empty_like(src)
    out["copy_1gib"] = rate(lambda: dst.copy_(src), 2 * n * 4)
    del src, dst
    for rows, n in ((2, 64 << 20), (6, 4096 * 4096)):
        a = torch.ones((rows, n), dtype=torch.float32, device=gpu.dev)
        o = torch.empty(n, dtype=torch.float32, device=gpu.dev)
        out["sum_%d_rows_of_%d" % (rows, n)] = rate(lambda: torch.sum(a, dim=0, out=o), (rows + 1) * n * 4)
        del a, o
    return out


def with_hbm_fraction(line, calib):
    """Adds the kernel's fraction of the calibrated read rate to an
    HBM-bound line."""
    if line.get("roofline", {}).get("bound") == "hbm":
        line["hbm_calibration"] = dict(calib)
        line["hbm_calibration"]["kernel_frac_of_read"] = round(line["roofline"]["achieved"] / calib["read_gbs"], 4)
    return line


def summary(line):
    """The compact record of a workload timed after the headline."""
    keep = ("steps", "warmup", "ms_per_step", "value", "unit", "dtype", "config", "gmm_us", "gmm_us_median",
            "gmm_us_min", "w13_us", "w2_us", "active_experts", "algorithmic_bytes", "roofline",
            "mfma_calibration", "hbm_calibration", "cpu_baseline", "gpu_over_cpu")
    out = {key: line[key] for key in keep if key in line}
    out.update({key: v for key, v in line.items() if key.startswith("mxfp4_")})
    return out


def run_workload(gpu, name, steps, warmup, cpu_s, args):
    if name in LAYER_WORKLOADS:
        return run_layer(gpu, name, steps, warmup, cpu_s)
    if name in W4A4_WORKLOADS:
        return run_w4a4(gpu, name, steps, warmup)
    if name in ROUTE_WORKLOADS:
        return run_route(gpu, name, steps, warmup)
    return run_gmm(gpu, name, steps, warmup, cpu_s, kernel=args.kernel, out_dtype=args.out_dtype,
                   tokens=args.tokens)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.0,
                    help="keep warming up the named workload until this much time has passed")
    ap.add_argument("--workload", default="w13_decode", choices=WORKLOADS)
    ap.add_argument("--tokens", type=int, default=None,
                    help="token count in place of the workload's (grouped-matmul workloads only)")
    ap.add_argument("--kernel", default="auto", choices=sorted(KERNELS))
    ap.add_argument("--out-dtype", default=None, choices=["f32", "bf16"])
    ap.add_argument("--only", action="store_true",
                    help="time the named workload alone (no other workloads after the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-breakdown", action="store_true",
                    help="only print the matrix-unit rate of the tiled kernel's wave tile with each "
                         "part of its data movement added (moe_calib_mfma_parts), and a plain bf16 "
                         "torch.matmul of the 4,096-token w13 shape")
    ap.add_argument("--mixed-calibration", action="store_true",
                    help="only print the HBM rates of plain PyTorch copy and row-sum kernels "
                         "(read:write 1:1, 2:1 and 6:1)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer --steps times (a plain copy "
                         "kernel of known size, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the routed-expert matmul would shard by experts, 32 per GPU on 8 GPUs)",
              file=sys.stderr)
        sys.exit(2)
    if args.tokens is not None and args.workload not in GMM_WORKLOADS:
        print("--tokens applies to the grouped-matmul workloads only", file=sys.stderr)
        sys.exit(2)

    gpu = Gpu()
    if args.prefill_breakdown:
        print(json.dumps({"prefill_breakdown": prefill_breakdown(gpu), "library_matmul": library_matmul(gpu)}),
              flush=True)
        return
    if args.mixed_calibration:
        print(json.dumps({"mixed_calibration": mixed_calibration(gpu)}), flush=True)
        return
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = gpu.torch.ones(n, dtype=gpu.torch.uint8, device=gpu.dev)
        dst = gpu.torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        gpu.torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps}), flush=True)
        return

    cpu_s = 0.0 if args.no_cpu_baseline else 15.0
    gpu.min_warmup_s = args.warmup_seconds
    line = run_workload(gpu, args.workload, args.steps, args.warmup, cpu_s, args)
    extras = args.workload == "w13_decode" and not args.only and args.tokens is None
    calib = hbm_calibration(gpu) if (line.get("roofline", {}).get("bound") == "hbm" or extras) else None
    if calib is not None:
        with_hbm_fraction(line, calib)
    if extras:
        sub_args = argparse.Namespace(**vars(args))
        sub_args.kernel, sub_args.out_dtype, sub_args.tokens = "auto", None, None
        sub_cpu = 0.0 if args.no_cpu_baseline else 3.0
        work = {}
        # each workload warms up for at least a quarter second: the matrix-bound
        # ones reach their steady clock after a few dozen calls
        gpu.min_warmup_s = 0.25
        for name in EXTRA_WORKLOADS:
            sub = run_workload(gpu, name, min(args.steps, 20), min(args.warmup, 5), sub_cpu, sub_args)
            work[name] = summary(with_hbm_fraction(sub, calib))
            print("bench: %s done" % name, file=sys.stderr, flush=True)
        line["workloads"] = work
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
