"""Shared helpers of the GPU parity tests: run the HIP path through the
binding on a synthetic problem, and compare against the oracle."""

import numpy as np
import torch

import moe_grouped_gemm_route_amd as moe
import oracle

DEV = "cuda"
REL_TOL = 1e-5        # max|gpu - oracle| / max|oracle| for f32 outputs


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def weights_for(p, fmt):
    """Oracle weight dict and device tensors for format fmt ('mxfp4'|'nvfp4').
    NVFP4 scales come from the oracle's lossless cast of the MXFP4 scales."""
    if fmt == "mxfp4":
        w = {"fmt": "mxfp4", "codes": p["codes"], "scales": p["scales"]}
        packed = moe.mxfp4_encode(to_dev(p["codes"]), to_dev(p["scales"]), None, moe.MXFP4)
    else:
        if "block_scales" in p:
            bs, ts = p["block_scales"], p["tensor_scale"]
        else:
            bs, ts = oracle.mxfp4_to_nvfp4(p["scales"])
        w = {"fmt": "nvfp4", "codes": p["codes"], "block_scales": bs, "tensor_scale": ts}
        packed = moe.mxfp4_encode(to_dev(p["codes"]), to_dev(bs), to_dev(ts), moe.NVFP4)
    return w, packed


def run_gpu(p, packed, fmt, kernel=moe.GMM_AUTO, out_dtype=moe.F32, routed=None, act=moe.ACT_NONE):
    """Route-sort on the GPU, then moe_gmm.  Returns (route dict, y tensor)."""
    E, K, N = p["E"], p["K"], p["N"]
    M = p["T"] * p["k"]
    r = routed if routed is not None else moe.route_sort(to_dev(p["topk_ids"]), E)
    x = to_dev(p["x"])
    f = {"mxfp4": moe.MXFP4, "nvfp4": moe.NVFP4, "bf16": moe.W_BF16}[fmt]
    y = moe.moe_gmm(packed, f, E, N, K, x, r["group_offsets"], M,
                    row_index=r["sorted_token"] if p["gather"] else None,
                    out_dtype=out_dtype, kernel=kernel, act=act)
    return r, y


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


def bf16_bits_to_f64(bits):
    from oracle.gmm import bf16_bits_to_f64 as to_f64
    return to_f64(np.asarray(bits).view(np.uint16))


def bf16_ulp(ref):
    """One bf16 unit in the last place at |ref| (normal range)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def _expert_slice(w, e):
    """The one-expert weight dict of expert e (the oracle's own format)."""
    sub = {"fmt": w["fmt"], "codes": w["codes"][e:e + 1]}
    if w["fmt"] == "mxfp4":
        sub["scales"] = w["scales"][e:e + 1]
    else:
        sub["block_scales"] = w["block_scales"][e:e + 1]
        sub["tensor_scale"] = np.asarray(w["tensor_scale"])[e:e + 1]
    return sub


def oracle_gmm_bands(x_bits, row_index, group_offsets, w, experts=None, quantized=None):
    """The oracle's grouped matmul over the bands of the given experts (all by
    default), one oracle.gmm call per expert on that expert's slice, spread
    over host threads (numpy releases the GIL in the decode and the matmul).
    quantized = (codes, scales) of MXFP4 activations runs oracle.gmm_w4a4
    instead.  Returns {expert: [band rows, N] float64}."""
    import concurrent.futures
    import os
    off = np.asarray(group_offsets, dtype=np.int64)
    if experts is None:
        experts = [e for e in range(off.size - 1) if off[e + 1] > off[e]]

    def one(e):
        lo, hi = int(off[e]), int(off[e + 1])
        sub_off = np.array([0, hi - lo], dtype=np.int64)
        ri = None if row_index is None else np.asarray(row_index)[lo:hi]
        if quantized is not None:
            qc, qs = quantized
            if row_index is None:
                qc, qs = qc[lo:hi], qs[lo:hi]
            return e, oracle.gmm_w4a4(qc, qs, ri, sub_off, _expert_slice(w, e))
        xs = x_bits if row_index is not None else x_bits[lo:hi]
        return e, oracle.gmm(xs, ri, sub_off, _expert_slice(w, e))

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        return dict(ex.map(one, experts))
