"""Seeded synthetic inputs for the routed-expert grouped matmul.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic (no decoding, scaling, sorting or matmul).  The CPU oracle
and the HIP path are both fed from it.

Workload shapes follow the pages' grouped-matmul benchmark ("Running DeepSeek
V4 Flash on TPU v6", section "Grouped matmul performance vs bf16": 256 experts,
random top-6 routing, the fused gate/up weight with K = N = 4096 and the down
weight with K = 2048, N = 4096) and the model's sizes ("DeepSeek-V4-Flash"
PocketLLM docs, section "Model specification": hidden 4096, expert
intermediate 2048, 256 routed experts, top-6).  Real checkpoint weights are not
available, so codes and scales are random with the recipe below.

Recipe (per problem, numpy PCG64 seeded with ``seed``; draws in this order):
1. x: float32 standard normal, rounded to bf16 with round-to-nearest-even,
   returned as uint16 bit patterns.
2. routing keys [T, E]: uniform keys, or for Zipf routing log p_e plus
   standard Gumbel noise with p_e proportional to (e + 1)^-s; each token takes
   the k largest keys (descending), so ids are distinct within a token.
   Forced-empty experts get a key below every other.
3. codes [E, N, K/2]: raw little-endian bytes of the generator's 64-bit output
   (every nibble uniform over the 16 e2m1 codes, -0 included).
4. scales [E, N, K/32]: E8M0 bytes 127 + uniform integer in [lo, hi].
5. router logits [T, k] standard normal; weights are their softmax over the k
   slots (float64, stored float32).
"""

from functools import lru_cache

import numpy as np


def f32_to_bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_bf16_bits(rng, shape):
    """Fast seeded bf16 bit patterns for very large activation matrices:
    random sign and 7-bit mantissa, exponent uniform over 2^-4 .. 2^3 (so
    magnitudes in [1/16, 16)).  Two uint16 draws from rng, in this order."""
    a = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    e = rng.integers(123, 131, size=shape, dtype=np.uint16)
    return (a & np.uint16(0x807F)) | (e << np.uint16(7))


def _topk_desc(keys, k):
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def make_problem(*, T, k, E, K, N, seed, routing="uniform", zipf_s=1.1,
                 exp_range=(-8, -3), empty_experts=(), x_rows=None):
    """Draw one routed grouped-matmul problem.

    x_rows: number of activation rows; None means T (the gate/up matmul
    gathers token rows), an int M means an [M, K] input already in band order
    (the down matmul).
    Returns a dict of numpy arrays plus the shape fields."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    rows = T if x_rows is None else int(x_rows)
    x = f32_to_bf16_bits(rng.standard_normal((rows, K), dtype=np.float32))
    if routing == "uniform":
        keys = rng.random((T, E))
    elif routing == "zipf":
        logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        keys = logp[None, :] + rng.gumbel(size=(T, E))
    else:
        raise ValueError("routing must be 'uniform' or 'zipf'")
    for e in empty_experts:
        keys[:, e] = -np.inf
    if k > E - len(empty_experts):
        raise ValueError("top-k larger than the number of selectable experts")
    topk_ids = _topk_desc(keys, k)
    n_bytes = E * N * (K // 2)
    raw = rng.bit_generator.random_raw((n_bytes + 7) // 8).view(np.uint8)[:n_bytes]
    codes = raw.reshape(E, N, K // 2)
    lo, hi = exp_range
    scales = (rng.integers(lo, hi + 1, size=(E, N, K // 32)) + 127).astype(np.uint8)
    logits = rng.standard_normal((T, k))
    ez = np.exp(logits - logits.max(axis=1, keepdims=True))
    topk_weights = (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)
    return {
        "T": T, "k": k, "E": E, "K": K, "N": N,
        "gather": x_rows is None,
        "x": x, "topk_ids": topk_ids, "topk_weights": topk_weights,
        "codes": codes, "scales": scales,
    }


# The five benchmark workloads.  Shapes and routing follow the pages' MoE
# (see the module docstring); config 5 reuses config 2's weights.
CONFIGS = {
    1: dict(name="tiny", T=64, k=2, E=8, K=256, N=512, routing="uniform",
            exp_range=(-6, -2), empty_experts=(7,), out="f32"),
    2: dict(name="w13_decode", T=64, k=6, E=256, K=4096, N=4096, routing="uniform",
            exp_range=(-8, -3), out="bf16"),
    3: dict(name="w2_decode", T=256, k=6, E=256, K=2048, N=4096, routing="zipf",
            exp_range=(-8, -3), band_input=True, out="f32"),
    4: dict(name="w13_prefill", T=4096, k=6, E=256, K=4096, N=4096, routing="uniform",
            exp_range=(-8, -3), out="f32"),
    5: dict(name="nvfp4_w13", T=256, k=6, E=256, K=4096, N=4096, routing="uniform",
            exp_range=(-8, -3), out="f32", weights_from=2),
}


@lru_cache(maxsize=2)
def make_config(i):
    """The benchmark workload number i (1..5), seeded with i.

    Config 5 takes config 2's codes and E8M0 scales (seed 2) with its own
    activations and routing (seed 5); its NVFP4 scales are derived from them
    by the consumer with the lossless cast."""
    c = CONFIGS[i]
    p = make_problem(T=c["T"], k=c["k"], E=c["E"], K=c["K"], N=c["N"], seed=i,
                     routing=c["routing"], exp_range=c["exp_range"],
                     empty_experts=c.get("empty_experts", ()),
                     x_rows=c["T"] * c["k"] if c.get("band_input") else None) \
        if "weights_from" not in c else None
    if p is None:
        src = make_config(c["weights_from"])
        q = make_problem(T=c["T"], k=c["k"], E=c["E"], K=c["K"], N=8, seed=i,
                         routing=c["routing"], exp_range=c["exp_range"])
        p = dict(q)
        p["N"] = c["N"]
        p["codes"], p["scales"] = src["codes"], src["scales"]
    p["name"] = c["name"]
    p["out"] = c["out"]
    p["config"] = i
    return p


def make_tokens_problem(cfg, T):
    """Config cfg's weights with T tokens: x and routing drawn like the
    config's (same routing law and top-k; seed 1000 * cfg + T), the codes and
    scales taken from make_config(cfg).  For a band-ordered input (the down
    matmul) x has T * k rows."""
    c = CONFIGS[cfg]
    src = make_config(c.get("weights_from", cfg))
    q = make_problem(T=T, k=c["k"], E=c["E"], K=c["K"], N=8, seed=1000 * cfg + T,
                     routing=c["routing"], exp_range=c["exp_range"],
                     empty_experts=c.get("empty_experts", ()),
                     x_rows=T * c["k"] if c.get("band_input") else None)
    p = dict(q)
    p["N"] = c["N"]
    p["codes"], p["scales"] = src["codes"], src["scales"]
    p["name"] = "%s_%dtok" % (c["name"], T)
    p["out"] = c["out"]
    p["config"] = cfg
    return p


def make_ep_share(cfg, gpus=8, rank=0):
    """Config cfg as GPU `rank` holds it when the experts are dealt
    round-robin to `gpus` GPUs (expert e on GPU e % gpus, which spreads a
    Zipf head over the GPUs; rank 0 holds expert 0, the hottest), after the
    dispatch: its E / gpus experts under local ids e // gpus, and one row per
    (token, slot) pair routed to them, in pair order, each routed top-1 to its
    local expert.  A gate/up problem receives the pairs' token rows, which the
    local sort gathers again; a band-ordered input (the down matmul, fed by the
    local gate/up output) takes the config's first rows."""
    p = make_config(cfg)
    if p["E"] % gpus:
        raise ValueError("the experts must divide evenly over the GPUs")
    ids = p["topk_ids"].reshape(-1)
    mine = np.nonzero(ids % gpus == rank)[0]
    M = len(mine)
    q = dict(p)
    q["E"], q["T"], q["k"] = p["E"] // gpus, M, 1
    q["topk_ids"] = (ids[mine] // gpus).astype(np.int32).reshape(M, 1)
    q["topk_weights"] = p["topk_weights"].reshape(-1)[mine].reshape(M, 1)
    q["codes"] = np.ascontiguousarray(p["codes"][rank::gpus])
    q["scales"] = np.ascontiguousarray(p["scales"][rank::gpus])
    q["x"] = p["x"][mine // p["k"]] if p["gather"] else p["x"][:M]
    q["name"] = "ep%d_%s" % (gpus, p["name"])
    return q


@lru_cache(maxsize=1)
def make_layer_decode():
    """One MoE layer at decode: config 2's tokens, routing, router weights and
    fused gate+up (w13) weights, plus down-projection (w2) weights of the
    expert intermediate size (K = 2048, N = 4096) drawn with seed 6 (only
    their codes and scales are taken from that draw)."""
    return _layer(2, "layer_decode")


def make_layer_prefill():
    """One MoE layer at prefill: config 4's 4096 tokens, routing, router
    weights and w13 weights, plus the same w2 weights as make_layer_decode."""
    return _layer(4, "layer_prefill")


def _layer(cfg, name):
    p = dict(make_config(cfg))
    w2 = make_problem(T=8, k=6, E=p["E"], K=p["N"] // 2, N=p["K"], seed=6,
                      exp_range=CONFIGS[2]["exp_range"])
    p["w2_codes"], p["w2_scales"] = w2["codes"], w2["scales"]
    p["name"] = name
    return p

