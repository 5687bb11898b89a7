"""The seeded input generator: determinism, shapes and workload structure."""

import numpy as np
import torch

from moe_grouped_gemm_route_amd.synth import (
    CONFIGS, f32_to_bf16_bits, make_config, make_problem)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.0, 0.0, -0.0], dtype=np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(a), ref)


def test_same_seed_same_bytes():
    a = make_problem(T=8, k=2, E=4, K=64, N=16, seed=9)
    b = make_problem(T=8, k=2, E=4, K=64, N=16, seed=9)
    for key in ("x", "topk_ids", "topk_weights", "codes", "scales"):
        assert np.array_equal(a[key], b[key])
    c = make_problem(T=8, k=2, E=4, K=64, N=16, seed=10)
    assert not np.array_equal(a["codes"], c["codes"])


def test_routing_does_not_depend_on_weight_shape():
    a = make_problem(T=64, k=6, E=256, K=4096, N=8, seed=2)
    b = make_problem(T=64, k=6, E=256, K=4096, N=16, seed=2)
    assert np.array_equal(a["topk_ids"], b["topk_ids"]) and np.array_equal(a["x"], b["x"])


def test_config1_structure():
    c = make_config(1)
    assert c["x"].shape == (64, 256) and c["x"].dtype == np.uint16
    assert c["codes"].shape == (8, 512, 128) and c["scales"].shape == (8, 512, 8)
    assert not np.any(c["topk_ids"] == 7)
    for row in c["topk_ids"]:
        assert len(set(row.tolist())) == 2
    s = c["scales"].astype(int) - 127
    assert s.min() >= -6 and s.max() <= -2
    assert np.allclose(c["topk_weights"].sum(axis=1), 1.0, atol=1e-6)


def test_zipf_routing_is_skewed_and_distinct():
    c = CONFIGS[3]
    p = make_problem(T=c["T"], k=c["k"], E=c["E"], K=32, N=1, seed=3, routing="zipf")
    ids = p["topk_ids"]
    for row in ids:
        assert len(set(row.tolist())) == 6
    cnt = np.bincount(ids.reshape(-1), minlength=256)
    assert cnt[0] > 150 and cnt[0] == cnt.max()
    assert np.sum(cnt == 0) > 10


def test_code_nibbles_cover_all_16_values_uniformly():
    p = make_problem(T=4, k=2, E=2, K=1024, N=64, seed=1)
    nib = np.concatenate([p["codes"] & 0xF, p["codes"] >> 4]).reshape(-1)
    cnt = np.bincount(nib, minlength=16)
    assert cnt.min() > 0.8 * cnt.mean()


def test_random_bf16_bits_range_and_determinism():
    from moe_grouped_gemm_route_amd.synth import random_bf16_bits, bf16_bits_to_f32
    a = random_bf16_bits(np.random.default_rng(5), (300, 64))
    b = random_bf16_bits(np.random.default_rng(5), (300, 64))
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    v = np.abs(bf16_bits_to_f32(a))
    assert v.min() >= 1.0 / 16 and v.max() < 16.0
    assert 0.4 < np.mean(a >> 15) < 0.6                        # both signs


def test_ep_share_partitions_the_pairs():
    # the 8 shares of the w13 decode workload together hold every (token,
    # slot) pair once, each with its token's row, its router weight and its
    # expert's weights under local id e // 8
    from moe_grouped_gemm_route_amd.synth import make_config, make_ep_share
    p = make_config(2)
    ids = p["topk_ids"].reshape(-1)
    seen = np.zeros(ids.size, dtype=np.int64)
    for rank in range(8):
        q = make_ep_share(2, gpus=8, rank=rank)
        assert q["E"] == 32 and q["k"] == 1 and q["gather"]
        pairs = np.nonzero(ids % 8 == rank)[0]
        seen[pairs] += 1
        assert q["T"] == pairs.size
        assert np.array_equal(q["topk_ids"].reshape(-1) * 8 + rank, ids[pairs])
        assert np.array_equal(q["topk_weights"].reshape(-1), p["topk_weights"].reshape(-1)[pairs])
        assert np.array_equal(q["x"], p["x"][pairs // p["k"]])
        for le in (0, 31):
            assert np.array_equal(q["codes"][le], p["codes"][le * 8 + rank])
            assert np.array_equal(q["scales"][le], p["scales"][le * 8 + rank])
    assert np.all(seen == 1)


def test_ep_share_of_the_down_matmul_holds_the_zipf_head():
    from moe_grouped_gemm_route_amd.synth import make_config, make_ep_share
    p = make_config(3)
    q = make_ep_share(3, gpus=8, rank=0)
    counts = np.bincount(q["topk_ids"].reshape(-1), minlength=32)
    full = np.bincount(p["topk_ids"].reshape(-1), minlength=256)
    assert counts[0] == full[0] == full.max()          # expert 0, the head, on rank 0
    assert not q["gather"] and q["x"].shape == (q["T"], p["K"])
