"""Pins of the oracle's MXFP4 activation quantization (oracle/quant.py) and the
W4A4 grouped matmul: the e2m1 rounding grid with its ties and saturation
typed from the format's definition, hand-worked blocks, the exact round trip
of any block of e2m1 values times a common power of two, the rounding error
bound, and pure-Python brute force of the W4A4 matmul."""

import math

import numpy as np

import oracle
from oracle.gmm import bf16_bits_to_f64
from moe_grouped_gemm_route_amd.synth import f32_to_bf16_bits, make_problem


def test_nearest_e2m1_grid_ties_and_saturation():
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(oracle.nearest_e2m1(np.array(grid))) == list(range(8))
    # ties go to the even mantissa: 0|0.5 -> 0, 0.5|1 -> 1.0, 1|1.5 -> 1.0,
    # 1.5|2 -> 2.0, 2|3 -> 2.0, 3|4 -> 4.0, 4|6 -> 4.0
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert list(oracle.nearest_e2m1(np.array(ties))) == [0, 2, 2, 4, 4, 6, 6]
    near = [0.2, 0.3, 0.7, 0.8, 1.3, 1.8, 2.6, 3.4, 5.1, 6.5, 7.99, 1e6]
    assert list(oracle.nearest_e2m1(np.array(near))) == [0, 1, 1, 2, 3, 4, 5, 5, 7, 7, 7, 7]


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_quantize_hand_worked_blocks():
    # amax 0.75 = 1.5 * 2^-1: X = -1 - 2 = -3, byte 124; values x 8 sit on the grid
    blk = np.zeros(32)
    blk[:5] = [0.75, -0.375, 0.1875, 0.0625, -0.0]
    codes, scales = oracle.quantize_mxfp4_rows(_bits(blk[None]))
    assert scales[0, 0] == 124
    nib = np.stack([codes[0] & 0xF, codes[0] >> 4], axis=-1).reshape(-1)
    assert list(nib[:5]) == [7, 8 | 5, 3, 1, 8]            # 6, -3, 1.5, 0.5, -0
    # amax 7 (not on the grid): X = 2 - 2 = 0, 7 saturates to 6, 5 ties to 4
    blk = np.zeros(32)
    blk[:3] = [7.0, 5.0, -2.5]
    codes, scales = oracle.quantize_mxfp4_rows(_bits(blk[None]))
    nib = np.stack([codes[0] & 0xF, codes[0] >> 4], axis=-1).reshape(-1)
    assert scales[0, 0] == 127 and list(nib[:3]) == [7, 6, 8 | 4]
    # an all-zero block: scale byte 0, codes 0 (a -0 keeps its sign)
    blk = np.zeros(32)
    blk[1] = -0.0
    codes, scales = oracle.quantize_mxfp4_rows(_bits(blk[None]))
    nib = np.stack([codes[0] & 0xF, codes[0] >> 4], axis=-1).reshape(-1)
    assert scales[0, 0] == 0 and nib[0] == 0 and nib[1] == 8 and not nib[2:].any()


def test_quantize_round_trips_e2m1_blocks():
    # any block of e2m1 values times one power of two is reproduced exactly
    rng = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    rows = []
    for s in range(-20, 12):
        v = grid[rng.integers(0, 8, size=32)] * np.where(rng.random(32) < 0.5, -1, 1)
        v[rng.integers(0, 32)] = grid[rng.integers(1, 8)]      # a non-zero block
        rows.append(np.ldexp(v, s))
    x = np.array(rows)
    bits = _bits(x)
    back = oracle.dequantize_mxfp4_rows(*oracle.quantize_mxfp4_rows(bits))
    assert np.array_equal(back, x)


def test_quantize_error_bound():
    # |dequant - x| <= 2^X (half the widest grid gap, 4..6) below the
    # saturation point and < 2 * 2^X above it (values stay below 8 * 2^X)
    rng = np.random.default_rng(4)
    x_bits = _bits(rng.standard_normal((64, 256)) * np.exp(rng.normal(size=(64, 1)) * 3))
    codes, scales = oracle.quantize_mxfp4_rows(x_bits)
    x = bf16_bits_to_f64(x_bits)
    err = np.abs(oracle.dequantize_mxfp4_rows(codes, scales) - x)
    step = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    assert np.all(err <= 2 * step) and np.mean(err <= step) > 0.99
    # the scale comes from the block maximum: 4 * 2^X <= amax < 8 * 2^X
    amax = np.abs(x).reshape(64, 8, 32).max(axis=-1)
    s = np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert np.all((4 * s <= amax) & (amax < 8 * s))


def _e2m1_val(n):
    s, e, m = n >> 3, (n >> 1) & 3, n & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_gmm_w4a4_brute_force():
    p = make_problem(T=5, k=2, E=3, K=64, N=6, seed=16)
    qc, qs = oracle.quantize_mxfp4_rows(p["x"])
    r = oracle.route_sort(p["topk_ids"], p["E"])
    w = {"fmt": "mxfp4", "codes": p["codes"], "scales": p["scales"]}
    y = oracle.gmm_w4a4(qc, qs, r["sorted_token"], r["group_offsets"], w)
    for t in range(p["T"]):
        for j in range(p["k"]):
            e = int(p["topk_ids"][t, j])
            row = r["pair_row"][t * p["k"] + j]
            for n in range(p["N"]):
                ref = 0.0
                for kk in range(p["K"]):
                    xa = _e2m1_val((int(qc[t, kk // 2]) >> (4 * (kk % 2))) & 0xF) \
                        * math.ldexp(1.0, int(qs[t, kk // 32]) - 127)
                    wb = _e2m1_val((int(p["codes"][e, n, kk // 2]) >> (4 * (kk % 2))) & 0xF) \
                        * math.ldexp(1.0, int(p["scales"][e, n, kk // 32]) - 127)
                    ref += xa * wb
                assert abs(y[row, n] - ref) <= 1e-12 * (1 + abs(ref))


def _e4m3_val(b):
    """E4M3FN byte from its bit fields (finite bytes only): bias 7, subnormal
    at exponent field 0."""
    ex, m = (b >> 3) & 0xF, b & 7
    v = (m / 8.0) * 2.0 ** -6 if ex == 0 else (1 + m / 8.0) * 2.0 ** (ex - 7)
    return -v if b & 0x80 else v


def test_gmm_w4a4_nvfp4_brute_force():
    # NVFP4 weights (arbitrary finite E4M3 block scales, a tensor scale per
    # expert) under the W4A4 oracle, every nibble and scale decoded from its
    # bit fields
    p = make_problem(T=4, k=2, E=3, K=64, N=5, seed=17)
    rng = np.random.default_rng(18)
    bs = rng.integers(0, 0x7F, size=(3, 5, 4)).astype(np.uint8)
    ts = np.array([0.5, 3.0, 2.0 ** -7], dtype=np.float32)
    qc, qs = oracle.quantize_mxfp4_rows(p["x"])
    r = oracle.route_sort(p["topk_ids"], p["E"])
    w = {"fmt": "nvfp4", "codes": p["codes"], "block_scales": bs, "tensor_scale": ts}
    y = oracle.gmm_w4a4(qc, qs, r["sorted_token"], r["group_offsets"], w)
    for t in range(p["T"]):
        for j in range(p["k"]):
            e = int(p["topk_ids"][t, j])
            row = r["pair_row"][t * p["k"] + j]
            for n in range(p["N"]):
                ref = 0.0
                for kk in range(p["K"]):
                    xa = _e2m1_val((int(qc[t, kk // 2]) >> (4 * (kk % 2))) & 0xF) \
                        * math.ldexp(1.0, int(qs[t, kk // 32]) - 127)
                    wb = _e2m1_val((int(p["codes"][e, n, kk // 2]) >> (4 * (kk % 2))) & 0xF) \
                        * _e4m3_val(int(bs[e, n, kk // 16])) * float(ts[e])
                    ref += xa * wb
                assert abs(y[row, n] - ref) <= 1e-12 * (1 + abs(ref))
