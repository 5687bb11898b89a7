"""Pins for the oracle's number formats (CPU only).

Each check compares the oracle against something other than itself: the code
table typed from the pages, the pages' clip decode formula, the field
definition of e2m1, torch's float8 conversions, and hand-worked cast values.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_e2m1_table():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_codes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, sign, e, m, value, q = line.split()
            rows.append((int(code, 16), int(sign), int(e), int(m), float(value), int(q)))
    return rows


def _clip_decode(q):
    # "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that v6e
    # can't hold": decode of the signed code q by two clips.
    return 2 * q - min(max(q, -6), 6) - 0.5 * min(max(q, -4), 4)


def test_e2m1_all_16_codes_against_table_formula_and_fields():
    table = _load_e2m1_table()
    assert [r[0] for r in table] == list(range(16))
    got = F.e2m1_decode(np.arange(16, dtype=np.uint8))
    for code, sign, e, m, value, q in table:
        assert code == (sign << 3) | (e << 1) | m
        # field definition: e == 0 is subnormal (m / 2), else 2^(e-1) (1 + m/2)
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        by_fields = -mag if sign else mag
        assert got[code] == value == by_fields
        assert math.copysign(1.0, got[code]) == math.copysign(1.0, value)
        # signed re-encoding and the pages' clip formula reproduce the value
        assert q == (-(2 * e + m) if sign else 2 * e + m)
        assert _clip_decode(q) == value
        # the re-encoding never produces the int4 code -8
        assert -7 <= q <= 7


def test_clip_formula_outside_e2m1_is_not_a_code():
    # q = -8 (0b1000 as two's complement) would decode to -8, not an e2m1 value
    assert _clip_decode(-8) == -8.0
    assert 8.0 not in set(np.abs(F.E2M1_MAGNITUDES))


def test_unpack_nibbles_low_nibble_is_even_k():
    b = np.array([[0x21, 0xF0, 0x8C]], dtype=np.uint8)
    assert F.unpack_nibbles(b).tolist() == [[1, 2, 0, 15, 12, 8]]


def test_e8m0_all_bytes_against_ldexp_and_torch():
    b = np.arange(256)
    v = F.e8m0_decode(b)
    ref_torch = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for i in range(255):
        assert v[i] == math.ldexp(1.0, i - 127)
        if i > 0:  # torch flushes 2^-127 (subnormal in float32) on conversion
            assert v[i] == ref_torch[i]
    assert np.isnan(v[255]) and np.isnan(ref_torch[255])


def test_e4m3_all_bytes_against_torch():
    v = F.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(v), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(v[~nan], ref[~nan])


def test_e4m3_powers_of_two_representable():
    p = np.arange(-9, 9)
    b = F.e4m3_encode_pow2(p)
    assert np.array_equal(F.e4m3_decode(b), np.ldexp(1.0, p))
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ref, np.ldexp(1.0, p))
    for bad in (-10, 9):
        with pytest.raises(ValueError):
            F.e4m3_encode_pow2(np.array([bad]))


def test_nvfp4_cast_hand_worked_example():
    lines = {}
    with open(os.path.join(GOLDEN, "nvfp4_cast_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            lines[key] = vals
    sc = np.array([int(v) for v in lines["e8m0"]], dtype=np.uint8).reshape(1, 1, 4)
    bs, ts = F.mxfp4_to_nvfp4(sc)
    assert ts.dtype == np.float32 and ts.tolist() == [float(lines["tensor_scale"][0])]
    assert bs.reshape(-1).tolist() == [int(v, 16) for v in lines["e4m3"]]


def test_nvfp4_cast_is_lossless_on_random_weights():
    rng = np.random.default_rng(123)
    E, N, K = 3, 5, 256
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    # per-expert exponent spreads up to the 17 the cast can hold
    base = np.array([-8, 0, 20])
    scales = (base[:, None, None] + rng.integers(-17, 1, size=(E, N, K // 32)) + 127)
    scales[:, 0, 0] = base + 127      # make each expert's k_max explicit
    scales = scales.astype(np.uint8)
    bs, ts = F.mxfp4_to_nvfp4(scales)
    a = F.decode_mxfp4(codes, scales)
    b = F.decode_nvfp4(codes, bs, ts)
    assert np.array_equal(a, b)
    assert np.array_equal(ts, np.ldexp(1.0, base - 8).astype(np.float32))


def test_nvfp4_cast_rejects_out_of_range_blocks_and_nan():
    sc = np.array([[[127, 127 - 18]]], dtype=np.uint8)
    with pytest.raises(ValueError):
        F.mxfp4_to_nvfp4(sc)
    with pytest.raises(ValueError):
        F.mxfp4_to_nvfp4(np.array([[[255]]], dtype=np.uint8))


def test_nvfp4_cast_experts_with_tiny_kmax():
    # an expert whose largest E8M0 byte is 5 (k_max = -122) and an all-zero
    # expert (k_max = -127): the tensor scales 2^-130 and 2^-135 are float32
    # subnormals with the single mantissa bit 19 and 14, the block scales stay
    # 2^8 at k_max, and the cast stays lossless in float64
    sc = np.array([[[5, 3, 0, 5]], [[0, 0, 0, 0]]], dtype=np.uint8)
    bs, ts = F.mxfp4_to_nvfp4(sc)
    assert ts.view(np.uint32).tolist() == [1 << 19, 1 << 14]
    assert bs[1].reshape(-1).tolist() == [0x78] * 8                 # 2^8 = E4M3 exponent field 15
    assert bs[0].reshape(-1).tolist() == [0x78, 0x78, 0x68, 0x68, 0x50, 0x50, 0x78, 0x78]
    codes = np.arange(64, dtype=np.uint8).reshape(2, 1, 32) * 3
    a = F.decode_mxfp4(codes.repeat(2, axis=2)[:, :, :64], sc)
    b = F.decode_nvfp4(codes.repeat(2, axis=2)[:, :, :64], bs, ts)
    assert np.array_equal(a, b)


def test_decode_mxfp4_scale_blocks_run_along_k():
    codes = np.full((1, 2, 32), 0x22, dtype=np.uint8)       # every weight 1.0
    scales = np.array([[[127, 128], [126, 130]]], dtype=np.uint8)
    w = F.decode_mxfp4(codes, scales)[0]
    assert np.all(w[0, :32] == 1.0) and np.all(w[0, 32:] == 2.0)
    assert np.all(w[1, :32] == 0.5) and np.all(w[1, 32:] == 8.0)
