"""MXFP4 quantization of activations, for the W4A4 variant (test
infrastructure; see the package docstring).

"DeepSeek-V4-Flash-0731-NVFP4" (model card), the routed-expert row of its
table and the "Performance" discussion, runs the experts W4A4: activations
are quantized to 4-bit floats as well.  That card quantizes with NVFP4 and
calibrated per-tensor scales; gfx950's scaled matrix instructions take
power-of-two (E8M0) block scales, so this path quantizes activations to
MXFP4 instead: per block of 32 consecutive K values of a row,

    X = floor(log2(max |v|)) - 2          (2 = the largest e2m1 exponent)
    code_i = the e2m1 value nearest to v_i / 2^X, a tie going to the code
             with the even mantissa bit; magnitudes past 6 therefore land on
             6 (saturation); the sign is kept, so a negative value that
             rounds to zero becomes -0
    scale = E8M0 byte X + 127, clamped to [0, 254]; an all-zero block gets
            scale byte 0 and zero codes (with their signs).

Inputs are finite bf16 values.  Written out in float64, where v / 2^X and
every distance are exact.
"""

import numpy as np

from .formats import E2M1_MAGNITUDES

_GRID = np.asarray(E2M1_MAGNITUDES, dtype=np.float64)    # magnitude codes 0..7


def nearest_e2m1(a):
    """Magnitude codes (0..7) of the e2m1 values nearest to a >= 0 (array):
    the grid point at the smallest distance, a tie between two neighbours
    going to the even code (even mantissa bit)."""
    a = np.asarray(a, dtype=np.float64)
    d = np.abs(a[..., None] - _GRID)                         # [..., 8]
    best = d == d.min(axis=-1, keepdims=True)
    even = best & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, best)
    return np.argmax(pick, axis=-1).astype(np.uint8)


def quantize_mxfp4_rows(x_bits):
    """bf16 bit patterns [R, K] -> (codes [R, K/2] uint8 with the even K index
    in the low nibble, E8M0 scales [R, K/32] uint8)."""
    from .gmm import bf16_bits_to_f64
    x = bf16_bits_to_f64(x_bits)
    R, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    v = x.reshape(R, K // 32, 32)
    amax = np.abs(v).max(axis=-1)
    _, ex = np.frexp(amax)                                   # amax = m * 2^ex, m in [0.5, 1)
    byte = np.where(amax > 0, np.clip(ex - 1 - 2 + 127, 0, 254), 0)
    X = byte.astype(np.int64) - 127
    mag = nearest_e2m1(np.ldexp(np.abs(v), -X[..., None]))
    codes = (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8).reshape(R, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, byte.astype(np.uint8)


def dequantize_mxfp4_rows(codes, scales):
    """Inverse view: [R, K/2] codes and [R, K/32] E8M0 scales -> float64 [R, K]."""
    from .formats import decode_mxfp4
    return decode_mxfp4(codes, scales)
