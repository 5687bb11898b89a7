"""Number formats of the routed-expert weights, decoded exactly in float64.

Test infrastructure (see the package docstring): only tests, the smoke check
and the bench's CPU-baseline leg use this module.

Sources
-------
* "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that v6e can't
  hold": an e2m1 weight has a sign bit, a 2-bit exponent field e and a 1-bit
  mantissa m; its eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4 and 6, indexed
  by 2e + m.  A power-of-two scale covers each block of 32 weights and is
  applied to the decoded tile before the matmul.
* Same page, section "Grouped matmul performance vs bf16": the NVFP4 variant
  scales every 16 weights with an E4M3 byte.
* "DeepSeek-V4-Flash-0731-NVFP4", section "The lossless weight cast": the
  MXFP4 E8M0 scales map exactly onto NVFP4's two levels, a per-tensor scale of
  2^(k_max - 8) times a per-16 E4M3 block scale, with k_max shared by the
  fused gate/up pair of an expert.  Every nibble is unchanged.

Readings where the pages are silent:
* Two codes per byte, the even K index in the low nibble; codes are stored
  [.., N, K/2] with K contiguous (the checkpoint's [out, in] orientation).
* E8M0 is the OCP MX scale byte: 2^(b - 127), 0xFF is NaN.
* E4M3 is OCP E4M3FN: bias 7, no infinities, S.1111.111 is NaN.
* The garbled block-scale exponent on the model card is read as
  k_j - (k_max - 8), which makes tensor scale x block scale = 2^(k_j).
"""

import numpy as np

# The eight e2m1 magnitudes, indexed by the 3-bit field 2e + m.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def unpack_nibbles(codes):
    """[.., K/2] uint8 -> [.., K] uint8 nibbles; even K index = low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def e2m1_decode(nibbles):
    """Value of each 4-bit e2m1 code: bit 3 is the sign, bits 0-2 index the
    magnitude table.  Code 0x8 decodes to -0.0."""
    nib = np.asarray(nibbles, dtype=np.uint8) & 0x0F
    mag = E2M1_MAGNITUDES[nib & 0x7]
    return np.where(nib & 0x8, -mag, mag)


def e8m0_decode(b):
    """OCP E8M0 scale byte -> 2^(b - 127) in float64; 0xFF -> NaN."""
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def e4m3_decode(b):
    """OCP E4M3FN byte -> float64.

    Exponent field E (4 bits, bias 7), mantissa field M (3 bits):
    E == 0 is subnormal, (M / 8) * 2^-6; otherwise (1 + M / 8) * 2^(E - 7).
    The two codes with E == 15 and M == 7 are NaN; there is no infinity."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    ex = (b >> 3) & 0xF
    man = b & 0x7
    sub = (man / 8.0) * 2.0 ** -6
    nrm = (1.0 + man / 8.0) * np.ldexp(1.0, ex - 7)
    v = sign * np.where(ex == 0, sub, nrm)
    return np.where((ex == 15) & (man == 7), np.nan, v)


def e4m3_encode_pow2(p):
    """E4M3FN byte holding exactly 2^p, for integer p in [-9, 8].

    p >= -6 is a normal number (exponent field p + 7, mantissa 0); p in
    [-9, -7] is a subnormal with mantissa field 2^(p + 9).  Outside [-9, 8]
    no E4M3 byte holds 2^p and ValueError is raised."""
    p = np.asarray(p, dtype=np.int64)
    if p.size and (p.min() < -9 or p.max() > 8):
        raise ValueError("power of two outside the E4M3 range 2^-9 .. 2^8")
    normal = (p + 7) << 3
    subnormal = np.left_shift(1, np.clip(p + 9, 0, 2))
    return np.where(p >= -6, normal, subnormal).astype(np.uint8)


def decode_mxfp4(codes, scales):
    """Dense weights W[.., n, k] = e2m1(code) * 2^(E8M0 - 127), float64.

    codes [.., N, K/2] uint8, scales [.., N, K/32] uint8 (one per 32 along K).
    """
    v = e2m1_decode(unpack_nibbles(codes))
    s = np.repeat(e8m0_decode(scales), 32, axis=-1)
    return v * s


def decode_nvfp4(codes, block_scales, tensor_scale):
    """Dense weights W[e, n, k] = e2m1(code) * E4M3(block) * tensor_scale[e].

    codes [E, N, K/2] uint8, block_scales [E, N, K/16] E4M3 bytes,
    tensor_scale [E] float32 (one per expert)."""
    v = e2m1_decode(unpack_nibbles(codes))
    s = np.repeat(e4m3_decode(block_scales), 16, axis=-1)
    ts = np.asarray(tensor_scale, dtype=np.float64).reshape((-1,) + (1,) * (v.ndim - 1))
    return v * s * ts


def mxfp4_to_nvfp4(scales):
    """The lossless MXFP4 -> NVFP4 scale cast (model card, "The lossless
    weight cast").

    scales: [E, N, K/32] E8M0 bytes of one expert tensor (for the fused
    gate/up weight the whole tensor shares one k_max per expert).
    Returns (block_scales [E, N, K/16] E4M3 bytes, tensor_scale [E] float32).

    k_j is the unbiased exponent of block j and k_max its maximum over the
    expert; the tensor scale is 2^(k_max - 8) and both 16-halves of block j
    get the E4M3 byte of 2^(k_j - k_max + 8).  Raises ValueError when a block
    cannot be held exactly (k_j < k_max - 17) or a scale byte is NaN."""
    s = np.asarray(scales, dtype=np.int64)
    if np.any(s == 255):
        raise ValueError("NaN E8M0 scale cannot be cast")
    k = s - 127
    kmax = k.reshape(k.shape[0], -1).max(axis=1)
    rel = k - kmax.reshape((-1,) + (1,) * (k.ndim - 1)) + 8
    bs = e4m3_encode_pow2(rel)
    bs = np.repeat(bs, 2, axis=-1)
    ts = np.ldexp(1.0, kmax - 8).astype(np.float32)
    return bs, ts
