// Device-side definitions shared by the gfx950 kernels: vector types, the
// packed weight layout, and the exact e2m1 -> bf16 decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// A buffer-load lane offset that lies past every buffer range the kernels
// build: a load given it returns zeros (or, for a direct-to-LDS load, writes
// zeros) without touching memory.  The host rejects sizes that would make a
// range reach it.
constexpr uint32_t kLaneOob = 0x7FFF0000u;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Packed weight layout (written once by mxfp4_encode, streamed by moe_gmm).
//
// The canonical weight is [E, N, K/2] bytes: for column n, the 32 codes of
// scale block kb (K indices kb*32 .. kb*32+31) are 16 contiguous bytes.  The
// packed layout keeps those 16-byte runs whole and only reorders them so that
// one wave's 16-byte-per-lane load is one contiguous 1 KiB:
//
//   chunk (e, nt, kc) = 1 KiB  covers columns nt*16 .. +16 and K indices
//                               kc*128 .. +128 (four scale blocks);
//   lane l of that chunk holds column nt*16 + (l & 15), scale block
//   kc*4 + (l >> 4): exactly one MX block, so one scale per lane per chunk.
//
// Scales follow the codes.  MXFP4: for each (e, nt) and group of four chunks
// a 256-byte record in which lane l's dword holds the E8M0 byte of its block
// for chunks 4q .. 4q+3 (byte i = chunk 4q+i).  NVFP4: 256-byte records per
// pair of chunks; lane l's dword holds, for chunk 2q+c, the E4M3 bytes of the
// low and high 16-halves of its block at bytes 2c and 2c+1.  Missing chunks
// of the last record are zero.  NVFP4 appends E floats of tensor scales,
// then one word per (e, nt): nonzero when some E4M3 scale of that subtile is
// not a positive power of two (the tiled kernel's choice of decode).
// ---------------------------------------------------------------------------
struct Layout {
  int64_t E, N, K;
  int64_t NT, KC, KB;     // 16-column tiles, 128-deep chunks, 32-blocks
  int64_t groups;         // scale records per (e, nt)
  int64_t codes_bytes, scales_off, scales_bytes, tscale_off, flags_off, total_bytes;
};

__host__ __device__ inline Layout make_layout(int fmt, int64_t E, int64_t N, int64_t K) {
  Layout L;
  L.E = E; L.N = N; L.K = K;
  L.NT = N / 16; L.KC = K / 128; L.KB = K / 32;
  if (fmt == 2) {
    // bf16 weights (the comparison arm): 4 KiB chunks, no scales
    L.groups = 0;
    L.codes_bytes = E * N * K * 2;
    L.scales_off = L.tscale_off = L.flags_off = L.total_bytes = L.codes_bytes;
    L.scales_bytes = 0;
    return L;
  }
  const int64_t per = fmt == 0 ? 4 : 2;   // chunks per 256-byte scale record
  L.groups = (L.KC + per - 1) / per;
  L.codes_bytes = E * N * K / 2;
  L.scales_off = L.codes_bytes;
  L.scales_bytes = E * L.NT * L.groups * 256;
  L.tscale_off = L.scales_off + L.scales_bytes;
  L.flags_off = L.tscale_off + (fmt == 0 ? 0 : ((E * 4 + 255) / 256) * 256);
  L.total_bytes = L.flags_off + (fmt == 0 ? 0 : ((E * L.NT * 4 + 255) / 256) * 256);
  return L;
}

// bf16 weights (the comparison arm) use the same chunks and the same K
// assignment, four times as large: chunk (e, nt, kc) = 4 KiB at
// ((e*NT + nt)*KC + kc) * 4 KiB, holding for step s (1 KiB at s * 1 KiB)
// lane l's eight bf16 of column nt*16 + (l & 15), K indices
// kc*128 + (l >> 4)*32 + s*8 .. +7, at byte 16 l.
__host__ __device__ inline int64_t bf16_run_offset(const Layout& L, int64_t e, int64_t n, int64_t k8) {
  const int64_t k = k8 * 8;
  const int64_t nt = n >> 4, kc = k >> 7, g = (k >> 5) & 3, st = (k >> 3) & 3;
  const int64_t lane = (g << 4) | (n & 15);
  return (((e * L.NT + nt) * L.KC + kc) << 12) + (st << 10) + (lane << 4);
}

// Byte offset of the 16-byte code run of (e, column n, scale block kb).
__host__ __device__ inline int64_t code_run_offset(const Layout& L, int64_t e, int64_t n, int64_t kb) {
  const int64_t nt = n >> 4, kc = kb >> 2;
  const int64_t lane = ((kb & 3) << 4) | (n & 15);
  return (((e * L.NT + nt) * L.KC + kc) << 10) + (lane << 4);
}

// ---------------------------------------------------------------------------
// Exact decode.  v_cvt_scalef32_pk_bf16_fp4 turns the two e2m1 codes of one
// byte into two bf16 values times an f32 scale (low nibble -> element 0).
// An e2m1 value has at most two significant bits, so value * 2^k is exact in
// bf16 while it stays normal; value * E4M3 has at most six significant bits
// and is exact as well.
//
// The four converted pairs are only ever moved as whole 32-bit words (bit
// casts of the packed bf16x2 results): splitting them into bf16 elements lets
// this compiler fold the four byte selects into one, which duplicates values.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t decode8(uint32_t codes8, float scale) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes8, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes8, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes8, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes8, scale, 3));
  return r;
}

// The scaled convert applies only the exponent of its f32 scale operand, which
// is exact for every E8M0 scale and for power-of-two E4M3 scales.  A general
// E4M3 scale s (up to four significant bits) goes through f32 instead: codes
// -> f32 (scale 1), times s (exact: at most six significant bits), then the
// upper halves are packed into bf16 pairs (exact: the values fit bf16).
__device__ __forceinline__ u32x4_t decode8_any_scale(uint32_t codes8, float s) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  u32x4_t r;
#define MOE_PAIR(i)                                                                 \
  {                                                                                 \
    const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes8, 1.0f, i);    \
    r[i] = __builtin_amdgcn_perm(__float_as_uint(v[1] * s), __float_as_uint(v[0] * s), \
                                 0x07060302u);                                      \
  }
  MOE_PAIR(0) MOE_PAIR(1) MOE_PAIR(2) MOE_PAIR(3)
#undef MOE_PAIR
  return r;
}

// True for a positive power of two (the scales decode8 handles exactly).
__device__ __forceinline__ bool is_pow2_scale(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x807FFFFFu) == 0 && (u & 0x7F800000u) != 0 && (u & 0x7F800000u) != 0x7F800000u;
}

// Flags (bit 7 of each byte) the E4M3 bytes of w that are not a positive
// power of two: a sign, a zero, a normal with a nonzero mantissa (NaN
// included), or a subnormal whose mantissa has more than one bit.  Byte-wise
// arithmetic: every partial value stays below 0x80 per byte, so no carry or
// borrow crosses a byte.
__host__ __device__ inline uint32_t e4m3x4_not_pow2(uint32_t w) {
  constexpr uint32_t H = 0x80808080u, L7 = 0x7F7F7F7Fu;
  const uint32_t m = w & 0x07070707u, e = w & 0x78787878u;
  const uint32_t mnz = (m + L7) & H, enz = (e + L7) & H;
  const uint32_t mbad = ((((m | H) - 0x01010101u) & m) + L7) & H;   // m & (m - 1) != 0
  return (w & H) | (mnz & enz) | (~enz & H & (~mnz | mbad));
}

// E8M0 byte b (1..254) -> 2^(b - 127) as f32, by placing b in the exponent.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b << 23);
}

// E4M3FN byte (selected byte of a dword) -> f32.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  // NaN stays NaN (quiet) instead of rounding into infinity.
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? (uint16_t)((u >> 16) | 0x40u) : (uint16_t)(r >> 16);
}

}  // namespace moe
