// Measurement support.
//
// Matrix-unit calibration: the bf16 MFMA rate this part sustains with no
// memory traffic, the ceiling that the tiled kernel's MFMA-bound fraction is
// read against (the published dense peak assumes the full shader clock on
// every cycle).
//
// Each wave keeps eight A and four B 16-byte fragments of its lanes in
// registers and issues iters rounds of 32 v_mfma_f32_16x16x32_bf16 over a
// 128 x 64 accumulator tile (the tiled kernel's wave tile: 8 row subtiles x
// 4 column subtiles).  Round i pairs row subtile m with A fragment
// (m + i) % 8 and column subtile n with B fragment (n + i) % 4, so every
// instruction's operands differ from the previous one's, as they do when
// the tiled kernel streams real activations and decoded weights.  The
// accumulators are summed into out so nothing is dead code.
#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256, 2) void calib_mfma_kernel(const u32x4_t* __restrict__ a,
                                                            const u32x4_t* __restrict__ b, int iters,
                                                            float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4_t af[8], bfr[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) af[i] = a[gid * 8 + i];
#pragma unroll
  for (int j = 0; j < 4; ++j) bfr[j] = b[gid * 4 + j];
  f32x4_t acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // four rounds per iteration: the rotation (m + s) % 8, (n + s) % 4 has
  // compile-time register indices
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, af[(m + s) & 7]), __builtin_bit_cast(bf16x8_t, bfr[(n + s) & 3]),
              acc[m][n], 0, 0, 0);
  }
  float total = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) total += (acc[m][n][0] + acc[m][n][1]) + (acc[m][n][2] + acc[m][n][3]);
  out[gid] = total;
}

hipError_t launch_calib_mfma(const uint16_t* a, const uint16_t* b, int32_t blocks, int32_t iters, float* out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(a), reinterpret_cast<const u32x4_t*>(b), iters, out);
  return hipGetLastError();
}

// HBM read calibration: the rate at which this part streams a buffer into the
// CUs with the access pattern of the weight-streaming kernel: each wave walks
// its own contiguous region in 1 KiB runs (one 16-byte non-temporal buffer
// load per lane), with HBM_RING runs in flight in a register ring that is
// refilled as each run is consumed.  Lane l of wave w XORs the 32-bit words
// of its 16-byte slots into one value, so no load is dead and the XOR of all
// outputs is the XOR of the buffer's 32-bit words (the bytes past the last
// whole run are read by wave 0).
constexpr int HBM_RING = 8;

__global__ __launch_bounds__(256) void calib_hbm_read_kernel(const uint8_t* __restrict__ src, uint32_t words_lo,
                                                             uint32_t words_hi, uint32_t* __restrict__ out) {
  const uint64_t words = ((uint64_t)words_hi << 32) | words_lo;   // 16-byte words
  const uint64_t runs = words / 64;                                 // whole 1 KiB runs
  const uint64_t waves = (uint64_t)gridDim.x * 4;
  const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint64_t per = (runs + waves - 1) / waves;
  const uint64_t r0 = wave * per < runs ? wave * per : runs;
  const uint64_t r1 = r0 + per < runs ? r0 + per : runs;
  const int n = (int)(r1 - r0);                                     // runs of this wave (< 2^22)
  // the region of one wave is below 4 GiB (the buffer is at most 2^40 bytes
  // over at least 256 waves)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(src) + r0 * 1024, 0, (int)((uint32_t)n << 10), 0x00020000);
  const uint32_t voff = lane * 16;
  uint32_t x = 0;
  u32x4_t ring[HBM_RING];
#pragma unroll
  for (int d = 0; d < HBM_RING; ++d)
    if (d < n) ring[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (uint32_t)d << 10, 2);
  for (int r = 0; r < n; r += HBM_RING) {
#pragma unroll
    for (int d = 0; d < HBM_RING; ++d) {
      if (r + d < n) {
        const u32x4_t v = ring[d];
        if (r + d + HBM_RING < n)
          ring[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (uint32_t)(r + d + HBM_RING) << 10, 2);
        x ^= (v[0] ^ v[1]) ^ (v[2] ^ v[3]);
      }
    }
  }
  if (wave == 0)
    for (uint64_t i = runs * 64 + lane; i < words; i += 64) {
      const u32x4_t v = reinterpret_cast<const u32x4_t*>(src)[i];
      x ^= (v[0] ^ v[1]) ^ (v[2] ^ v[3]);
    }
  out[(uint64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

hipError_t launch_calib_hbm_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out,
                                 hipStream_t stream) {
  const uint64_t words = bytes / 16;
  hipLaunchKernelGGL(calib_hbm_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(src), (uint32_t)words, (uint32_t)(words >> 32), out);
  return hipGetLastError();
}

}  // namespace moe
