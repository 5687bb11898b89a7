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

}  // namespace moe
