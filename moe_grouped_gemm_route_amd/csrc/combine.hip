// moe_combine: top-k weighted unpermute back to token order.
//
// The band layout ("Running DeepSeek V4 Flash on TPU v6", section "1. Four
// bits that v6e can't hold") puts pair p = t*k + j at band row pair_row[p];
// the token's output sums its k rows weighted by the router, in slot order
// j = 0..k-1 with f32 fused multiply-adds, without atomics, as the
// deterministic expert reduction of "DeepSeek-V4-Flash" (PocketLLM docs,
// section "Correctness and precision") requires.
//
// HBM-bound: each thread produces 4 consecutive columns of one token with
// 16-byte (f32) or 8-byte (bf16) loads per slot.  The band rows and router
// weights of up to CB slots are loaded first and then all of their row
// loads are issued together, so a thread keeps CB row loads in flight
// instead of one; the FMAs still run in slot order.
#include "common.h"
#include "launch.h"

namespace moe {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <bool YBF16, bool OBF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ pair_row,
                                                      int32_t T, int32_t k, int32_t N,
                                                      void* __restrict__ out) {
  const int64_t quads = (int64_t)N >> 2;
  const int64_t total = (int64_t)T * quads;
  // one quad per thread; a grid capped below the dispatch limit strides on
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / quads;
    const int64_t c = (i - t * quads) << 2;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    constexpr int CB = 8;   // slots whose row loads are in flight together
    for (int j0 = 0; j0 < k; j0 += CB) {
      int32_t row[CB];
      float wj[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int j = j0 + u;
        row[u] = j < k ? pair_row[t * k + j] : -1;
        wj[u] = j < k ? w[t * k + j] : 0.f;
      }
      float v[CB][4];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0.f;
        if (row[u] >= 0) {
          if (YBF16) {
            const uint2 q =
                *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(y) + (int64_t)row[u] * N + c);
            v[u][0] = bf16_to_f32(q.x & 0xFFFF); v[u][1] = bf16_to_f32(q.x >> 16);
            v[u][2] = bf16_to_f32(q.y & 0xFFFF); v[u][3] = bf16_to_f32(q.y >> 16);
          } else {
            const float4 q = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + (int64_t)row[u] * N + c);
            v[u][0] = q.x; v[u][1] = q.y; v[u][2] = q.z; v[u][3] = q.w;
          }
        }
      }
      // slot order; a dropped pair (row < 0) contributes nothing
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (row[u] >= 0) {
          a0 = fmaf(wj[u], v[u][0], a0);
          a1 = fmaf(wj[u], v[u][1], a1);
          a2 = fmaf(wj[u], v[u][2], a2);
          a3 = fmaf(wj[u], v[u][3], a3);
        }
      }
    }
    if (OBF16) {
      uint2 q;
      q.x = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
      q.y = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + t * N + c) = q;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + t * N + c) = make_float4(a0, a1, a2, a3);
    }
  }
}

hipError_t launch_combine(const void* y, int y_bf16, const float* w, const int32_t* pair_row,
                          int32_t T, int32_t k, int32_t N, void* out, int out_bf16,
                          hipStream_t stream) {
  const int64_t threads = (int64_t)T * (N / 4);
  // 2^22 workgroups of 256 (2^30 work-items) keep the dispatch within its
  // 32-bit work-item count; larger problems stride
  const int64_t groups = (threads + 255) / 256;
  const unsigned grid = (unsigned)(groups < (int64_t(1) << 22) ? groups : (int64_t(1) << 22));
  if (y_bf16) {
    if (out_bf16) hipLaunchKernelGGL((combine_kernel<true, true>), dim3(grid), dim3(256), 0, stream, y, w, pair_row, T, k, N, out);
    else hipLaunchKernelGGL((combine_kernel<true, false>), dim3(grid), dim3(256), 0, stream, y, w, pair_row, T, k, N, out);
  } else {
    if (out_bf16) hipLaunchKernelGGL((combine_kernel<false, true>), dim3(grid), dim3(256), 0, stream, y, w, pair_row, T, k, N, out);
    else hipLaunchKernelGGL((combine_kernel<false, false>), dim3(grid), dim3(256), 0, stream, y, w, pair_row, T, k, N, out);
  }
  return hipGetLastError();
}

}  // namespace moe
