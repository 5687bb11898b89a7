// Load-time weight repack (mxfp4_encode, and moe_bf16_encode for the bf16
// comparison arm), its inverse check (moe_debug_decode) and the lossless
// MXFP4 -> NVFP4 scale cast.
//
// "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that v6e can't
// hold": the weights are re-laid-out once at load and stay 4 bits each.  Here
// the repack moves whole 16-byte code runs (one column x one 32-block) into
// the chunk order of the packed layout (common.h) and regroups scale bytes.
// "DeepSeek-V4-Flash-0731-NVFP4", section "The lossless weight cast": the
// per-expert tensor scale 2^(k_max - 8) and per-16 E4M3 scales
// 2^(k_j - k_max + 8).
#include "common.h"
#include "launch.h"

namespace moe {

// One thread per 16-byte code run, in canonical order (coalesced reads).
__global__ __launch_bounds__(256) void encode_codes_kernel(const u32x4_t* __restrict__ codes,
                                                           Layout L, uint8_t* __restrict__ packed) {
  const int64_t runs = L.E * L.N * L.KB;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < runs;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t kb = i % L.KB;
    const int64_t n = (i / L.KB) % L.N;
    const int64_t e = i / (L.KB * L.N);
    *reinterpret_cast<u32x4_t*>(packed + code_run_offset(L, e, n, kb)) = codes[i];
  }
}

// One thread per packed scale dword (lane l of record (e, nt, q)).  Every
// scale byte is read by exactly one thread, which also counts the bytes
// outside the exact-decode domain: E8M0 bytes other than 2..252 (block
// exponents -125..125; 255 is NaN), E4M3 NaN bytes, and non-finite tensor
// scales.
__global__ __launch_bounds__(256) void encode_scales_kernel(int fmt, const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ tscale, Layout L,
                                                            uint8_t* __restrict__ packed,
                                                            int32_t* __restrict__ err_count) {
  const int64_t words = L.E * L.NT * L.groups * 64;
  uint32_t* out = reinterpret_cast<uint32_t*>(packed + L.scales_off);
  int bad = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = i & 63;
    const int64_t q = (i >> 6) % L.groups;
    const int64_t nt = (i >> 6) / L.groups % L.NT;
    const int64_t e = (i >> 6) / (L.groups * L.NT);
    const int64_t n = nt * 16 + (lane & 15);
    uint32_t word = 0;
    if (fmt == 0) {
      for (int c = 0; c < 4; ++c) {
        const int64_t kc = q * 4 + c;
        if (kc < L.KC) {
          const int64_t kb = kc * 4 + (lane >> 4);
          const uint32_t b = scales[(e * L.N + n) * L.KB + kb];
          bad += (b < 2u || b > 252u) ? 1 : 0;
          word |= b << (8 * c);
        }
      }
    } else {
      for (int c = 0; c < 2; ++c) {
        const int64_t kc = q * 2 + c;
        if (kc < L.KC) {
          const int64_t kb = kc * 4 + (lane >> 4);
          const uint8_t* s = scales + (e * L.N + n) * (L.KB * 2) + kb * 2;
          bad += ((s[0] & 0x7F) == 0x7F ? 1 : 0) + ((s[1] & 0x7F) == 0x7F ? 1 : 0);
          word |= ((uint32_t)s[0] | ((uint32_t)s[1] << 8)) << (16 * c);
        }
      }
    }
    out[i] = word;
  }
  if (fmt == 1) {
    float* ts = reinterpret_cast<float*>(packed + L.tscale_off);
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < L.E;
         e += (int64_t)gridDim.x * blockDim.x) {
      const float t = tscale[e];
      bad += (__float_as_uint(t) & 0x7F800000u) == 0x7F800000u ? 1 : 0;
      ts[e] = t;
    }
  }
  if (err_count && bad) atomicAdd(err_count, bad);
}

// NVFP4: the per-subtile flag word of the layout, from the packed scale
// words just written: one wave per (e, nt), nonzero when some E4M3 scale of
// the subtile is not a positive power of two.  Bytes past the last chunk
// (the zero padding of the last record) are not tested.
__global__ __launch_bounds__(256) void encode_flags_kernel(Layout L, uint8_t* __restrict__ packed) {
  const int lane = threadIdx.x & 63;
  for (int64_t sub = blockIdx.x * 4 + (threadIdx.x >> 6); sub < L.E * L.NT; sub += (int64_t)gridDim.x * 4) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(packed + L.scales_off) + sub * L.groups * 64;
    uint32_t bad = 0;
    for (int64_t q = 0; q < L.groups; ++q) {
      const uint32_t valid = 2 * q + 1 < L.KC ? 0xFFFFFFFFu : 0x0000FFFFu;   // chunk 2q + 1 exists?
      bad |= e4m3x4_not_pow2(w[q * 64 + lane]) & valid;
    }
    const bool any = __ballot(bad != 0) != 0;
    if (lane == 0) reinterpret_cast<uint32_t*>(packed + L.flags_off)[sub] = any ? 1u : 0u;
  }
}

// Clears a small int32 counter with a kernel (kept out of memset nodes so the
// call stays safe to record into a HIP graph).
__global__ void zero_i32_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

void launch_zero_i32(int32_t* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, stream, p, n);
}

hipError_t launch_encode(int fmt, const uint8_t* codes, const uint8_t* scales,
                         const float* tensor_scale, int32_t E, int32_t N, int32_t K,
                         uint8_t* packed, int32_t* err_count, hipStream_t stream) {
  const Layout L = make_layout(fmt, E, N, K);
  if (err_count) launch_zero_i32(err_count, 1, stream);
  const int64_t runs = L.E * L.N * L.KB;
  const int grid_c = (int)((runs + 255) / 256 < 65536 ? (runs + 255) / 256 : 65536);
  hipLaunchKernelGGL(encode_codes_kernel, dim3(grid_c), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(codes), L, packed);
  const int64_t words = L.E * L.NT * L.groups * 64;
  const int grid_s = (int)((words + 255) / 256 < 65536 ? (words + 255) / 256 : 65536);
  hipLaunchKernelGGL(encode_scales_kernel, dim3(grid_s), dim3(256), 0, stream, fmt, scales,
                     tensor_scale, L, packed, err_count);
  if (fmt == 1) {
    const int64_t subs = L.E * L.NT;
    const int grid_f = (int)((subs + 3) / 4 < 65536 ? (subs + 3) / 4 : 65536);
    hipLaunchKernelGGL(encode_flags_kernel, dim3(grid_f), dim3(256), 0, stream, L, packed);
  }
  return hipGetLastError();
}

// bf16 weights [E, N, K] -> packed chunks: one thread per 16-byte run of
// eight consecutive K indices (canonical order, coalesced reads).
__global__ __launch_bounds__(256) void encode_bf16_kernel(const u32x4_t* __restrict__ w, Layout L,
                                                          uint8_t* __restrict__ packed) {
  const int64_t runs = L.E * L.N * (L.K / 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < runs;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k8 = i % (L.K / 8);
    const int64_t n = (i / (L.K / 8)) % L.N;
    const int64_t e = i / ((L.K / 8) * L.N);
    *reinterpret_cast<u32x4_t*>(packed + bf16_run_offset(L, e, n, k8)) = w[i];
  }
}

hipError_t launch_bf16_encode(const uint16_t* w, int32_t E, int32_t N, int32_t K, uint8_t* packed,
                              hipStream_t stream) {
  const Layout L = make_layout(2, E, N, K);
  const int64_t runs = L.E * L.N * (L.K / 8);
  const int grid = (int)((runs + 255) / 256 < 65536 ? (runs + 255) / 256 : 65536);
  hipLaunchKernelGGL(encode_bf16_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(w), L, packed);
  return hipGetLastError();
}

// Dense bf16 [E, N, K] from packed bf16 chunks (the inverse of the above).
__global__ __launch_bounds__(256) void unpack_bf16_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                          u32x4_t* __restrict__ w) {
  const int64_t runs = L.E * L.N * (L.K / 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < runs;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k8 = i % (L.K / 8);
    const int64_t n = (i / (L.K / 8)) % L.N;
    const int64_t e = i / ((L.K / 8) * L.N);
    w[i] = *reinterpret_cast<const u32x4_t*>(packed + bf16_run_offset(L, e, n, k8));
  }
}

// Dense bf16 [E, N, K] from the packed buffer: one thread per code run.
__global__ __launch_bounds__(256) void debug_decode_kernel(const uint8_t* __restrict__ packed, int fmt,
                                                           Layout L, uint16_t* __restrict__ w) {
  const int64_t runs = L.E * L.N * L.KB;
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(packed + L.scales_off);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < runs;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t kb = i % L.KB;
    const int64_t n = (i / L.KB) % L.N;
    const int64_t e = i / (L.KB * L.N);
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(packed + code_run_offset(L, e, n, kb));
    const int64_t nt = n >> 4, kc = kb >> 2;
    const int64_t lane = ((kb & 3) << 4) | (n & 15);
    float s_lo, s_hi;
    if (fmt == 0) {
      const uint32_t word = sw[((e * L.NT + nt) * L.groups + (kc >> 2)) * 64 + lane];
      s_lo = s_hi = e8m0_to_f32((word >> (8 * (kc & 3))) & 0xFF);
    } else {
      const uint32_t word = sw[((e * L.NT + nt) * L.groups + (kc >> 1)) * 64 + lane];
      const uint32_t pair = (word >> (16 * (kc & 1))) & 0xFFFF;
      s_lo = e4m3_to_f32<0>(pair);
      s_hi = e4m3_to_f32<1>(pair);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(w + i * 32);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float s = d < 2 ? s_lo : s_hi;
      dst[d] = is_pow2_scale(s) || fmt == 0 ? decode8(c[d], s) : decode8_any_scale(c[d], s);
    }
  }
}

hipError_t launch_debug_decode(const uint8_t* packed, int fmt, int32_t E, int32_t N, int32_t K,
                               uint16_t* w, hipStream_t stream) {
  const Layout L = make_layout(fmt, E, N, K);
  if (fmt == 2) {
    const int64_t runs = L.E * L.N * (L.K / 8);
    const int grid = (int)((runs + 255) / 256 < 65536 ? (runs + 255) / 256 : 65536);
    hipLaunchKernelGGL(unpack_bf16_kernel, dim3(grid), dim3(256), 0, stream, packed, L,
                       reinterpret_cast<u32x4_t*>(w));
    return hipGetLastError();
  }
  const int64_t runs = L.E * L.N * L.KB;
  const int grid = (int)((runs + 255) / 256 < 65536 ? (runs + 255) / 256 : 65536);
  hipLaunchKernelGGL(debug_decode_kernel, dim3(grid), dim3(256), 0, stream, packed, fmt, L, w);
  return hipGetLastError();
}

// MXFP4 quantization of bf16 activation rows (the W4A4 variant): one thread
// per block of 32 K values.  Scale exponent X = floor(log2(max |v|)) - 2 from
// the bf16 bits of the block maximum (magnitudes of finite bf16 values order
// like their 15-bit patterns); each value goes to the nearest e2m1 value of
// v / 2^X, a tie to the even mantissa bit and magnitudes past 6 to 6, with its
// sign.  v / 2^X is exact in f32 (a power-of-two product) and so is every
// comparison with the rounding thresholds.
__device__ __forceinline__ uint32_t e2m1_nearest_code(float a) {
  // thresholds between neighbouring e2m1 magnitudes; an equal value is a tie
  // and goes to the even code
  return a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
       : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
}

__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const u32x4_t* __restrict__ x, int64_t blocks,
                                                             u32x4_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < blocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    u32x4_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = x[b * 4 + i];
    uint32_t amax = 0;   // largest 15-bit magnitude pattern
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = v[i][j] & 0x7FFFu, hi = (v[i][j] >> 16) & 0x7FFFu;
        amax = amax > lo ? amax : lo;
        amax = amax > hi ? amax : hi;
      }
    int byte = 0;
    if (amax != 0) {
      const int ef = (int)(amax >> 7);
      // floor(log2 amax): the exponent of a normal value; for a subnormal,
      // -133 + the position of the leading mantissa bit
      const int fl = ef != 0 ? ef - 127 : -133 + (31 - __builtin_clz(amax & 0x7Fu));
      const int X = fl - 2;
      byte = X + 127 < 0 ? 0 : (X + 127 > 254 ? 254 : X + 127);
    }
    // 2^-X with X = byte - 127: the f32 with exponent field 254 - byte.  A
    // finite bf16 maximum gives byte <= 252 (its exponent is at most 127),
    // so the field lies in [2, 254] and the value is a normal power of two.
    const float inv = __builtin_bit_cast(float, (uint32_t)(254 - (byte > 252 ? 252 : byte)) << 23);
    u32x4_t out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t bits = (v[i][j] >> (16 * h)) & 0xFFFFu;
          const float a = __builtin_bit_cast(float, (bits & 0x7FFFu) << 16) * inv;
          const uint32_t code = e2m1_nearest_code(a) | ((bits >> 12) & 8u);
          const int k = (i * 4 + j) * 2 + h;          // 0..31 within the block
          out[k >> 3] |= code << (4 * (k & 7));
        }
    codes[b] = out;
    scales[b] = (uint8_t)byte;
  }
}

hipError_t launch_quantize_mxfp4(const uint16_t* x, int32_t R, int32_t K, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  const int64_t blocks = (int64_t)R * (K / 32);
  const int grid = (int)((blocks + 255) / 256 < 65536 ? (blocks + 255) / 256 : 65536);
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(x), blocks, reinterpret_cast<u32x4_t*>(codes), scales);
  return hipGetLastError();
}

// Lossless scale cast: one workgroup per expert.  Pass 1 finds the largest
// block exponent; pass 2 writes both 16-half E4M3 bytes of every block.
__global__ __launch_bounds__(256) void mxfp4_to_nvfp4_kernel(const uint8_t* __restrict__ scales,
                                                             int64_t per_expert,
                                                             uint8_t* __restrict__ bs,
                                                             float* __restrict__ ts,
                                                             int32_t* __restrict__ err_count) {
  __shared__ int s_max;
  __shared__ int s_bad;
  const int64_t e = blockIdx.x;
  const uint8_t* src = scales + e * per_expert;
  if (threadIdx.x == 0) { s_max = 0; s_bad = 0; }
  __syncthreads();
  int mx = 0, bad = 0;
  for (int64_t i = threadIdx.x; i < per_expert; i += blockDim.x) {
    const int b = src[i];
    if (b == 255) ++bad;
    else mx = mx > b ? mx : b;
  }
  atomicMax(&s_max, mx);
  __syncthreads();
  const int bmax = s_max;           // biased k_max
  uint16_t* dst = reinterpret_cast<uint16_t*>(bs + e * per_expert * 2);
  for (int64_t i = threadIdx.x; i < per_expert; i += blockDim.x) {
    const int b = src[i];
    const int p = b - bmax + 8;     // power of two of the block scale
    uint32_t byte;
    if (b == 255 || p < -9) {
      byte = 0;
      if (b != 255) ++bad;
    } else if (p >= -6) {
      byte = (uint32_t)(p + 7) << 3;            // normal: exponent field p + 7
    } else {
      byte = 1u << (p + 9);                     // subnormal: mantissa 2^(p + 9)
    }
    dst[i] = (uint16_t)(byte | (byte << 8));
  }
  if (bad) atomicAdd(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    // 2^(k_max - 8) = 2^(bmax - 135): a normal f32 for bmax >= 9, else the
    // subnormal with mantissa bit bmax + 14 (exact down to bmax = 0)
    ts[e] = __uint_as_float(bmax >= 9 ? (uint32_t)(bmax - 8) << 23 : 1u << (bmax + 14));
    if (err_count && s_bad) atomicAdd(err_count, s_bad);
  }
}

hipError_t launch_mxfp4_to_nvfp4(const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                                 uint8_t* block_scales, float* tensor_scale, int32_t* err_count,
                                 hipStream_t stream) {
  const int64_t per_expert = (int64_t)N * (K / 32);
  if (err_count) launch_zero_i32(err_count, 1, stream);
  hipLaunchKernelGGL(mxfp4_to_nvfp4_kernel, dim3(E), dim3(256), 0, stream, scales, per_expert,
                     block_scales, tensor_scale, err_count);
  return hipGetLastError();
}

}  // namespace moe
