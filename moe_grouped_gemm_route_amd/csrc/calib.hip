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

#include <type_traits>

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

// Matrix-unit build-up: the bf16 MFMA rate of the tiled kernel's wave tile
// (row subtiles R of 8 x 4 column subtiles, 16x16x32 MFMAs, 128-deep chunks
// of 4 steps) with chosen parts of the tiled kernel's data movement added
// one at a time, so that the cost of each is measured on its own:
//   PARTS_LDS_A      A fragments read from LDS (one 1 KiB read per wave, row
//                    subtile and step) instead of registers;
//   PARTS_CODES      B decoded (the exact scaled convert) from codes streamed
//                    from HBM, 1 KiB per column subtile and chunk, one chunk
//                    ahead in a two-slot register ring;
//   PARTS_STAGE      an activation chunk copied into LDS per chunk (8 KiB per
//                    wave by direct-to-LDS 16-byte loads), then a wait for all
//                    of the wave's loads and a workgroup barrier;
//   PARTS_BARRIER    a workgroup barrier per chunk and nothing else;
//   PARTS_REG_DECODE B decoded from codes held in registers that change at
//                    every chunk (the decode without the stream);
//   PARTS_CODES_XOR  the code stream, each word only XOR-ed into a register
//                    (the stream without the decode).
// The codes buffer is cut into one region per wave, read as four streams (one
// per column subtile) that wrap inside the region; the staging source wraps
// at x_blocks KiB, so a small x stays in L2 and a large one comes from HBM.
enum : int {
  PARTS_LDS_A = 1,
  PARTS_CODES = 2,
  PARTS_STAGE = 4,
  PARTS_BARRIER = 8,
  PARTS_REG_DECODE = 16,
  PARTS_CODES_XOR = 32,
};

template <int PARTS, int R>
__global__ __launch_bounds__(256, 2) void calib_parts_kernel(const u32x4_t* __restrict__ a,
                                                             const u32x4_t* __restrict__ b,
                                                             const uint8_t* __restrict__ codes, uint32_t region,
                                                             const uint8_t* __restrict__ x, uint32_t x_blocks,
                                                             float scale, int chunks, float* __restrict__ out) {
  constexpr bool LDS_A = PARTS & PARTS_LDS_A, CODES = PARTS & PARTS_CODES, STAGE = PARTS & PARTS_STAGE;
  constexpr bool BAR = PARTS & PARTS_BARRIER, REG_DECODE = PARTS & PARTS_REG_DECODE;
  constexpr bool XOR = PARTS & PARTS_CODES_XOR, STREAM = CODES || XOR;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  __shared__ __attribute__((aligned(1024))) u32x4_t lds[2][2048];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  // LDS starts out holding A fragments, for the LDS reads of runs without staging
  const int64_t nfrag = (int64_t)gridDim.x * 256 * 8;
  for (int i = threadIdx.x; i < 4096; i += 256) (&lds[0][0])[i] = a[((int64_t)blockIdx.x * 4096 + i) % nfrag];
  __syncthreads();
  u32x4_t af[8], bfr[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) af[i] = a[gid * 8 + i];
#pragma unroll
  for (int j = 0; j < 4; ++j) bfr[j] = b[gid * 4 + j];
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes) + gw * region, 0, (int)region, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(x), 0, (int)(x_blocks << 10), 0x00020000);
  const uint32_t stream_bytes = region / 4, stream_chunks = stream_bytes >> 10;
  f32x4_t acc[R][4];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t cw[2][4];
  auto load_codes = [&](u32x4_t (&dst)[4], int c) {
    const uint32_t off = ((uint32_t)c % stream_chunks) << 10;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j] = __builtin_amdgcn_raw_buffer_load_b128(cr, lane * 16, off + j * stream_bytes, 2);
  };
  auto stage = [&](int buf, int c) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(&lds[buf][0]) + wave * 8192;
    const uint64_t blk0 = (uint64_t)gw * 8 + (uint64_t)c * 7919;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(dst + j * 1024), 16, lane * 16,
                                               (uint32_t)((blk0 + j) % x_blocks) << 10, 0, 0);
  };
  if constexpr (STREAM) load_codes(cw[0], 0);
  uint32_t sink = 0;
  auto chunk = [&](auto slotc, int c) {
    constexpr int slot = decltype(slotc)::value;
    if constexpr (STAGE) stage((c + 1) & 1, c + 1);
    if constexpr (STREAM) load_codes(cw[slot ^ 1], c + 1);
    if constexpr (XOR) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sink ^= (cw[slot][j][0] ^ cw[slot][j][1]) ^ (cw[slot][j][2] ^ cw[slot][j][3]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // one step's LDS reads at a time, as in the tiled kernel (left alone,
      // the compiler hoists a whole chunk's reads and runs out of registers)
      asm volatile("" ::: "memory");
      u32x4_t av[R], bv[4];
#pragma unroll
      for (int i = 0; i < R; ++i) av[i] = LDS_A ? lds[c & 1][(s * 8 + i) * 64 + lane] : af[(i + s) & 7];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (CODES) bv[j] = decode8(cw[slot][j][s], scale);
        else if constexpr (REG_DECODE) bv[j] = decode8(af[(j + s) & 7][j] ^ ((uint32_t)c * 0x9E3779B9u), scale);
        else bv[j] = bfr[(j + s) & 3];
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[i]),
                                                              __builtin_bit_cast(bf16x8_t, bv[j]), acc[i][j], 0,
                                                              0, 0);
    }
    if constexpr (STAGE) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else if constexpr (BAR) {
      __builtin_amdgcn_s_barrier();
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if constexpr (STAGE) {
    stage(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
  }
  for (int c = 0; c < chunks; c += 2) {
    chunk(S0{}, c);
    chunk(S1{}, c + 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  float total = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) total += (acc[i][j][0] + acc[i][j][1]) + (acc[i][j][2] + acc[i][j][3]);
  out[gid] = total + (float)(sink & 1);
}

template <int PARTS, int R>
static void launch_parts_t(const u32x4_t* a, const u32x4_t* b, const uint8_t* codes, uint32_t region,
                           const uint8_t* x, uint32_t x_blocks, float scale, int32_t blocks, int32_t chunks,
                           float* out, hipStream_t stream) {
  hipLaunchKernelGGL((calib_parts_kernel<PARTS, R>), dim3((unsigned)blocks), dim3(256), 0, stream, a, b, codes,
                     region, x, x_blocks, scale, chunks, out);
}

template <int R>
static bool launch_parts_r(int32_t parts, const u32x4_t* a, const u32x4_t* b, const uint8_t* codes,
                           uint32_t region, const uint8_t* x, uint32_t x_blocks, float scale, int32_t blocks,
                           int32_t chunks, float* out, hipStream_t stream) {
  switch (parts) {
#define MOE_PARTS_CASE(P)                                                                            \
  case P:                                                                                            \
    launch_parts_t<P, R>(a, b, codes, region, x, x_blocks, scale, blocks, chunks, out, stream); \
    return true;
    MOE_PARTS_CASE(0)
    MOE_PARTS_CASE(PARTS_LDS_A)
    MOE_PARTS_CASE(PARTS_CODES)
    MOE_PARTS_CASE(PARTS_STAGE)
    MOE_PARTS_CASE(PARTS_BARRIER)
    MOE_PARTS_CASE(PARTS_REG_DECODE)
    MOE_PARTS_CASE(PARTS_CODES_XOR)
    MOE_PARTS_CASE(PARTS_LDS_A | PARTS_CODES | PARTS_STAGE)
#undef MOE_PARTS_CASE
    default:
      return false;
  }
}

bool calib_parts_supported(int32_t parts) {
  switch (parts) {
    case 0: case PARTS_LDS_A: case PARTS_CODES: case PARTS_STAGE: case PARTS_BARRIER: case PARTS_REG_DECODE:
    case PARTS_CODES_XOR: case PARTS_LDS_A | PARTS_CODES | PARTS_STAGE:
      return true;
    default:
      return false;
  }
}

hipError_t launch_calib_parts(int32_t parts, int32_t rows16, const uint16_t* a, const uint16_t* b,
                              const void* codes, uint32_t region, const uint16_t* x, uint32_t x_blocks,
                              float scale, int32_t blocks, int32_t chunks, float* out, hipStream_t stream) {
  const u32x4_t* av = reinterpret_cast<const u32x4_t*>(a);
  const u32x4_t* bv = reinterpret_cast<const u32x4_t*>(b);
  const uint8_t* cv = static_cast<const uint8_t*>(codes);
  const uint8_t* xv = reinterpret_cast<const uint8_t*>(x);
  const bool ok = rows16 == 8 ? launch_parts_r<8>(parts, av, bv, cv, region, xv, x_blocks, scale, blocks, chunks, out, stream)
                              : launch_parts_r<6>(parts, av, bv, cv, region, xv, x_blocks, scale, blocks, chunks, out, stream);
  if (!ok) return hipErrorInvalidValue;
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
