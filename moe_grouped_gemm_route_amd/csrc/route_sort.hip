// moe_route_sort: deterministic counting sort of token-expert pairs into
// expert bands ("Running DeepSeek V4 Flash on TPU v6", section "1. Four bits
// that v6e can't hold": tokens sorted by expert, one band of rows per
// expert).
//
// One workgroup of 512 threads (8 wave64s):
//   1. histogram of expert ids in LDS (integer counts: the order of the LDS
//      increments cannot change them);
//   2. exclusive scan of the counts -> band starts (one wave, 16 experts per
//      lane, then a wavefront scan);
//   3. stable scatter, 512 pairs per round in pair order.  Inside a wave the
//      lanes holding the same expert are found with ballots over the id bits;
//      a lane's rank is the number of such lanes below it.  Per-wave counts
//      go to LDS, and the waves' offsets are summed in wave order, so every
//      position comes from counts and scans, not from atomics.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int RS_THREADS = 512;
constexpr int RS_WAVES = RS_THREADS / 64;
constexpr int RS_EMAX = 1024;

__global__ __launch_bounds__(RS_THREADS) void route_sort_kernel(
    const int32_t* __restrict__ ids, int32_t M, int32_t k, int32_t E, int32_t id_bits,
    int32_t* __restrict__ group_offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ err_count) {
  __shared__ int32_t s_base[RS_EMAX];
  __shared__ int32_t s_wave_cnt[RS_WAVES][RS_EMAX];
  __shared__ int32_t s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < E; e += RS_THREADS) {
    s_base[e] = 0;
    for (int w = 0; w < RS_WAVES; ++w) s_wave_cnt[w][e] = 0;
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // 1. histogram
  int bad = 0;
  for (int p = tid; p < M; p += RS_THREADS) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&s_base[e], 1);
    else ++bad;
  }
  if (bad) atomicAdd(&s_bad, bad);
  __syncthreads();

  // 2. exclusive scan over experts (wave 0)
  if (wave == 0) {
    constexpr int PER = RS_EMAX / 64;
    int local[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      local[i] = e < E ? s_base[e] : 0;
      sum += local[i];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      if (e < E) {
        s_base[e] = run;
        group_offsets[e] = run;
      }
      run += local[i];
    }
    if (lane == 63) group_offsets[E] = incl;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // 3. stable scatter, one round of RS_THREADS pairs at a time
  for (int p0 = 0; p0 < M; p0 += RS_THREADS) {
    const int p = p0 + tid;
    const int e = p < M ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    const bool leader = valid && rank == 0;
    if (leader) s_wave_cnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (p < M) {
      if (valid) {
        int pos = s_base[e] + rank;
        for (int w = 0; w < wave; ++w) pos += s_wave_cnt[w][e];
        sorted_token[pos] = p / k;
        sorted_pair[pos] = p;
        pair_row[p] = pos;
      } else {
        pair_row[p] = -1;
      }
    }
    __syncthreads();
    // advance band cursors by this round's counts, clear the per-wave counts
    for (int x = tid; x < E; x += RS_THREADS) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < RS_WAVES; ++w) {
        add += s_wave_cnt[w][x];
        s_wave_cnt[w][x] = 0;
      }
      s_base[x] += add;
    }
    __syncthreads();
  }

  // rows past the last band belong to dropped pairs
  const int valid_rows = M - s_bad;
  for (int r = valid_rows + tid; r < M; r += RS_THREADS) {
    sorted_token[r] = -1;
    sorted_pair[r] = -1;
  }
  if (tid == 0 && err_count) *err_count = s_bad;
}

hipError_t launch_route_sort(const int32_t* ids, int32_t T, int32_t k, int32_t E,
                             int32_t* group_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                             int32_t* pair_row, int32_t* err_count, hipStream_t stream) {
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(RS_THREADS), 0, stream, ids, T * k, k, E,
                     bits, group_offsets, sorted_token, sorted_pair, pair_row, err_count);
  return hipGetLastError();
}

}  // namespace moe
