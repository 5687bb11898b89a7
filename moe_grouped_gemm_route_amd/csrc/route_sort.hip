// moe_route_sort: deterministic counting sort of token-expert pairs into
// expert bands ("Running DeepSeek V4 Flash on TPU v6", section "1. Four bits
// that v6e can't hold": tokens sorted by expert, one band of rows per
// expert).
//
// G workgroups of 8 wave64s; workgroup g owns the contiguous pair segment
// [g*S, (g+1)*S) and wave w of it the sub-segment [g*S + w*S8, ... + S8).
//   1. histograms (integer counts, so the order of the LDS increments cannot
//      change them): over all M pairs, tot[e]; over the pairs before the
//      segment, bef[e]; over each wave's sub-segment, cnt[w][e];
//   2. scan (all threads): band starts off[e] = sum of tot over experts
//      < e, and each wave's cursor cur[w][e] = off[e] + bef[e] + sum over
//      w' < w of cnt[w'][e];
//   3. place: each wave walks its sub-segment 64 pairs at a time in pair
//      order; lanes holding the same expert are found with ballots over the
//      id bits; a pair's row is cur[w][e] + the number of such lanes below
//      it, and the lowest such lane advances cur[w][e].
// Rows are ordered by expert, then by pair index; every position comes from
// counts, scans and lane order.  Workgroup 0 writes group_offsets, the
// error count and the -1 rows past the last band.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int RS_WAVES = 8;
constexpr int RS_THREADS = RS_WAVES * 64;
constexpr int RS_SEGMENT = 2048;     // pairs placed per workgroup (large M)
constexpr int RS_MAX_GROUPS = 64;
constexpr int RS_UNROLL = 8;         // id loads in flight per thread

__global__ __launch_bounds__(RS_THREADS) void route_sort_kernel(
    const int32_t* __restrict__ ids, int32_t M, int32_t k, int32_t E, int32_t id_bits, int32_t S,
    int32_t* __restrict__ group_offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ err_count) {
  extern __shared__ int32_t s_mem[];
  int32_t* s_tot = s_mem;                 // [E]
  int32_t* s_bef = s_mem + E;             // [E]
  int32_t* s_cnt = s_mem + 2 * E;         // [RS_WAVES][E], later the cursors
  __shared__ int32_t s_bad;
  __shared__ int32_t s_wsum[RS_WAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int seg_begin = min(M, (int)blockIdx.x * S);
  const int seg_end = min(M, seg_begin + S);
  const int S8 = (S + RS_WAVES - 1) / RS_WAVES;
  const int w_begin = min(seg_end, seg_begin + wave * S8);
  const int w_end = min(seg_end, w_begin + S8);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  for (int i = tid; i < (2 + RS_WAVES) * E; i += RS_THREADS) s_mem[i] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // 1. histograms (ids are loaded RS_UNROLL at a time, so that one wait
  // covers several loads)
  int bad = 0;
  for (int p0 = 0; p0 < M; p0 += RS_THREADS * RS_UNROLL) {
    int ev[RS_UNROLL];
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u) {
      const int p = p0 + u * RS_THREADS + tid;
      ev[u] = p < M ? ids[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u) {
      const int p = p0 + u * RS_THREADS + tid;
      const int e = ev[u];
      if (p >= M) break;
      if (e >= 0 && e < E) {
        atomicAdd(&s_tot[e], 1);
        if (p < seg_begin) atomicAdd(&s_bef[e], 1);
      } else {
        ++bad;
      }
    }
  }
  int32_t* cnt = s_cnt + wave * E;
  for (int p0 = w_begin; p0 < w_end; p0 += 64 * RS_UNROLL) {
    int ev[RS_UNROLL];
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u) {
      const int p = p0 + u * 64 + lane;
      ev[u] = p < w_end ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < RS_UNROLL; ++u)
      if (ev[u] >= 0 && ev[u] < E) atomicAdd(&cnt[ev[u]], 1);
  }
  for (int d = 32; d > 0; d >>= 1) bad += __shfl_xor(bad, d, 64);
  if (lane == 0 && bad) atomicAdd(&s_bad, bad);
  __syncthreads();

  // 2. scan (all threads): thread t covers experts [t*per, t*per + per);
  // an exclusive block scan of their totals gives the band starts, and each
  // expert's per-wave cursors follow from its before-segment count and the
  // per-wave counts
  {
    const int per = (E + RS_THREADS - 1) / RS_THREADS;
    const int e0 = tid * per;
    int mine = 0;
    for (int i = 0; i < per; ++i)
      if (e0 + i < E) mine += s_tot[e0 + i];
    int incl = mine;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    int run = base + incl - mine;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        if (blockIdx.x == 0) group_offsets[e] = run;
        int n[RS_WAVES];
#pragma unroll
        for (int w = 0; w < RS_WAVES; ++w) n[w] = s_cnt[w * E + e];
        int c = run + s_bef[e];
#pragma unroll
        for (int w = 0; w < RS_WAVES; ++w) {
          s_cnt[w * E + e] = c;
          c += n[w];
        }
        run += s_tot[e];
      }
    }
    if (blockIdx.x == 0 && tid == RS_THREADS - 1) group_offsets[E] = base + incl;
  }
  __syncthreads();

  // 3. place this wave's sub-segment in pair order (the ids of the next
  // round are loaded while this one is placed)
  int e_next = (w_begin + lane < w_end) ? ids[w_begin + lane] : -1;
  for (int p0 = w_begin; p0 < w_end; p0 += 64) {
    const int p = p0 + lane;
    const bool in_seg = p < w_end;
    const int e = e_next;
    e_next = (p + 64 < w_end) ? ids[p + 64] : -1;
    const bool valid = in_seg && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid) {
      const int pos = cnt[e] + rank;
      sorted_token[pos] = p / k;
      sorted_pair[pos] = p;
      pair_row[p] = pos;
    } else if (in_seg) {
      pair_row[p] = -1;
    }
    // every lane has read its cursor before the leaders advance them
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) cnt[e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }

  if (blockIdx.x == 0) {
    // rows past the last band belong to dropped pairs
    const int valid_rows = M - s_bad;
    for (int r = valid_rows + tid; r < M; r += RS_THREADS) {
      sorted_token[r] = -1;
      sorted_pair[r] = -1;
    }
    if (tid == 0 && err_count) *err_count = s_bad;
  }
}

hipError_t launch_route_sort(const int32_t* ids, int32_t T, int32_t k, int32_t E,
                             int32_t* group_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                             int32_t* pair_row, int32_t* err_count, hipStream_t stream) {
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const int32_t M = T * k;
  int groups = (M + RS_SEGMENT - 1) / RS_SEGMENT;
  if (groups > RS_MAX_GROUPS) groups = RS_MAX_GROUPS;
  if (groups < 1) groups = 1;
  const int32_t S = (M + groups - 1) / groups;
  const size_t lds = (size_t)(2 + RS_WAVES) * E * sizeof(int32_t);
  hipLaunchKernelGGL(route_sort_kernel, dim3(groups), dim3(RS_THREADS), lds, stream, ids, M, k, E,
                     bits, S, group_offsets, sorted_token, sorted_pair, pair_row, err_count);
  return hipGetLastError();
}

}  // namespace moe
