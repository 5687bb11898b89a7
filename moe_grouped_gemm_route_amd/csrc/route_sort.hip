// moe_route_sort: deterministic counting sort of token-expert pairs into
// expert bands ("Running DeepSeek V4 Flash on TPU v6", section "1. Four bits
// that v6e can't hold": tokens sorted by expert, one band of rows per
// expert).
//
// The M pairs are cut into G segments of S consecutive pairs, one workgroup
// of 8 waves each, and every segment into 8 wave sub-segments.  The row of
// pair p, of expert e, in segment g and sub-segment w, is
//     start of band e
//   + pairs of expert e in the segments before g
//   + pairs of expert e in the sub-segments of g before w
//   + pairs of expert e before p inside w,
// so rows are ordered by expert, then by pair index.  Two kernels compute it:
//   count  each workgroup histograms its segment in LDS (integer counts, so
//          the order of the LDS increments cannot change them) and writes
//          cnt[g][e] to the caller's workspace;
//   place  each workgroup reads the whole [G][E] table (G <= 64), giving the
//          expert totals and the counts before its segment; histograms its
//          own sub-segments; turns them into per-wave cursors (a block scan
//          of the totals gives the band starts); then each wave walks its
//          sub-segment 64 pairs at a time in pair order: lanes holding the
//          same expert are found with ballots over the id bits, a pair's row
//          is its cursor plus the number of such lanes below it, and the
//          lowest such lane advances the cursor.
// Up to RS_FUSED_MAX pairs one workgroup does all of it with every id held in
// registers and no workspace.  No atomic decides a position.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int RS_FUSED_MAX = 4096;   // pairs sorted by the one-workgroup kernel
constexpr int RS_WAVES = 8;          // waves per workgroup
constexpr int RS_THREADS = RS_WAVES * 64;
constexpr int RS_SEGMENT_MIN = 1024; // pairs per segment of the two-kernel path
constexpr int RS_MAX_SEGMENTS = 64;
constexpr int RS_BATCH = 8;          // rounds of 64 ids loaded together
constexpr int RS_TABLE_BATCH = 32;   // count-table rows loaded together

RoutePlan route_plan(int64_t M, int32_t E) {
  RoutePlan pl;
  if (M <= RS_FUSED_MAX) {
    // one segment; each wave's share of at most RS_BATCH rounds
    pl.fused = 1;
    pl.S = (int)((((M + RS_WAVES - 1) / RS_WAVES) + 63) / 64 * 64) * RS_WAVES;
    pl.G = 1;
    pl.ws_bytes = 0;
    return pl;
  }
  int64_t s = (M + RS_MAX_SEGMENTS - 1) / RS_MAX_SEGMENTS;
  s = (s + RS_THREADS - 1) / RS_THREADS * RS_THREADS;
  pl.fused = 0;
  pl.S = (int)(s < RS_SEGMENT_MIN ? RS_SEGMENT_MIN : s);
  pl.G = (int)((M + pl.S - 1) / pl.S);
  pl.ws_bytes = (size_t)pl.G * (size_t)E * sizeof(int32_t);
  return pl;
}

// ids of up to RS_BATCH rounds: round r, lane l holds pair p0 + 64 r + l
// (-1 past end).
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ ids, int p0, int end, int (&ev)[RS_BATCH]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < RS_BATCH; ++r) {
    const int p = p0 + r * 64 + lane;
    ev[r] = p < end ? ids[p] : -1;
  }
}

__device__ __forceinline__ void count_ids(const int (&ev)[RS_BATCH], int E, int32_t* cnt) {
#pragma unroll
  for (int r = 0; r < RS_BATCH; ++r)
    if (ev[r] >= 0 && ev[r] < E) atomicAdd(&cnt[ev[r]], 1);
}

// Places the rounds of one batch (pairs [p0, min(end, p0 + 64 RS_BATCH))),
// with the wave's cursors in cur (LDS).
__device__ __forceinline__ void place_ids(const int (&ev)[RS_BATCH], int p0, int end, int k, int E, int id_bits,
                                          int32_t* cur, int32_t* __restrict__ sorted_token,
                                          int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < RS_BATCH; ++r) {
    const int base = p0 + r * 64;
    if (base >= end) break;                 // uniform over the wave
    const int p = base + lane;
    const bool in_range = p < end;
    const int e = ev[r];
    const bool valid = in_range && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid) {
      const int pos = cur[e] + rank;
      sorted_token[pos] = p / k;
      sorted_pair[pos] = p;
      pair_row[p] = pos;
    } else if (in_range) {
      pair_row[p] = -1;
    }
    // every lane has read its cursor before the leaders advance them
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) cur[e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

// Sub-segment of wave w of a segment [begin, end) of S pairs (S a multiple of
// 64 RS_WAVES).
__device__ __forceinline__ void wave_range(int seg_begin, int seg_end, int S, int wave, int& b, int& e) {
  const int S8 = S / RS_WAVES;
  b = min(seg_end, seg_begin + wave * S8);
  e = min(seg_end, b + S8);
}

// Per-wave histograms of the segment's sub-segments into s_cnt[wave][E]
// (zeroed beforehand); ev holds the wave's first batch of ids.
__device__ __forceinline__ void count_subsegment(const int32_t* __restrict__ ids, const int (&ev)[RS_BATCH],
                                                 int w_begin, int w_end, int E, int32_t* cnt) {
  count_ids(ev, E, cnt);
  for (int p0 = w_begin + 64 * RS_BATCH; p0 < w_end; p0 += 64 * RS_BATCH) {
    int ev2[RS_BATCH];
    load_ids(ids, p0, w_end, ev2);
    count_ids(ev2, E, cnt);
  }
}

// Turns the per-wave counts s_cnt[w][e] into cursors: thread t covers
// experts [t per, t per + per); tot and bef are its experts' totals and
// counts before the segment.  Returns the number of valid pairs (the end of
// the last band) to every thread; workgroup 0 writes group_offsets and the
// error count.
template <int PER>
__device__ __forceinline__ int scan_cursors(int32_t* s_cnt, int32_t* s_wsum, const int (&tot)[PER],
                                            const int (&bef)[PER], int E, int M, bool write_offsets,
                                            int32_t* __restrict__ group_offsets, int32_t* __restrict__ err_count) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int e0 = tid * PER;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += tot[i];
  int incl = mine;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < RS_WAVES; ++w) {
    if (w < wave) base += s_wsum[w];
    total += s_wsum[w];
  }
  int run = base + incl - mine;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = e0 + i;
    if (e < E) {
      if (write_offsets) group_offsets[e] = run;
      int c = run + bef[i];
#pragma unroll
      for (int w = 0; w < RS_WAVES; ++w) {
        const int n = s_cnt[w * E + e];
        s_cnt[w * E + e] = c;
        c += n;
      }
      run += tot[i];
    }
  }
  if (write_offsets && tid == 0) {
    group_offsets[E] = total;
    if (err_count) *err_count = M - total;
  }
  return total;
}

// Places a wave's sub-segment (first batch in ev) with the cursors in cur.
__device__ __forceinline__ void place_subsegment(const int32_t* __restrict__ ids, const int (&ev)[RS_BATCH],
                                                 int w_begin, int w_end, int k, int E, int id_bits, int32_t* cur,
                                                 int32_t* __restrict__ sorted_token,
                                                 int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row) {
  place_ids(ev, w_begin, w_end, k, E, id_bits, cur, sorted_token, sorted_pair, pair_row);
  for (int p0 = w_begin + 64 * RS_BATCH; p0 < w_end; p0 += 64 * RS_BATCH) {
    int ev2[RS_BATCH];
    load_ids(ids, p0, w_end, ev2);
    place_ids(ev2, p0, w_end, k, E, id_bits, cur, sorted_token, sorted_pair, pair_row);
  }
}

// The whole sort in one workgroup (M <= RS_FUSED_MAX, so every wave's share
// is one batch of ids held in registers).
template <int PER>
__global__ __launch_bounds__(RS_THREADS) void route_sort_fused_kernel(
    const int32_t* __restrict__ ids, int32_t M, int32_t k, int32_t E, int32_t id_bits, int32_t S,
    int32_t* __restrict__ group_offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row, int32_t* __restrict__ err_count) {
  extern __shared__ int32_t s_cnt[];      // [waves][E], later the cursors
  __shared__ int32_t s_wsum[RS_WAVES];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  int w_begin, w_end;
  wave_range(0, M, S, wave, w_begin, w_end);
  int ev[RS_BATCH];
  load_ids(ids, w_begin, w_end, ev);
  for (int i = tid; i < RS_WAVES * E; i += RS_THREADS) s_cnt[i] = 0;
  __syncthreads();
  int32_t* cnt = s_cnt + wave * E;
  count_ids(ev, E, cnt);
  __syncthreads();
  int tot[PER], bef[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    tot[i] = 0;
    bef[i] = 0;
    if (e < E)
#pragma unroll
      for (int w = 0; w < RS_WAVES; ++w) tot[i] += s_cnt[w * E + e];
  }
  const int total = scan_cursors<PER>(s_cnt, s_wsum, tot, bef, E, M, true, group_offsets, err_count);
  __syncthreads();
  place_ids(ev, w_begin, w_end, k, E, id_bits, cnt, sorted_token, sorted_pair, pair_row);
  // rows past the last band belong to dropped pairs
  for (int r = total + tid; r < M; r += RS_THREADS) {
    sorted_token[r] = -1;
    sorted_pair[r] = -1;
  }
}

// Two-kernel path, step 1: cnt[g][e], the pairs of expert e in segment g.
__global__ __launch_bounds__(RS_THREADS) void route_count_kernel(const int32_t* __restrict__ ids, int32_t M,
                                                                 int32_t E, int32_t S,
                                                                 int32_t* __restrict__ cnt_out) {
  extern __shared__ int32_t s_cnt[];      // [waves][E]
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int seg_begin = blockIdx.x * S;
  const int seg_end = min(M, seg_begin + S);
  int w_begin, w_end;
  wave_range(seg_begin, seg_end, S, wave, w_begin, w_end);
  int ev[RS_BATCH];
  load_ids(ids, w_begin, w_end, ev);
  for (int i = tid; i < RS_WAVES * E; i += RS_THREADS) s_cnt[i] = 0;
  __syncthreads();
  count_subsegment(ids, ev, w_begin, w_end, E, s_cnt + wave * E);
  __syncthreads();
  for (int e = tid; e < E; e += RS_THREADS) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < RS_WAVES; ++w) c += s_cnt[w * E + e];
    cnt_out[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Two-kernel path, step 2: cursors from the count table and the segment's own
// per-wave counts, then placement.  Every workgroup writes -1 into the rows
// of its index range past the last band.
template <int PER>
__global__ __launch_bounds__(RS_THREADS) void route_place_kernel(
    const int32_t* __restrict__ ids, int32_t M, int32_t k, int32_t E, int32_t id_bits, int32_t S, int32_t G,
    const int32_t* __restrict__ cnt_tab, int32_t* __restrict__ group_offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ err_count) {
  extern __shared__ int32_t s_cnt[];      // [waves][E], later the cursors
  __shared__ int32_t s_wsum[RS_WAVES];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int g = blockIdx.x;
  const int seg_begin = g * S;
  const int seg_end = min(M, seg_begin + S);
  int w_begin, w_end;
  wave_range(seg_begin, seg_end, S, wave, w_begin, w_end);
  int ev[RS_BATCH];
  load_ids(ids, w_begin, w_end, ev);
  // the first batch of count-table rows is loaded together with the ids and
  // summed only after the segment's own histogram, which hides its latency
  int v[PER][RS_TABLE_BATCH];
  auto load_table = [&](int g0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid * PER + i;
#pragma unroll
      for (int j = 0; j < RS_TABLE_BATCH; ++j)
        v[i][j] = (e < E && g0 + j < G) ? cnt_tab[(int64_t)(g0 + j) * E + e] : 0;
    }
  };
  load_table(0);

  for (int i = tid; i < RS_WAVES * E; i += RS_THREADS) s_cnt[i] = 0;
  __syncthreads();
  int32_t* cnt = s_cnt + wave * E;
  count_subsegment(ids, ev, w_begin, w_end, E, cnt);

  // totals and counts before this segment, for this thread's experts
  int tot[PER], bef[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    tot[i] = 0;
    bef[i] = 0;
  }
  for (int g0 = 0; g0 < G; g0 += RS_TABLE_BATCH) {
    if (g0 > 0) load_table(g0);
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
      for (int j = 0; j < RS_TABLE_BATCH; ++j) {
        tot[i] += v[i][j];
        if (g0 + j < g) bef[i] += v[i][j];
      }
  }
  __syncthreads();
  const int total = scan_cursors<PER>(s_cnt, s_wsum, tot, bef, E, M, g == 0, group_offsets, err_count);
  __syncthreads();
  place_subsegment(ids, ev, w_begin, w_end, k, E, id_bits, cnt, sorted_token, sorted_pair, pair_row);
  for (int r = max(seg_begin, total) + tid; r < seg_end; r += RS_THREADS) {
    sorted_token[r] = -1;
    sorted_pair[r] = -1;
  }
}

template <int PER>
static void launch_route_t(const RoutePlan& pl, const int32_t* ids, int32_t M, int32_t k, int32_t E, int bits,
                           int32_t* group_offsets, int32_t* sorted_token, int32_t* sorted_pair, int32_t* pair_row,
                           int32_t* err_count, int32_t* ws, hipStream_t stream) {
  const size_t lds = (size_t)RS_WAVES * E * sizeof(int32_t);
  if (pl.fused) {
    hipLaunchKernelGGL(route_sort_fused_kernel<PER>, dim3(1), dim3(RS_THREADS), lds, stream, ids, M, k, E, bits,
                       pl.S, group_offsets, sorted_token, sorted_pair, pair_row, err_count);
    return;
  }
  hipLaunchKernelGGL(route_count_kernel, dim3(pl.G), dim3(RS_THREADS), lds, stream, ids, M, E, pl.S, ws);
  hipLaunchKernelGGL(route_place_kernel<PER>, dim3(pl.G), dim3(RS_THREADS), lds, stream, ids, M, k, E, bits, pl.S,
                     pl.G, ws, group_offsets, sorted_token, sorted_pair, pair_row, err_count);
}

// Count table of moe_route_sort_noalloc: one per GPU, for the life of the
// process.  The largest table any accepted size needs is RS_MAX_SEGMENTS x
// 1024 experts of int32 (256 KiB).  In host code `scratch` names a host-side
// stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t RS_SCRATCH_BYTES = (size_t)RS_MAX_SEGMENTS * 1024 * sizeof(int32_t);
static __device__ __align__(256) int32_t scratch[RS_SCRATCH_BYTES / sizeof(int32_t)];

hipError_t route_sort_scratch(int32_t** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // resolved once per device, with that device current
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    addr[dev] = static_cast<int32_t*>(p);
  }
  *ptr = addr[dev];
  *bytes = RS_SCRATCH_BYTES;
  return hipSuccess;
}

hipError_t launch_route_sort(const int32_t* ids, int32_t T, int32_t k, int32_t E,
                             int32_t* group_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                             int32_t* pair_row, int32_t* err_count, int32_t* ws, hipStream_t stream) {
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const int32_t M = T * k;
  const RoutePlan pl = route_plan(M, E);
  // experts per scan thread: E <= 1024 over 512 threads
  if (E <= RS_THREADS)
    launch_route_t<1>(pl, ids, M, k, E, bits, group_offsets, sorted_token, sorted_pair, pair_row, err_count, ws,
                      stream);
  else
    launch_route_t<2>(pl, ids, M, k, E, bits, group_offsets, sorted_token, sorted_pair, pair_row, err_count, ws,
                      stream);
  return hipGetLastError();
}

}  // namespace moe
