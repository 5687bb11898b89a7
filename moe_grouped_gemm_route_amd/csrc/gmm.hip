// moe_gmm: routed-expert grouped matmul, W4A16 on bf16 MFMA (gfx950).
//
// "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that v6e can't
// hold": the grid walks (expert, M-tile) x N-tile pairs over the expert
// bands, the inner loop walks K, each 4-bit weight tile is decoded to bf16 as
// soon as it is on chip, multiplied by its block scale, and accumulated in an
// f32 tile that never leaves the chip; ragged and empty bands are handled.
// Section "Grouped matmul performance vs bf16": the NVFP4 variant reads
// per-16 E4M3 block scales (and a per-expert tensor scale, applied here in
// the epilogue).
//
// MFMA mapping.  v_mfma_f32_16x16x32_bf16 multiplies a 16x32 A fragment by a
// 32x16 B fragment; lane l supplies row (l & 15) of A and column (l & 15) of
// B for eight K slots picked by l >> 4, and both operands use the same slots,
// so any fixed assignment of K indices to (lane group, slot) gives the same
// dot products.  We assign lane group g, step s, slot i to
//     k = chunk*128 + g*32 + s*8 + i,
// so over the four steps of a 128-deep chunk one lane consumes one whole
// 32-element scale block of its column: one 16-byte load of codes and one
// scale per lane per chunk, and 64 contiguous activation bytes per row.
//
// Both kernels below issue, for every output element, the same MFMAs in the
// same order (chunks ascending, steps 0..3), so they return identical bits.
#include "common.h"
#include "launch.h"

namespace moe {

struct Tile {
  int e;      // expert, or -1 past the last tile
  int m0;     // first band row of the tile
  int rows;   // valid rows in the tile (1..BM)
};

// Per-wave view of the tile list "for each expert e, ceil(count_e / BM)
// tiles": lane l covers experts [l*per, l*per + per) and holds the number of
// tiles before them (excl) and up to their end (incl).  total is uniform.
struct TileScan {
  int per, excl, incl, total;
};

__device__ __forceinline__ TileScan scan_tiles(const int32_t* __restrict__ goff, int E, int BM) {
  const int lane = threadIdx.x & 63;
  TileScan ts;
  ts.per = (E + 63) >> 6;
  const int e0 = lane * ts.per;
  int mine = 0;
  for (int i = 0; i < ts.per; ++i) {
    const int e = e0 + i;
    if (e < E) mine += (goff[e + 1] - goff[e] + BM - 1) / BM;
  }
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  ts.excl = incl - mine;
  ts.incl = incl;
  ts.total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  return ts;
}

// Tile t (< ts.total) of the list, found by every lane of the wave.
__device__ __forceinline__ Tile locate_tile(const int32_t* __restrict__ goff, int E, int BM,
                                            const TileScan& ts, int t) {
  const int lane = threadIdx.x & 63;
  const uint64_t hit = __ballot(ts.excl <= t && t < ts.incl);
  const int src = __ffsll((unsigned long long)hit) - 1;
  int fe = -1, fm0 = 0, frows = 0;
  if (lane == src) {
    int acc = ts.excl;
    for (int i = 0; i < ts.per; ++i) {
      const int e = lane * ts.per + i;
      if (e >= E) break;
      const int c = goff[e + 1] - goff[e];
      const int nt = (c + BM - 1) / BM;
      if (t < acc + nt) {
        const int j = t - acc;
        fe = e;
        fm0 = goff[e] + j * BM;
        frows = c - j * BM < BM ? c - j * BM : BM;
        break;
      }
      acc += nt;
    }
  }
  Tile out;
  out.e = __builtin_amdgcn_readfirstlane(__shfl(fe, src, 64));
  out.m0 = __builtin_amdgcn_readfirstlane(__shfl(fm0, src, 64));
  out.rows = __builtin_amdgcn_readfirstlane(__shfl(frows, src, 64));
  return out;
}

// Work item of this workgroup among G = tiles * NB real items, or -1.  With
// xcd_order, consecutive workgroup ids (which the dispatcher deals round-robin
// to the 8 XCDs) are remapped so that each XCD walks one contiguous run of
// items: the N tiles of one M tile then share that XCD's L2.
__device__ __forceinline__ int work_item(int G, bool xcd_order) {
  const int bx = blockIdx.x;
  if (bx >= G) return -1;
  if (!xcd_order) return bx;
  const int x = bx & 7, idx = bx >> 3;
  const int q = G >> 3, rem = G & 7;
  return x * q + (x < rem ? x : rem) + idx;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Block scales of one lane for chunk kc.  MXFP4: one E8M0 byte for the whole
// block; NVFP4: E4M3 bytes of the low (steps 0, 1) and high (2, 3) halves.
template <int FMT>
__device__ __forceinline__ void chunk_scales(uint32_t word, int kc, float& lo, float& hi) {
  if (FMT == 0) {
    lo = hi = e8m0_to_f32((word >> (8 * (kc & 3))) & 0xFFu);
  } else {
    const uint32_t pair = (kc & 1) ? (word >> 16) : word;
    lo = e4m3_to_f32<0>(pair);
    hi = e4m3_to_f32<1>(pair);
  }
}

// NVFP4 chunks whose E4M3 scales are all powers of two (for instance every
// chunk made by the lossless MXFP4 cast) take the one-instruction decode; a
// wave with any other scale in the chunk takes the general exact decode.
// Both give the same bits.
template <int FMT, int NS>
__device__ __forceinline__ bool general_scales(const float (&lo)[NS], const float (&hi)[NS]) {
  if (FMT == 0) return false;
  bool all = true;
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) all = all && is_pow2_scale(lo[ns]) && is_pow2_scale(hi[ns]);
  return __ballot(!all) != 0;
}

template <int FMT>
__device__ __forceinline__ u32x4_t decode_step(uint32_t codes8, float scale, bool general) {
  if (FMT == 1 && general) return decode8_any_scale(codes8, scale);
  return decode8(codes8, scale);
}

template <int FMT>
__device__ __forceinline__ bool new_scale_record(int kc) {
  return FMT == 0 ? (kc & 3) == 0 : (kc & 1) == 0;
}

template <int FMT>
__device__ __forceinline__ int scale_record(int kc) {
  return FMT == 0 ? (kc >> 2) : (kc >> 1);
}

// Stores the f32 accumulator of one 16x16 MFMA tile: lane l holds column
// (l & 15), rows 4*(l >> 4) .. +3.
template <bool OBF16>
__device__ __forceinline__ void store_tile(void* y, int64_t N, int row0, int rows_valid, int col,
                                           f32x4_t acc, float post) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 4 * g + i;
    if (rl < rows_valid) {
      const float v = acc[i] * post;
      const int64_t off = (int64_t)(row0 + rl) * N + col;
      if (OBF16) reinterpret_cast<uint16_t*>(y)[off] = f32_to_bf16_rne(v);
      else reinterpret_cast<float*>(y)[off] = v;
    }
  }
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

constexpr int BUF_NT = 2;                  // buffer-load cache policy: non-temporal
constexpr uint32_t BUF_OOB = 0x7FFF0000u;  // a lane offset that reads zeros

// ---------------------------------------------------------------------------
// Weight-streaming kernel, for bands of a few rows (decode).  Each wave owns
// NS 16-column subtiles and up to MS 16-row subtiles of one tile (tiles are
// MS * 16 rows), walks the whole K, and has no LDS and no barrier.  Every
// code word loaded feeds one MFMA per row subtile, so a band of up to
// MS * 16 rows streams its expert's codes once per column group.
//
// Pipelining.  A wave's vector loads complete in issue order, so waiting for
// one load also waits for every load issued before it.  The activations of a
// step are therefore loaded together with its codes, D steps ahead, into a
// ring of D register slots: step kc reads slot kc % D, then refills it with
// step kc + D.  Waiting for step kc's data then never waits for a later
// step's, and D steps of codes stay in flight.  Codes, scale words and
// activations go through buffer loads (base in scalar registers, 32-bit
// lane offsets); activation rows past the band read zeros from outside the
// buffer.
// ---------------------------------------------------------------------------
template <int NS, int D, int MSUB, int FMT, bool OBF16>
__device__ __forceinline__ void stream_walk(const uint8_t* __restrict__ packed, const Layout& L,
                                            const Tile& tile, int n0, __amdgpu_buffer_rsrc_t xr,
                                            const uint32_t (&a_voff)[2], __amdgpu_buffer_rsrc_t cr,
                                            __amdgpu_buffer_rsrc_t sr, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int KC = (int)L.KC;
  const int groups = (int)L.groups;
  const uint32_t c_voff = lane * 16;
  const uint32_t s_voff = lane * 4;

  u32x4_t cring[D][NS];
  uint32_t sring[D][NS];
  u32x4_t aring[D][MSUB][4];
  auto load_step = [&](int slot, int kc) {
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        aring[slot][ms][q] = __builtin_amdgcn_raw_buffer_load_b128(xr, a_voff[ms], kc * 256 + q * 16, 0);
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      cring[slot][ns] = __builtin_amdgcn_raw_buffer_load_b128(cr, c_voff, (ns * KC + kc) << 10, BUF_NT);
      const int rec = FMT == 0 ? (kc >> 2) : (kc >> 1);
      sring[slot][ns] = __builtin_amdgcn_raw_buffer_load_b32(sr, s_voff, (ns * groups + rec) * 256, 0);
    }
  };

  f32x4_t acc[MSUB][NS];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[ms][ns] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < KC) load_step(d, d);

  for (int k0 = 0; k0 < KC; k0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kc = k0 + d;
      if (kc < KC) {
        u32x4_t c[NS], a[MSUB][4];
        uint32_t w[NS];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          c[ns] = cring[d][ns];
          w[ns] = sring[d][ns];
        }
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
          for (int q = 0; q < 4; ++q) a[ms][q] = aring[d][ms][q];
        if (kc + D < KC) load_step(d, kc + D);
        float lo[NS], hi[NS];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) chunk_scales<FMT>(w[ns], kc, lo[ns], hi[ns]);
        const bool general = general_scales<FMT, NS>(lo, hi);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
            const u32x4_t b = decode_step<FMT>(c[ns][s], s < 2 ? lo[ns] : hi[ns], general);
#pragma unroll
            for (int ms = 0; ms < MSUB; ++ms)
              acc[ms][ns] = mfma(as_bf16x8(a[ms][s]), as_bf16x8(b), acc[ms][ns]);
          }
        }
      }
    }
  }

  const float post = FMT == 1 ? reinterpret_cast<const float*>(packed + L.tscale_off)[tile.e] : 1.0f;
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
      store_tile<OBF16>(y, L.N, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + ns * 16 + r, acc[ms][ns], post);
}

template <int NS, int D, int MS, int FMT, bool OBF16>
__global__ __launch_bounds__(256, 3) void gmm_stream_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                         const uint16_t* __restrict__ x,
                                                         uint32_t x_bytes,
                                                         const int32_t* __restrict__ row_index,
                                                         const int32_t* __restrict__ goff, int E,
                                                         void* __restrict__ y, int NB) {
  constexpr int BM = 16 * MS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Tiles are dealt round-robin to the 8 XCDs (the dispatcher deals
  // consecutive workgroup ids round-robin), and each XCD walks all NB column
  // groups of its tile before the next one: one expert's codes stream
  // through one XCD in order, while the tiles of a popular expert spread
  // over all XCDs and keep their work balanced.
  const TileScan ts = scan_tiles(goff, E, BM);
  const int bx = blockIdx.x;
  const int xcd = bx & 7, kth = bx >> 3;
  const int t = xcd + 8 * (kth / NB);
  const int nb = kth - (kth / NB) * NB;
  if (t >= ts.total) return;
  const Tile tile = locate_tile(goff, E, BM, ts, t);
  const int n0 = (nb * 4 + wave) * NS * 16;
  if (n0 >= L.N) return;
  const int K = (int)L.K;
  const int r = lane & 15;
  const int g = lane >> 4;

  const int64_t et = (int64_t)tile.e * L.NT + (n0 >> 4);
  const __amdgpu_buffer_rsrc_t cr = buffer_rsrc(packed + ((et * L.KC) << 10), (uint32_t)(NS * L.KC) << 10);
  const __amdgpu_buffer_rsrc_t sr =
      buffer_rsrc(packed + L.scales_off + et * L.groups * 256, (uint32_t)(NS * L.groups) * 256);
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, x_bytes);
  uint32_t a_voff[2] = {BUF_OOB, BUF_OOB};
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int rl = ms * 16 + r;
    if (rl < tile.rows) {
      const int row = tile.m0 + rl;
      const int64_t src = row_index ? row_index[row] : row;
      a_voff[ms] = (uint32_t)(src * K * 2 + g * 64);
    }
  }
  if (MS == 2 && tile.rows > 16)
    stream_walk<NS, (D > 1 ? D - 1 : 1), 2, FMT, OBF16>(packed, L, tile, n0, xr, a_voff, cr, sr, y);
  else
    stream_walk<NS, D, 1, FMT, OBF16>(packed, L, tile, n0, xr, a_voff, cr, sr, y);
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel, for bands of many rows (prefill).  A workgroup of four
// waves owns a 128-row tile and 256 columns; wave w owns columns 64w..64w+63
// (four 16-column subtiles) for all 128 rows, so every decoded weight feeds
// eight MFMAs.  The activation tile of each 128-deep chunk (gathered rows) is
// copied HBM -> LDS by direct-to-LDS 16-byte loads (no staging registers),
// double-buffered.  A staged row is 256 bytes with its 16-byte segments
// XOR-swizzled by (row & 15), so the 16 rows read by one fragment load hit 16
// different bank groups.  Codes stream into registers one chunk ahead.
// 16-row subtiles past the band end are skipped.
// ---------------------------------------------------------------------------
constexpr int TL_MS = 8;                    // 16-row subtiles per tile
constexpr int TL_NS = 4;                    // 16-column subtiles per wave
constexpr int TL_BM = 16 * TL_MS;           // 128
constexpr int TL_BN = 4 * 16 * TL_NS;       // 256
constexpr int TL_ROW_BYTES = 128 * 2;       // one staged row of a chunk
constexpr int TL_BUF_BYTES = TL_BM * TL_ROW_BYTES;
constexpr int TL_LOADS = TL_BUF_BYTES / 1024 / 4;   // 1 KiB wave loads per wave per chunk

// Copies the activation chunk kc into an LDS buffer.  Load j of wave w fills
// LDS bytes [(8w + j) KiB, +1 KiB): rows 4(8w + j) .. +3, lane l landing at
// byte 16 l, i.e. row 4(8w + j) + l/16, physical segment l & 15, which holds
// logical segment (l & 15) ^ (row & 15).
__device__ __forceinline__ void stage_chunk(uint8_t* buf, const uint8_t* const (&ap)[TL_LOADS],
                                            const bool (&av)[TL_LOADS], int kc, int wave) {
#pragma unroll
  for (int j = 0; j < TL_LOADS; ++j) {
    if (av[j])
      __builtin_amdgcn_global_load_lds(ap[j] + kc * 256, buf + (wave * TL_LOADS + j) * 1024, 16, 0, 0);
  }
}

// The K walk of one tiled workgroup for a tile with NSUB valid 16-row
// subtiles (a compile-time count, so the inner loops carry no branches and
// the compiler can batch the LDS fragment reads ahead of the MFMAs).
//
// Per 128-deep chunk kc: issue the activation copy of chunk kc+1 (direct to
// LDS), the codes of chunk kc+1 and the scale words of chunk kc+1, then
// compute chunk kc from registers and LDS filled one iteration earlier, then
// one barrier.  Nothing loaded in an iteration is consumed before that
// iteration's barrier, so no wait inside the compute phase touches the
// loads in flight.
template <int NSUB, int FMT>
__device__ __forceinline__ void tiled_k_walk(uint8_t (*s_a)[TL_BUF_BYTES], const uint8_t* const (&ap)[TL_LOADS],
                                             const bool (&av)[TL_LOADS], const u32x4_t* const (&cp)[TL_NS],
                                             const uint32_t* const (&sp)[TL_NS], bool wave_active, int KC,
                                             int wave, const int (&aoff)[4],
                                             f32x4_t (&acc)[TL_MS][TL_NS]) {
  u32x4_t c[TL_NS];
  uint32_t sw[TL_NS];
  if (wave_active) {
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) {
      c[ns] = __builtin_nontemporal_load(cp[ns]);
      sw[ns] = sp[ns][0];
    }
  }
  __syncthreads();
  for (int kc = 0; kc < KC; ++kc) {
    const int buf = kc & 1;
    const bool more = kc + 1 < KC;
    if (more) stage_chunk(s_a[buf ^ 1], ap, av, kc + 1, wave);
    u32x4_t cn[TL_NS];
    uint32_t swn[TL_NS];
    if (wave_active && more) {
#pragma unroll
      for (int ns = 0; ns < TL_NS; ++ns) {
        cn[ns] = __builtin_nontemporal_load(cp[ns] + (kc + 1) * 64);
        swn[ns] = sp[ns][scale_record<FMT>(kc + 1) * 64];
      }
    }
    if (wave_active) {
      float lo[TL_NS], hi[TL_NS];
#pragma unroll
      for (int ns = 0; ns < TL_NS; ++ns) chunk_scales<FMT>(sw[ns], kc, lo[ns], hi[ns]);
      const bool general = general_scales<FMT, TL_NS>(lo, hi);
      const uint8_t* abase = s_a[buf];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4_t a[NSUB];
#pragma unroll
        for (int ms = 0; ms < NSUB; ++ms)
          a[ms] = *reinterpret_cast<const u32x4_t*>(abase + ms * 16 * TL_ROW_BYTES + aoff[s]);
        u32x4_t b[TL_NS];
#pragma unroll
        for (int ns = 0; ns < TL_NS; ++ns) b[ns] = decode_step<FMT>(c[ns][s], s < 2 ? lo[ns] : hi[ns], general);
#pragma unroll
        for (int ms = 0; ms < NSUB; ++ms)
#pragma unroll
          for (int ns = 0; ns < TL_NS; ++ns) acc[ms][ns] = mfma(as_bf16x8(a[ms]), as_bf16x8(b[ns]), acc[ms][ns]);
      }
    }
    if (wave_active && more) {
#pragma unroll
      for (int ns = 0; ns < TL_NS; ++ns) {
        c[ns] = cn[ns];
        sw[ns] = swn[ns];
      }
    }
    __syncthreads();
  }
}

template <int FMT, bool OBF16>
__global__ __launch_bounds__(256, 2) void gmm_tiled_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                           const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ row_index,
                                                           const int32_t* __restrict__ goff, int E,
                                                           void* __restrict__ y, int NB) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_a[2][TL_BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const TileScan ts = scan_tiles(goff, E, TL_BM);
  const int item = work_item(ts.total * NB, true);
  if (item < 0) return;
  const int t = item / NB;
  const int nb = item - t * NB;
  const Tile tile = locate_tile(goff, E, TL_BM, ts, t);
  const int K = (int)L.K;
  const int KC = (int)L.KC;
  const int n0 = nb * TL_BN + wave * 16 * TL_NS;
  const bool wave_active = n0 < L.N;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int nsub = (tile.rows + 15) >> 4;

  // Source of each of this lane's staging loads (rows past the band are not
  // loaded: their LDS rows only feed accumulator rows that are never stored).
  const uint8_t* ap[TL_LOADS];
  bool av[TL_LOADS];
#pragma unroll
  for (int j = 0; j < TL_LOADS; ++j) {
    const int rl = 4 * (wave * TL_LOADS + j) + (lane >> 4);
    av[j] = rl < tile.rows;
    const int row = tile.m0 + (av[j] ? rl : 0);
    const int64_t src = row_index ? row_index[row] : row;
    const int logical_seg = (lane & 15) ^ (rl & 15);
    ap[j] = reinterpret_cast<const uint8_t*>(x + src * K) + logical_seg * 16;
  }
  const u32x4_t* cp[TL_NS];
  const uint32_t* sp[TL_NS];
#pragma unroll
  for (int ns = 0; ns < TL_NS; ++ns) {
    const int64_t nt = wave_active ? (n0 >> 4) + ns : 0;
    const int64_t et = (int64_t)tile.e * L.NT + nt;
    cp[ns] = reinterpret_cast<const u32x4_t*>(packed + ((et * L.KC) << 10)) + lane;
    sp[ns] = reinterpret_cast<const uint32_t*>(packed + L.scales_off) + et * L.groups * 64 + lane;
  }
  // fragment read offsets: row ms*16 + r, logical segment g*4 + s
  int aoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoff[s] = r * TL_ROW_BYTES + (((g * 4 + s) ^ r) << 4);

  f32x4_t acc[TL_MS][TL_NS];
#pragma unroll
  for (int ms = 0; ms < TL_MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) acc[ms][ns] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  stage_chunk(s_a[0], ap, av, 0, wave);
  switch (nsub) {
    case 1: tiled_k_walk<1, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
    case 2: tiled_k_walk<2, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
    case 3: tiled_k_walk<3, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
    case 4: tiled_k_walk<4, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
    case 5: tiled_k_walk<5, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
    case 6: tiled_k_walk<6, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
    case 7: tiled_k_walk<7, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
    default: tiled_k_walk<8, FMT>(s_a, ap, av, cp, sp, wave_active, KC, wave, aoff, acc); break;
  }

  if (!wave_active) return;
  const float post = FMT == 1 ? reinterpret_cast<const float*>(packed + L.tscale_off)[tile.e] : 1.0f;
#pragma unroll
  for (int ms = 0; ms < TL_MS; ++ms) {
    if (ms < nsub) {
#pragma unroll
      for (int ns = 0; ns < TL_NS; ++ns)
        store_tile<OBF16>(y, L.N, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + ns * 16 + r,
                          acc[ms][ns], post);
    }
  }
}

// Stream-kernel shape: four 16-column subtiles per wave (64 columns, fewer
// and longer waves amortise the tile lookup and activation loads), a ring two
// chunks deep, and tiles of up to 32 rows: a popular expert's band streams
// its codes once per 32 rows instead of once per 16 (the two-subtile walk
// keeps a one-chunk ring so that both walks fit three workgroups per CU).
template <int FMT, bool OBF16>
static void launch_stream(const uint8_t* packed, const Layout& L, const uint16_t* x, uint32_t x_bytes,
                          const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                          void* y, hipStream_t stream) {
  constexpr int NS = 4, D = 2, MS = 2, BM = 16 * MS;
  const int NB = (int)((L.N + 64 * NS - 1) / (64 * NS));
  const int64_t em = E < M ? E : M;
  const int64_t tiles = ((M + BM - 1) / BM + em + 7) / 8 * 8;   // whole rounds of 8 tiles
  hipLaunchKernelGGL((gmm_stream_kernel<NS, D, MS, FMT, OBF16>), dim3((unsigned)(tiles * NB)),
                     dim3(256), 0, stream, packed, L, x, x_bytes, row_index, goff, E, y, NB);
}

template <int FMT, bool OBF16>
static void launch_gmm_t(const uint8_t* packed, const Layout& L, const uint16_t* x, int32_t x_rows,
                         const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                         void* y, int kernel, hipStream_t stream) {
  const uint32_t x_bytes = (uint32_t)((int64_t)x_rows * L.K * 2);
  if (kernel == 1) {
    launch_stream<FMT, OBF16>(packed, L, x, x_bytes, row_index, goff, E, M, y, stream);
  } else {
    const int64_t em = E < M ? E : M;
    const int NB = (int)((L.N + TL_BN - 1) / TL_BN);
    const int64_t tiles = (M + TL_BM - 1) / TL_BM + em;
    hipLaunchKernelGGL((gmm_tiled_kernel<FMT, OBF16>), dim3((unsigned)(tiles * NB)), dim3(256), 0,
                       stream, packed, L, x, row_index, goff, E, y, NB);
  }
}

hipError_t launch_gmm(const uint8_t* packed, int fmt, int32_t E, int32_t N, int32_t K,
                      const uint16_t* x, int32_t x_rows, const int32_t* row_index,
                      const int32_t* group_offsets,
                      int32_t M, void* y, int y_bf16, int kernel, hipStream_t stream) {
  const Layout L = make_layout(fmt, E, N, K);
  if (fmt == 0) {
    if (y_bf16) launch_gmm_t<0, true>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, kernel, stream);
    else launch_gmm_t<0, false>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, kernel, stream);
  } else {
    if (y_bf16) launch_gmm_t<1, true>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, kernel, stream);
    else launch_gmm_t<1, false>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, kernel, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
