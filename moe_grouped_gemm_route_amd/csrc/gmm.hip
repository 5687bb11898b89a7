// moe_gmm: routed-expert grouped matmul, W4A16 on bf16 MFMA (gfx950).
//
// Source: "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that
// v6e can't hold" (the loop nest and the decode placement) and section
// "Grouped matmul performance vs bf16" (the NVFP4 variant).  Here every
// workgroup owns one tile of rows of one expert's band and a range of output
// columns; it walks K in 128-deep chunks, turns each chunk's 4-bit codes
// into exact bf16 weights in registers right after they arrive (E8M0 or E4M3
// block scale folded into the convert), feeds them to the matrix cores with
// f32 accumulators held on chip for the whole walk, and writes only the
// band's real rows at the end.  Experts with no rows produce no work.  NVFP4's
// per-expert tensor scale is one multiply in that final write.
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
// The two W4A16 kernels below (the weight-streaming kernel for thin bands,
// the LDS-tiled one for thick bands) issue, for every output element, the
// same MFMAs in the same order (chunks ascending, steps 0..3), so they return
// identical bits.  The W4A4 kernel at the end of the file multiplies MXFP4
// activations by the same packed weights on the scaled FP4 MFMA.
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace moe {

struct Tile {
  int e;      // expert, or -1 past the last tile
  int m0;     // first band row of the tile
  int rows;   // valid rows in the tile (1..BM)
  int first;  // 1 for the first tile of its expert's band
};

// Per-wave view of the tile list "for each expert e whose band holds between
// lo and hi rows, ceil(count_e / BM) tiles" (every non-empty band by
// default): lane l covers experts [l*per, l*per + per) and holds the number of
// tiles before them (excl) and up to their end (incl); total is uniform.  The
// lane's band offsets go[0 .. per] are loaded in one batch and kept in
// registers, so finding a tile costs one round trip to memory, not one per
// expert (each round trip takes microseconds while the weights stream).
constexpr int TS_PER_MAX = 16;   // experts per lane: E <= 1024 over 64 lanes

struct TileScan {
  int per, excl, incl, total, lo, hi;
  int go[TS_PER_MAX + 1];
};

// Tiles of an expert whose band holds c rows, under the scan's band filter.
__device__ __forceinline__ int band_tiles(int c, int BM, int lo, int hi) {
  return (c >= lo && c <= hi) ? (c + BM - 1) / BM : 0;
}

__device__ __forceinline__ TileScan scan_tiles(const int32_t* __restrict__ goff, int E, int BM, int lo = 1,
                                               int hi = 1 << 30) {
  const int lane = threadIdx.x & 63;
  TileScan ts;
  ts.lo = lo;
  ts.hi = hi;
  ts.per = (E + 63) >> 6;
  const int e0 = lane * ts.per;
#pragma unroll
  for (int i = 0; i <= TS_PER_MAX; ++i) ts.go[i] = (i <= ts.per && e0 + i <= E) ? goff[e0 + i] : 0;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < TS_PER_MAX; ++i)
    if (i < ts.per && e0 + i < E) mine += band_tiles(ts.go[i + 1] - ts.go[i], BM, lo, hi);
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

// Tile t (< ts.total) of the list, found by every lane of the wave from the
// offsets the scan holds in registers.
__device__ __forceinline__ Tile locate_tile(int E, int BM, const TileScan& ts, int t) {
  const int lane = threadIdx.x & 63;
  const uint64_t hit = __ballot(ts.excl <= t && t < ts.incl);
  const int src = __ffsll((unsigned long long)hit) - 1;
  int fe = -1, fm0 = 0, frows = 0, ffirst = 0;
  if (lane == src) {
    const int e0 = lane * ts.per;
    int acc = ts.excl;
#pragma unroll
    for (int i = 0; i < TS_PER_MAX; ++i) {
      if (i < ts.per && e0 + i < E && fe < 0) {
        const int c = ts.go[i + 1] - ts.go[i];
        const int nt = band_tiles(c, BM, ts.lo, ts.hi);
        if (t < acc + nt) {
          const int j = t - acc;
          fe = e0 + i;
          fm0 = ts.go[i] + j * BM;
          frows = c - j * BM < BM ? c - j * BM : BM;
          ffirst = j == 0;
        }
        acc += nt;
      }
    }
  }
  Tile out;
  out.e = __builtin_amdgcn_readfirstlane(__shfl(fe, src, 64));
  out.m0 = __builtin_amdgcn_readfirstlane(__shfl(fm0, src, 64));
  out.rows = __builtin_amdgcn_readfirstlane(__shfl(frows, src, 64));
  out.first = __builtin_amdgcn_readfirstlane(__shfl(ffirst, src, 64));
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

// GEN (NVFP4 only): some block scale of the wave's columns is not a power of
// two (span_scales_pow2 below), so every step takes the general exact decode;
// otherwise the one-instruction decode.  Both give the same bits.
template <int FMT, bool GEN>
__device__ __forceinline__ u32x4_t decode_step(uint32_t codes8, float scale) {
  if (FMT == 1 && GEN) return decode8_any_scale(codes8, scale);
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

// Columns a wave multiplies.  Plain output (ACT 0): NS contiguous 16-column
// subtiles from column n0.  SiLU-gated gate/up output (ACT 1, four
// subtiles): subtiles 0 and 1 are the gate columns n0 .. n0+31, subtiles 2
// and 3 the up columns N/2 + n0 .. +31, and the wave writes columns
// n0 .. n0+31 of the [M, N/2] activation.  col_sub is a subtile's 16-column
// index relative to the wave's first subtile (h16 = N/32).
// Subtile ns of a wave that owns NS 16-column subtiles: with the fused
// activation the first NS / 2 are gate subtiles and the rest the matching up
// subtiles, h16 subtiles further on.
template <int ACT, int NS = 4>
__device__ __forceinline__ int col_sub(int ns, int h16) {
  return (ACT == 1 && ns >= NS / 2) ? ns - NS / 2 + h16 : ns;
}

// NVFP4: true when every block scale (E4M3) in a wave's four 16-column
// subtiles is a positive power of two, the case the one-instruction decode
// handles exactly (for instance every pack made by the lossless MXFP4 cast).
// The encoder stores a flag word per (expert, subtile); each kernel's wave
// reads its four (uniform loads) once, before its K walk, and walks with one
// decode.
template <int ACT>
__device__ __forceinline__ bool span_scales_pow2(const uint8_t* __restrict__ packed, const Layout& L, int64_t et,
                                                 int h16) {
  const uint32_t* flags = reinterpret_cast<const uint32_t*>(packed + L.flags_off) + et;
  uint32_t any = 0;
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) any |= flags[col_sub<ACT>(ns, h16)];
  return any == 0;
}

// The gate/up activation of one 16x16 tile pair: silu(gate) * up, with
// silu(z) = z / (1 + e^-z) in f32 (the NVFP4 tensor scale applies to both
// halves first); the layout and masking follow store_tile.
template <bool OBF16>
__device__ __forceinline__ void store_tile_silu_mul(void* y, int64_t ldy, int row0, int rows_valid,
                                                    int col, f32x4_t gate, f32x4_t up, float post) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 4 * g + i;
    if (rl < rows_valid) {
      const float gv = gate[i] * post;
      const float v = gv / (1.0f + __expf(-gv)) * (up[i] * post);
      const int64_t off = (int64_t)(row0 + rl) * ldy + col;
      if (OBF16) reinterpret_cast<uint16_t*>(y)[off] = f32_to_bf16_rne(v);
      else reinterpret_cast<float*>(y)[off] = v;
    }
  }
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Byte offset of chunk idx (chunks of 1 << SH bytes) inside a buffer range.
// The host checks that every range fits 32 bits; the shift is done unsigned
// so offsets past 2^31 stay well defined.
template <int SH>
__device__ __forceinline__ int chunk_off(int idx) {
  return (int)((uint32_t)idx << SH);
}

constexpr int BUF_NT = 2;                  // buffer-load cache policy: non-temporal
constexpr uint32_t BUF_OOB = kLaneOob;     // a lane offset that reads zeros

// ---------------------------------------------------------------------------
// Weight-streaming kernel, for bands of a few rows (decode).  Each wave owns
// NS 16-column subtiles and up to MS 16-row subtiles of one tile (tiles are
// MS * 16 rows), walks the whole K, and has no LDS and no barrier.  Every
// code word loaded feeds one MFMA per row subtile, so a band of up to
// MS * 16 rows streams its expert's codes once per column group.
//
// Pipelining.  A wave's vector loads into registers (this kernel has no
// others) complete in issue order, so waiting for one load also waits for
// every load issued before it.  The activations of a step are therefore
// loaded together with its codes, D steps ahead, into a ring of D + 1
// register slots: step kc first refills slot (kc + D) % (D + 1), which step
// kc - 1 has finished with, with step kc + D, then works on slot
// kc % (D + 1).  Waiting for step kc's data then never waits for a later
// step's, and D steps of codes stay in flight while a step computes.
//
// With only D slots, a slot is read and refilled in the same step; its new
// contents need a second set of registers, and the compiler's copy back
// into the slot at the loop's end waits for the refill just issued, so one
// step is in flight, not D.  The D + 1 ring took a batch-1 w13 decode from
// 25.5 to 20.7 us and the 64-token one from 267.8 to 264.7 us.  The
// eight-subtile waves (two per SIMD) keep D slots, which measured faster for
// them.
//
// Codes, scale words and activations go through buffer loads (base in
// scalar registers, 32-bit lane offsets); activation rows past the band read
// zeros from outside the buffer.
// ---------------------------------------------------------------------------
template <int NS, int D, int MSUB, int FMT, bool OBF16, int ACT, bool GEN>
__device__ __forceinline__ void stream_walk(const uint8_t* __restrict__ packed, const Layout& L,
                                            const Tile& tile, int n0, int h16, __amdgpu_buffer_rsrc_t xr,
                                            const uint32_t (&a_voff)[2], __amdgpu_buffer_rsrc_t cr,
                                            __amdgpu_buffer_rsrc_t sr, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int KC = (int)L.KC;
  const int groups = (int)L.groups;
  const uint32_t c_voff = lane * 16;
  const uint32_t s_voff = lane * 4;

  // 16-byte weight words per lane per chunk: one word of codes, or (bf16
  // weights, FMT 2) the four steps' bf16 operands themselves
  constexpr int CW = FMT == 2 ? 4 : 1;
  // D + 1 slots (four-subtile waves), or D (eight-subtile waves, below)
  constexpr bool SPARE = NS <= 4;
  constexpr int R = SPARE ? D + 1 : D;
  u32x4_t cring[R][NS][CW];
  uint32_t sring[R][NS];
  u32x4_t aring[R][MSUB][4];
  // The codes go first: they depend only on the expert, so the first ones
  // are in flight while the gathered row indices are still arriving.  A step
  // past the last chunk still issues its loads, with lane offsets past every
  // buffer (they fetch nothing and return zeros), so that no branch guards a
  // load: a guarded refill makes the compiler merge the wait counts of both
  // paths and wait for the refill just issued, which leaves one step in
  // flight instead of D.
  auto load_step = [&](int slot, int kc) {
    const bool live = kc < KC;
    const int kq = live ? kc : KC - 1;
    const uint32_t cv = live ? c_voff : BUF_OOB, sv = live ? s_voff : BUF_OOB;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int sub = col_sub<ACT, NS>(ns, h16);
      if constexpr (FMT == 2) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          cring[slot][ns][s] =
              __builtin_amdgcn_raw_buffer_load_b128(cr, cv, chunk_off<12>(sub * KC + kq) + s * 1024, BUF_NT);
      } else {
        cring[slot][ns][0] = __builtin_amdgcn_raw_buffer_load_b128(cr, cv, chunk_off<10>(sub * KC + kq), BUF_NT);
        const int rec = FMT == 0 ? (kq >> 2) : (kq >> 1);
        sring[slot][ns] = __builtin_amdgcn_raw_buffer_load_b32(sr, sv, (sub * groups + rec) * 256, 0);
      }
    }
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        aring[slot][ms][q] =
            __builtin_amdgcn_raw_buffer_load_b128(xr, live ? a_voff[ms] : BUF_OOB, kq * 256 + q * 16, 0);
  };

  f32x4_t acc[MSUB][NS];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[ms][ns] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // step kc's decode (codes c, scale words w) and MFMAs (activations a)
  auto mul = [&](const u32x4_t (&c)[NS][CW], const uint32_t (&w)[NS], const u32x4_t (&a)[MSUB][4], const int kc) {
    float lo[NS], hi[NS];
    if constexpr (FMT != 2) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) chunk_scales<FMT>(w[ns], kc, lo[ns], hi[ns]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        u32x4_t b;
        if constexpr (FMT == 2) b = c[ns][s];
        else b = decode_step<FMT, GEN>(c[ns][0][s], s < 2 ? lo[ns] : hi[ns]);
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms)
          acc[ms][ns] = mfma(as_bf16x8(a[ms][s]), as_bf16x8(b), acc[ms][ns]);
      }
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) load_step(d, d);
  if constexpr (SPARE) {
    // step kc on slot d = kc % R: refill slot (d + D) % R, which step kc - 1
    // finished with, with step kc + D, then work on slot d.  The scheduling
    // barrier keeps the refill whole and ahead of the step's work, so that
    // the loads stay grouped by step in issue order.  Whole rounds of R steps
    // with no branch inside, then the KC % R left.
    auto step = [&](const int d, const int kc) {
      load_step((d + D) % R, kc + D);
      __builtin_amdgcn_sched_barrier(0);
      mul(cring[d], sring[d], aring[d], kc);
    };
    const int KF = KC - KC % R;
    for (int k0 = 0; k0 < KF; k0 += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) step(d, k0 + d);
    }
#pragma unroll
    for (int d = 0; d + 1 < R; ++d)
      if (KF + d < KC) step(d, KF + d);
  } else {
    // Eight-subtile waves (two waves per SIMD, the streaming units of the
    // split kernel) keep D slots: step kc copies slot kc % D to registers,
    // refills it with step kc + D unless that is past the end, and works on
    // the copy.  Its waits are the compiler's merged ones, and with many
    // waves per CU that measured faster than the D + 1 ring (w13 at 512
    // tokens 365.8 against 381.3 us, w2 decode 174.0 against 176.3).
    for (int k0 = 0; k0 < KC; k0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int kc = k0 + d;
        if (kc < KC) {
          u32x4_t c[NS][CW], a[MSUB][4];
          uint32_t w[NS];
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
            for (int i = 0; i < CW; ++i) c[ns][i] = cring[d][ns][i];
            if (FMT != 2) w[ns] = sring[d][ns];
          }
#pragma unroll
          for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q) a[ms][q] = aring[d][ms][q];
          if (kc + D < KC) load_step(d, kc + D);
          mul(c, w, a, kc);
        }
      }
    }
  }

  const float post = FMT == 1 ? reinterpret_cast<const float*>(packed + L.tscale_off)[tile.e] : 1.0f;
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms) {
    if (ACT == 1) {
#pragma unroll
      for (int j = 0; j < NS / 2; ++j)
        store_tile_silu_mul<OBF16>(y, L.N / 2, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + j * 16 + r,
                                   acc[ms][j], acc[ms][j + NS / 2], post);
    } else {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
        store_tile<OBF16>(y, L.N, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + ns * 16 + r, acc[ms][ns],
                          post);
    }
  }
}

// One unit of the weight-streaming kernel: column group nb (four waves of NS
// 16-column subtiles each, or of NS / 2 gate and NS / 2 up subtiles) of a
// tile of up to MS * 16 rows.
template <int NS, int D, int MS, int FMT, bool OBF16, int ACT>
__device__ __forceinline__ void stream_unit(const uint8_t* __restrict__ packed, const Layout& L,
                                            const uint16_t* __restrict__ x, uint32_t x_bytes,
                                            const int32_t* __restrict__ row_index, void* __restrict__ y,
                                            const Tile& tile, int nb) {
  static_assert(ACT == 0 || NS % 2 == 0, "the gate/up activation pairs gate and up subtiles");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // first column (ACT 0) or first gate column (ACT 1) of this wave
  const int n0 = (nb * 4 + wave) * (ACT == 1 ? NS * 8 : NS * 16);
  if (n0 >= (ACT == 1 ? L.N / 2 : L.N)) return;
  const int h16 = ACT == 1 ? (int)(L.N / 32) : 0;
  const int span = ACT == 1 ? h16 + NS / 2 : NS;   // 16-column subtiles the buffer ranges cover
  const int K = (int)L.K;
  const int r = lane & 15;
  const int g = lane >> 4;

  const int64_t et = (int64_t)tile.e * L.NT + (n0 >> 4);
  constexpr int CSH = FMT == 2 ? 12 : 10;   // log2 of a chunk's bytes
  const __amdgpu_buffer_rsrc_t cr = buffer_rsrc(packed + ((et * L.KC) << CSH), (uint32_t)(span * L.KC) << CSH);
  const __amdgpu_buffer_rsrc_t sr =
      buffer_rsrc(packed + L.scales_off + et * L.groups * 256, (uint32_t)(span * L.groups) * 256);
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
  if constexpr (FMT == 1) {
    static_assert(NS == 4, "the NVFP4 flags cover a wave's four subtiles");
    if (!span_scales_pow2<ACT>(packed, L, et, h16)) {
      if (MS == 2 && tile.rows > 16)
        stream_walk<NS, (D > 1 ? D - 1 : 1), 2, FMT, OBF16, ACT, true>(packed, L, tile, n0, h16, xr, a_voff, cr, sr,
                                                                       y);
      else
        stream_walk<NS, D, 1, FMT, OBF16, ACT, true>(packed, L, tile, n0, h16, xr, a_voff, cr, sr, y);
      return;
    }
  }
  if (MS == 2 && tile.rows > 16)
    stream_walk<NS, (D > 1 ? D - 1 : 1), 2, FMT, OBF16, ACT, false>(packed, L, tile, n0, h16, xr, a_voff, cr, sr, y);
  else
    stream_walk<NS, D, 1, FMT, OBF16, ACT, false>(packed, L, tile, n0, h16, xr, a_voff, cr, sr, y);
}

template <int NS, int D, int MS, int FMT, bool OBF16, int ACT>
__global__ __launch_bounds__(256, (NS > 4 || FMT == 1 || D > 2) ? 2 : 3) void gmm_stream_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                         const uint16_t* __restrict__ x,
                                                         uint32_t x_bytes,
                                                         const int32_t* __restrict__ row_index,
                                                         const int32_t* __restrict__ goff, int E,
                                                         void* __restrict__ y, int NB) {
  constexpr int BM = 16 * MS;
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
  const Tile tile = locate_tile(E, BM, ts, t);
  stream_unit<NS, D, MS, FMT, OBF16, ACT>(packed, L, x, x_bytes, row_index, y, tile, nb);
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel, for bands of many rows (prefill).  A workgroup of four
// waves owns a 128-row tile and 256 columns; wave w owns columns 64w..64w+63
// (four 16-column subtiles) for all 128 rows, so every decoded weight feeds
// eight MFMAs.  The activation tile of each 128-deep chunk (gathered rows) is
// copied HBM -> LDS by direct-to-LDS 16-byte buffer loads (no staging
// registers), double-buffered.  A staged row is 256 bytes with its 16-byte
// segments XOR-swizzled by (row & 15), so the 16 rows read by one fragment
// load hit 16 different bank groups.  Codes and scale words stream into
// registers one chunk ahead.  The K walk is compiled per number of valid
// 16-row subtiles, so subtiles past the band end cost nothing.
//
// Waits are explicit.  Per chunk kc a wave issues its share of activation
// chunk kc+1 (LOADS direct-to-LDS loads) and the codes and scale words of
// chunk kc+1 (2 * NS loads), computes chunk kc, then waits for all of its
// loads (vmcnt 0; a count that left the code loads in flight relied on the
// order in which direct-to-LDS and register loads land, and measured no
// faster).  The barrier that follows makes every wave's share visible and
// guarantees that every wave has finished reading buffer kc & 1 before it
// is refilled with chunk kc+2.  The last chunk still stages into buffer
// (kc+1) & 1, which the previous barrier freed, but from an offset past the
// activation buffer, so those loads write zeros without fetching anything;
// its code loads take a lane offset past the codes, so they fetch nothing
// either.
//
// A-fragment reads are ds_read_b128 issued P - 1 fragments ahead of their
// MFMAs (inline asm, so the compiler cannot sink them next to their use);
// before fragment f's MFMAs the wave waits until only the reads issued after
// f are outstanding (LDS reads of a wave complete in order).  The wait is an
// asm statement that takes the fragment register as an in-out operand, so no
// MFMA reading that register can be scheduled above it.
// ---------------------------------------------------------------------------
constexpr int TL_MS = 8;                    // 16-row subtiles per tile
constexpr int TL_NS = 4;                    // 16-column subtiles per wave
static_assert(TL_NS == 4, "span_scales_pow2 reads the flags of four subtiles");
constexpr int TL_WAVES = 4;
constexpr int TL_BM = 16 * TL_MS;           // 128
constexpr int TL_BN = TL_WAVES * 16 * TL_NS;   // 256
constexpr int TL_ROW_BYTES = 128 * 2;       // one staged row of a chunk
constexpr int TL_BUF_BYTES = TL_BM * TL_ROW_BYTES;
constexpr int TL_LOADS = TL_BUF_BYTES / 1024 / TL_WAVES;   // 1 KiB loads per wave per chunk
constexpr int TL_PIPE = 4;                  // A-fragment registers in the read pipeline

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate for gfx9: vmcnt in [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; a field at its maximum does not wait.
template <int VM, int LGKM>
constexpr int waitcnt_imm() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt field");
  return (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8);
}

// Waits until at most VM vector loads of this wave are outstanding and all
// its LDS operations are done, then joins the workgroup barrier.
template <int VM>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<VM, 0>());
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void lds_read_wait(u32x4_t& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}

template <int OFF>
__device__ __forceinline__ u32x4_t lds_read16(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Fragment f of a chunk (step s = f / NSUB, row subtile ms = f % NSUB) of
// the LDS buffer BUF: decode the step's weights at its first fragment, wait
// for the fragment's read, issue its NS MFMAs, then issue the read of
// fragment f + P - 1 into the register of fragment f - 1 (whose MFMAs were
// issued one fragment earlier).
template <int NSUB, int P, int BUF, bool GEN, int F>
__device__ __forceinline__ void tiled_fragment(u32x4_t (&ar)[P], const uint32_t (&va)[4],
                                               u32x4_t (&b)[TL_NS], const u32x4_t (&cw)[TL_NS],
                                               const float (&lo)[TL_NS], const float (&hi)[TL_NS],
                                               f32x4_t (&acc)[TL_MS][TL_NS]) {
  constexpr int FT = 4 * NSUB;
  constexpr int s = F / NSUB, ms = F % NSUB;
  if constexpr (ms == 0) {
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) {
      const float sc = s < 2 ? lo[ns] : hi[ns];
      b[ns] = GEN ? decode8_any_scale(cw[ns][s], sc) : decode8(cw[ns][s], sc);
    }
  }
  constexpr int newest = (F + P - 2 < FT - 1) ? F + P - 2 : FT - 1;
  lds_read_wait<newest - F>(ar[F % P]);
#pragma unroll
  for (int ns = 0; ns < TL_NS; ++ns) acc[ms][ns] = mfma(as_bf16x8(ar[F % P]), as_bf16x8(b[ns]), acc[ms][ns]);
  constexpr int NF = F + P - 1;
  if constexpr (NF < FT)
    ar[NF % P] = lds_read16<(NF % NSUB) * 16 * TL_ROW_BYTES + BUF * TL_BUF_BYTES>(va[NF / NSUB]);
}

template <int NSUB, int P, int BUF, bool GEN, size_t... Fs>
__device__ __forceinline__ void tiled_chunk(std::index_sequence<Fs...>, u32x4_t (&ar)[P], const uint32_t (&va)[4],
                                            u32x4_t (&b)[TL_NS], const u32x4_t (&cw)[TL_NS],
                                            const float (&lo)[TL_NS], const float (&hi)[TL_NS],
                                            f32x4_t (&acc)[TL_MS][TL_NS]) {
  (tiled_fragment<NSUB, P, BUF, GEN, (int)Fs>(ar, va, b, cw, lo, hi, acc), ...);
}

template <int NSUB, int P, int BUF, size_t... Is>
__device__ __forceinline__ void tiled_prologue(std::index_sequence<Is...>, u32x4_t (&ar)[P], const uint32_t (&va)[4]) {
  ((ar[Is] = lds_read16<((int)Is % NSUB) * 16 * TL_ROW_BYTES + BUF * TL_BUF_BYTES>(va[Is / NSUB])), ...);
}

// bf16 weights (FMT 2): the weight words of a step are the MFMA B operands
// themselves, four times the bytes of the codes, so they stream one step at
// a time: bw[s] holds step s of the current chunk, and once the last row
// subtile of step s has issued its MFMAs, bw[s] is refilled with step s of
// the next chunk.  One chunk of weights stays in flight with 64 registers.
template <int NSUB, int P, int BUF, int ACT, int F>
__device__ __forceinline__ void tiled_fragment_bf16(u32x4_t (&ar)[P], const uint32_t (&va)[4],
                                                    u32x4_t (&bw)[4][TL_NS], __amdgpu_buffer_rsrc_t cr,
                                                    uint32_t c_voff, int KC, int h16, int kn,
                                                    f32x4_t (&acc)[TL_MS][TL_NS]) {
  constexpr int FT = 4 * NSUB;
  constexpr int s = F / NSUB, ms = F % NSUB;
  constexpr int newest = (F + P - 2 < FT - 1) ? F + P - 2 : FT - 1;
  lds_read_wait<newest - F>(ar[F % P]);
#pragma unroll
  for (int ns = 0; ns < TL_NS; ++ns) acc[ms][ns] = mfma(as_bf16x8(ar[F % P]), as_bf16x8(bw[s][ns]), acc[ms][ns]);
  constexpr int NF = F + P - 1;
  if constexpr (NF < FT)
    ar[NF % P] = lds_read16<(NF % NSUB) * 16 * TL_ROW_BYTES + BUF * TL_BUF_BYTES>(va[NF / NSUB]);
  if constexpr (ms == NSUB - 1) {
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) {
      const int sub = col_sub<ACT>(ns, h16);
      bw[s][ns] = __builtin_amdgcn_raw_buffer_load_b128(cr, c_voff, chunk_off<12>(sub * KC + kn) + s * 1024, BUF_NT);
    }
  }
}

template <int NSUB, int P, int BUF, int ACT, size_t... Fs>
__device__ __forceinline__ void tiled_chunk_bf16(std::index_sequence<Fs...>, u32x4_t (&ar)[P],
                                                 const uint32_t (&va)[4], u32x4_t (&bw)[4][TL_NS],
                                                 __amdgpu_buffer_rsrc_t cr, uint32_t c_voff, int KC, int h16,
                                                 int kn, f32x4_t (&acc)[TL_MS][TL_NS]) {
  (tiled_fragment_bf16<NSUB, P, BUF, ACT, (int)Fs>(ar, va, bw, cr, c_voff, KC, h16, kn, acc), ...);
}

// The K walk with bf16 weights.  Per chunk a wave issues its share of the
// next activation chunk (LOADS direct-to-LDS loads), then, step by step, the
// next chunk's weights (4 * NS loads); the wait before the barrier leaves
// only those weight loads outstanding (they are issued late in the chunk,
// and a full wait would take them off the pipeline), trusting that the
// 16-byte direct-to-LDS loads issued before them have landed once that many
// loads remain.  On the last chunk the staging loads read past the buffer
// (zeros, no fetch) and the weight loads repeat the last chunk's into the
// unused registers, so the counts stay the same.
template <int NSUB, int ACT>
__device__ __forceinline__ void tiled_k_walk_bf16(uint8_t* s_a, __amdgpu_buffer_rsrc_t xr,
                                                  const uint32_t (&avo)[TL_LOADS], __amdgpu_buffer_rsrc_t cr,
                                                  int KC, int h16, int wave, const uint32_t (&va)[4],
                                                  f32x4_t (&acc)[TL_MS][TL_NS]) {
  constexpr int P = TL_PIPE;
  constexpr int FT = 4 * NSUB;
  constexpr int PRO = (P - 1 < FT) ? P - 1 : FT;
  const int lane = threadIdx.x & 63;
  const uint32_t c_voff = lane * 16;
  u32x4_t bw[4][TL_NS];
  // The staging loads of chunk kn into LDS buffer `buf`: chunk kn's 256-byte
  // slice of every activation row (scalar offset), each lane's row and
  // segment (lane offset avo).  Past the last chunk the lane offsets are
  // moved beyond the activation buffer, so the loads write zeros without a
  // fetch.
  auto stage = [&](int buf, int kn) {
    const bool live = kn < KC;
    const uint32_t soff = live ? (uint32_t)kn * 256u : 0u;
    uint8_t* dst = s_a + buf * TL_BUF_BYTES + wave * TL_LOADS * 1024;
#pragma unroll
    for (int j = 0; j < TL_LOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(dst + j * 1024), 16, live ? avo[j] : BUF_OOB, soff,
                                               0, 0);
  };
  auto chunk = [&](auto bc, int kc) {
    constexpr int d = decltype(bc)::value;   // kc & 1: LDS buffer
    const int kn = min(kc + 1, KC - 1);
    const uint32_t cvn = kc + 1 < KC ? c_voff : BUF_OOB;   // past the last chunk: no fetch
    stage(d ^ 1, kc + 1);
    __builtin_amdgcn_sched_barrier(0);       // the activation loads go first
    u32x4_t ar[P];
    tiled_prologue<NSUB, P, d>(std::make_index_sequence<PRO>{}, ar, va);
    tiled_chunk_bf16<NSUB, P, d, ACT>(std::make_index_sequence<FT>{}, ar, va, bw, cr, cvn, KC, h16, kn, acc);
    vm_wait_barrier<4 * TL_NS>();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  stage(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns)
      bw[s][ns] = __builtin_amdgcn_raw_buffer_load_b128(cr, c_voff, chunk_off<12>(col_sub<ACT>(ns, h16) * KC) + s * 1024,
                                                        BUF_NT);
  vm_wait_barrier<0>();
  int k0 = 0;
  for (; k0 + 2 <= KC; k0 += 2) {
    chunk(B0{}, k0);
    chunk(B1{}, k0 + 1);
  }
  if (k0 < KC) chunk(B0{}, k0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<0, 15>());
}

// The K walk of one wave for a tile with NSUB valid 16-row subtiles.  GEN
// (NVFP4 only): some block scale of the wave's columns is not a power of
// two, so every step takes the general exact decode.
template <int NSUB, int FMT, int ACT, bool GEN = false>
__device__ __forceinline__ void tiled_k_walk(uint8_t* s_a, __amdgpu_buffer_rsrc_t xr,
                                             const uint32_t (&avo)[TL_LOADS], __amdgpu_buffer_rsrc_t cr,
                                             __amdgpu_buffer_rsrc_t sr, int KC, int groups, int h16, int wave,
                                             const uint32_t (&va)[4], f32x4_t (&acc)[TL_MS][TL_NS]) {
  constexpr int P = TL_PIPE;
  constexpr int FT = 4 * NSUB;
  constexpr int PRO = (P - 1 < FT) ? P - 1 : FT;
  const int lane = threadIdx.x & 63;
  const uint32_t c_voff = lane * 16, s_voff = lane * 4;
  u32x4_t cs[2][TL_NS];
  uint32_t ws[2][TL_NS];
  // Load j of wave w fills LDS bytes [(LOADS w + j) KiB, +1 KiB) of the
  // buffer: rows 4(LOADS w + j) .. +3, lane l landing at byte 16 l, i.e. row
  // 4(LOADS w + j) + l/16, physical segment l & 15, which holds logical
  // segment (l & 15) ^ (row & 15) (avo carries the source offsets).
  // The staging loads of chunk kn into LDS buffer `buf`: chunk kn's 256-byte
  // slice of every activation row (scalar offset), each lane's row and
  // segment (lane offset avo).  Past the last chunk the lane offsets are
  // moved beyond the activation buffer, so the loads write zeros without a
  // fetch.
  auto stage = [&](int buf, int kn) {
    const bool live = kn < KC;
    const uint32_t soff = live ? (uint32_t)kn * 256u : 0u;
    uint8_t* dst = s_a + buf * TL_BUF_BYTES + wave * TL_LOADS * 1024;
#pragma unroll
    for (int j = 0; j < TL_LOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(dst + j * 1024), 16, live ? avo[j] : BUF_OOB, soff,
                                               0, 0);
  };
  // past the last chunk the lane offsets point beyond the codes and scale
  // words, so the loads fetch nothing (a branch around them would cost
  // registers across the unrolled walk)
  auto load_codes = [&](int slot, int kc, bool live) {
    const int rec = scale_record<FMT>(kc);
    const uint32_t cv = live ? c_voff : BUF_OOB, sv = live ? s_voff : BUF_OOB;
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) {
      const int sub = col_sub<ACT>(ns, h16);
      cs[slot][ns] = __builtin_amdgcn_raw_buffer_load_b128(cr, cv, chunk_off<10>(sub * KC + kc), BUF_NT);
      ws[slot][ns] = __builtin_amdgcn_raw_buffer_load_b32(sr, sv, (sub * groups + rec) * 256, 0);
    }
  };
  auto chunk = [&](auto bc, int kc) {
    constexpr int d = decltype(bc)::value;   // kc & 1: LDS buffer and code slot
    stage(d ^ 1, kc + 1);
    __builtin_amdgcn_sched_barrier(0);       // the activation loads go first
    load_codes(d ^ 1, min(kc + 1, KC - 1), kc + 1 < KC);
    float lo[TL_NS], hi[TL_NS];
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) chunk_scales<FMT>(ws[d][ns], kc, lo[ns], hi[ns]);
    u32x4_t ar[P];
    u32x4_t b[TL_NS];
    tiled_prologue<NSUB, P, d>(std::make_index_sequence<PRO>{}, ar, va);
    tiled_chunk<NSUB, P, d, GEN>(std::make_index_sequence<FT>{}, ar, va, b, cs[d], lo, hi, acc);
    vm_wait_barrier<0>();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  stage(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_codes(0, 0, true);
  vm_wait_barrier<0>();
  int k0 = 0;
  for (; k0 + 2 <= KC; k0 += 2) {
    chunk(B0{}, k0);
    chunk(B1{}, k0 + 1);
  }
  if (k0 < KC) chunk(B0{}, k0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm<0, 15>());
}

// One unit of the LDS-tiled kernel: column group nb (TL_BN columns, or
// TL_BN / 2 activation columns) of a tile of up to TL_BM rows, staged through
// the workgroup's LDS buffers s_a.
template <int FMT, bool OBF16, int ACT>
__device__ __forceinline__ void tiled_unit(uint8_t* s_a, const uint8_t* __restrict__ packed, const Layout& L,
                                           const uint16_t* __restrict__ x, uint32_t x_bytes,
                                           const int32_t* __restrict__ row_index, void* __restrict__ y,
                                           const Tile& tile, int nb) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = (int)L.K;
  const int KC = (int)L.KC;
  const int groups = (int)L.groups;
  // first column (ACT 0) or first gate column (ACT 1) of this wave
  const int n0 = ACT == 1 ? nb * (TL_BN / 2) + wave * 32 : nb * TL_BN + wave * 16 * TL_NS;
  // A wave past the last column still stages its share of the activations
  // and joins every barrier; its code loads read zeros and it stores nothing.
  const bool wave_active = n0 < (ACT == 1 ? L.N / 2 : L.N);
  const int h16 = ACT == 1 ? (int)(L.N / 32) : 0;
  const int span = ACT == 1 ? h16 + 2 : TL_NS;   // 16-column subtiles the buffer ranges cover
  const int r = lane & 15;
  const int g = lane >> 4;
  const int nsub = (tile.rows + 15) >> 4;

  // Source offsets of this lane's staging loads; rows past the band read
  // zeros (their accumulator rows are never stored).
  uint32_t avo[TL_LOADS];
#pragma unroll
  for (int j = 0; j < TL_LOADS; ++j) {
    const int rl = 4 * (wave * TL_LOADS + j) + (lane >> 4);
    avo[j] = BUF_OOB;
    if (rl < tile.rows) {
      const int row = tile.m0 + rl;
      const int64_t src = row_index ? row_index[row] : row;
      avo[j] = (uint32_t)(src * K * 2 + (((lane & 15) ^ (rl & 15)) << 4));
    }
  }
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, x_bytes);
  const int64_t et = (int64_t)tile.e * L.NT + (wave_active ? (n0 >> 4) : 0);
  constexpr int CSH = FMT == 2 ? 12 : 10;   // log2 of a chunk's bytes
  const __amdgpu_buffer_rsrc_t cr =
      buffer_rsrc(packed + ((et * L.KC) << CSH), wave_active ? (uint32_t)(span * KC) << CSH : 0u);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(packed + L.scales_off + et * L.groups * 256,
                                                wave_active ? (uint32_t)(span * groups) * 256 : 0u);
  // LDS address of this lane's fragment row for step s: row r of the
  // subtile, logical segment g*4 + s
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)s_a;
  uint32_t va[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) va[s] = lds0 + r * TL_ROW_BYTES + (((g * 4 + s) ^ r) << 4);

  f32x4_t acc[TL_MS][TL_NS];
#pragma unroll
  for (int ms = 0; ms < TL_MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) acc[ms][ns] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (FMT == 2) {
    switch (nsub) {
      case 1: tiled_k_walk_bf16<1, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
      case 2: tiled_k_walk_bf16<2, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
      case 3: tiled_k_walk_bf16<3, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
      case 4: tiled_k_walk_bf16<4, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
      case 5: tiled_k_walk_bf16<5, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
      case 6: tiled_k_walk_bf16<6, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
      case 7: tiled_k_walk_bf16<7, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
      default: tiled_k_walk_bf16<8, ACT>(s_a, xr, avo, cr, KC, h16, wave, va, acc); break;
    }
  } else if (FMT == 1 && wave_active && !span_scales_pow2<ACT>(packed, L, et, h16)) {
    // general E4M3 scales: one walk over all eight subtiles (the rows past
    // the band are zeros in LDS and are never stored)
    tiled_k_walk<8, FMT, ACT, true>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc);
  } else switch (nsub) {
    case 1: tiled_k_walk<1, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
    case 2: tiled_k_walk<2, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
    case 3: tiled_k_walk<3, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
    case 4: tiled_k_walk<4, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
    case 5: tiled_k_walk<5, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
    case 6: tiled_k_walk<6, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
    case 7: tiled_k_walk<7, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
    default: tiled_k_walk<8, FMT, ACT>(s_a, xr, avo, cr, sr, KC, groups, h16, wave, va, acc); break;
  }

  if (!wave_active) return;
  const float post = FMT == 1 ? reinterpret_cast<const float*>(packed + L.tscale_off)[tile.e] : 1.0f;
#pragma unroll
  for (int ms = 0; ms < TL_MS; ++ms) {
    if (ms < nsub) {
      if (ACT == 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          store_tile_silu_mul<OBF16>(y, L.N / 2, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + j * 16 + r,
                                     acc[ms][j], acc[ms][j + 2], post);
      } else {
#pragma unroll
        for (int ns = 0; ns < TL_NS; ++ns)
          store_tile<OBF16>(y, L.N, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + ns * 16 + r,
                            acc[ms][ns], post);
      }
    }
  }
}

template <int FMT, bool OBF16, int ACT>
__global__ __launch_bounds__(256, 2) void gmm_tiled_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                           const uint16_t* __restrict__ x, uint32_t x_bytes,
                                                           const int32_t* __restrict__ row_index,
                                                           const int32_t* __restrict__ goff, int E,
                                                           void* __restrict__ y, int NB) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_a[2 * TL_BUF_BYTES];

  const TileScan ts = scan_tiles(goff, E, TL_BM);
  const int item = work_item(ts.total * NB, true);
  if (item < 0) return;
  const int t = item / NB;
  const int nb = item - t * NB;
  const Tile tile = locate_tile(E, TL_BM, ts, t);
  tiled_unit<FMT, OBF16, ACT>(s_a, packed, L, x, x_bytes, row_index, y, tile, nb);
}

// ---------------------------------------------------------------------------
// Split kernel, for MXFP4 bands of mixed sizes (the eight-subtile streaming
// path: bands of 4 rows or more on average, for instance the down projection
// under skewed routing).  The weight-streaming units walk a band once per
// 32-row tile, so a band of 201 rows would stream its expert's codes seven
// times; here every band of more than SPLIT_TH rows runs as LDS-tiled units
// instead, which stream them once per 128 rows, and the other bands run as
// weight-streaming units.  (A threshold of 64 rows measured faster than 32:
// the host's bound on the tiled units, and so the workgroups that find none,
// halves.)  One launch, so both kinds share the chip: the
// first HB workgroups (an upper bound on the tiled units) take one tiled
// unit each or exit after the scan, the rest one streaming tile each.  (A
// loop over several tiled units per workgroup spilled registers; streaming
// tiles placed right after the real tiled units spilled scalar registers and
// measured the same.)  A tiled unit covers TBM = 128 rows of a band, or 64
// when the whole grid fits one round of workgroups (one GPU's share under
// expert parallelism, say): a few thick bands then spread over twice the
// CUs.  Both kinds issue the same MFMAs in the same order as the stream and
// tiled kernels, so the output bits are the same.
// ---------------------------------------------------------------------------
constexpr int SPLIT_TH = 64;   // bands of more rows run as tiled units
constexpr int SPLIT_BM = 32;   // rows of a streaming tile

template <bool OBF16>
__global__ __launch_bounds__(256, 2) void gmm_split_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                           const uint16_t* __restrict__ x, uint32_t x_bytes,
                                                           const int32_t* __restrict__ row_index,
                                                           const int32_t* __restrict__ goff, int E,
                                                           void* __restrict__ y, int NB, int HB, int TBM) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_a[2 * TL_BUF_BYTES];
  const int bx = blockIdx.x;
  if (bx < HB) {
    const int NBT = (int)((L.N + TL_BN - 1) / TL_BN);
    const TileScan ts = scan_tiles(goff, E, TBM, SPLIT_TH + 1);
    if (bx >= ts.total * NBT) return;
    const int t = bx / NBT;
    const Tile tile = locate_tile(E, TBM, ts, t);
    tiled_unit<0, OBF16, 0>(s_a, packed, L, x, x_bytes, row_index, y, tile, bx - t * NBT);
    return;
  }
  // streaming tiles dealt to the XCDs as in the stream kernel (HB is a
  // multiple of 8, so workgroup bx still runs on XCD bx & 7)
  const TileScan ts = scan_tiles(goff, E, SPLIT_BM, 1, SPLIT_TH);
  const int sb = bx - HB;
  const int xcd = sb & 7, kth = sb >> 3;
  const int t = xcd + 8 * (kth / NB);
  const int nb = kth - (kth / NB) * NB;
  if (t >= ts.total) return;
  const Tile tile = locate_tile(E, SPLIT_BM, ts, t);
  stream_unit<8, 2, 2, 0, OBF16, 0>(packed, L, x, x_bytes, row_index, y, tile, nb);
}

// ---------------------------------------------------------------------------
// W4A4 kernel (prefill): 4-bit weights times MXFP4-quantized activations on
// gfx950's scaled FP4 MFMA, v_mfma_scale_f32_16x16x128_f8f6f4 (e2m1 A and B).
// MXFP4 weights pass their E8M0 bytes to the instruction as they are.  NVFP4
// weights qualify when the two E4M3 scales of every 32-block are one equal
// power of two (so for every pack made by the lossless MXFP4 cast): that
// scale becomes the block's E8M0 byte and the per-expert tensor scale is one
// multiply in the epilogue, so the f32 sums are exactly those of the MXFP4
// weights the cast came from.  A block that does not qualify is counted in
// err_count (its outputs are unspecified).
// Its operands match the packed weights exactly: lane l supplies the 32 codes
// (16 bytes, low nibble first) of column (l & 15), K block (l >> 4) of a
// 128-deep chunk and that block's E8M0 scale (byte 0 of the scale operand);
// A is the same for row (l & 15) of the activations, and the f32 result has
// the layout of the bf16 MFMA's.  One MFMA covers a whole chunk of a 16 x 16
// tile.
//
// Same workgroup shape as the tiled kernel: 4 waves, 128 rows x 256
// columns, the activation chunk staged in LDS by direct-to-LDS loads.  Two
// chunks are staged (LDS buffers for the activations, register pairs for
// each wave's weight codes and weight scale words): chunk kc + 1 loads
// while chunk kc is computed, and the last chunk fetches nothing.  A staged
// chunk holds the 128 rows' codes (64 bytes per row, rows contiguous:
// 8 KiB) and their scale dwords (wave w loads rows 32w .. 32w+31 into its
// own 256-byte slot; lanes 32..63 read past the buffer and write zeros into
// the slot's unused half).
//
// Each chunk ends by waiting for all of the wave's loads (vmcnt 0), not for
// a count that leaves later loads in flight.  A counted wait let a third
// staged chunk's loads stay in flight, and on MI355X some 4-byte
// direct-to-LDS loads (the weight scale words, then staged in LDS) had not
// landed when their stage was read: one 16-column subtile of a few thin
// tiles came out wrong, differently from run to run.  With the full wait a
// third stage buys nothing, and two stages measured the same.  The weight
// scale words, which no other lane reads, now go to registers.
// ---------------------------------------------------------------------------
constexpr int Q_CODE_BYTES = TL_BM * 64;                     // 8 KiB
constexpr int Q_SCALE_BYTES = TL_WAVES * 256;
constexpr int Q_STAGE_BYTES = Q_CODE_BYTES + Q_SCALE_BYTES;
constexpr int Q_LOADS = Q_CODE_BYTES / 1024 / TL_WAVES;      // 1 KiB code loads per wave per chunk
constexpr int Q_STAGES = 2;                                   // chunks staged: one loading, one computed

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_fp4(u32x4_t a, uint32_t sa, u32x4_t b, uint32_t sb, f32x4_t c) {
  const i32x8_t A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8_t B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // cbsz = blgp = 4: e2m1 operands; op_sel 0: byte 0 of each scale operand
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// The E8M0 operand of one lane's 32-block in chunk kc from its packed scale
// word.  NVFP4: the block qualifies when its two E4M3 bytes are equal and
// hold a positive power of two (normal or subnormal); `bad` counts the
// lane's blocks that do not.
template <int FMT>
__device__ __forceinline__ uint32_t w4a4_block_scale(uint32_t word, int kc, int& bad) {
  if (FMT == 0) return (word >> (8 * (kc & 3))) & 0xFFu;
  // The hardware E4M3 convert gives the low byte's exact f32 value: a
  // positive power of two has a zero sign and mantissa, and its f32 exponent
  // field is the E8M0 byte.  Integer minima stand in for comparisons (lane
  // masks would sit in scalar registers across the unrolled walk).
  const uint32_t pair = word >> (16 * (kc & 1));
  const uint32_t bits = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8(pair, 0));
  const uint32_t off = min((pair ^ (pair >> 8)) & 0xFFu, 1u) | min(bits & 0x807FFFFFu, 1u) | (1u - min(bits, 1u));
  bad += (int)off;
  return off ? 127u : bits >> 23;
}

// The K walk of one wave over a tile with NSUB valid 16-row subtiles.
template <int NSUB, int FMT, int ACT>
__device__ __forceinline__ void w4a4_k_walk(uint8_t* s_q, __amdgpu_buffer_rsrc_t qcr, __amdgpu_buffer_rsrc_t qsr,
                                            const uint32_t (&cvo)[Q_LOADS], uint32_t svo,
                                            __amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr, int KC,
                                            int groups, int h16, int wave, f32x4_t (&acc)[TL_MS][TL_NS],
                                            int& bad) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const uint32_t c_voff = lane * 16, s_voff = lane * 4;
  u32x4_t cs[Q_STAGES][TL_NS];
  uint32_t ws[Q_STAGES][TL_NS];
  // all loads of chunk kc into stage `slot`: the activation codes and scales
  // (direct to LDS, shared by the four waves), then this wave's weight codes
  // and weight scale words (registers)
  // (live false: lane offsets past every buffer, so the loads fetch nothing;
  // a branch around them would cost registers across the unrolled walk)
  auto issue = [&](auto sc, int kc, bool live) {
    constexpr int slot = decltype(sc)::value;
    uint8_t* buf = s_q + slot * Q_STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < Q_LOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qcr, (lds_ptr_t)(buf + (wave * Q_LOADS + j) * 1024), 16,
                                               live ? cvo[j] : BUF_OOB, kc * 64, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qsr, (lds_ptr_t)(buf + Q_CODE_BYTES + wave * 256), 4,
                                             live ? svo : BUF_OOB, kc * 4, 0, 0);
    __builtin_amdgcn_sched_barrier(0);       // the activation loads go first
    const int rec = scale_record<FMT>(kc);
    const uint32_t cv = live ? c_voff : BUF_OOB, sv = live ? s_voff : BUF_OOB;
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) {
      const int sub = col_sub<ACT>(ns, h16);
      cs[slot][ns] = __builtin_amdgcn_raw_buffer_load_b128(cr, cv, chunk_off<10>(sub * KC + kc), BUF_NT);
      ws[slot][ns] = __builtin_amdgcn_raw_buffer_load_b32(sr, sv, (sub * groups + rec) * 256, 0);
    }
  };
  // Chunk kc (stage kc & 1) issues chunk kc + 1 into the other stage (freed
  // by the barrier that ended chunk kc - 1; the last chunk's loads fetch
  // nothing),
  // computes, then waits for every load of the wave: chunk kc + 1 has then
  // landed for every wave when the barrier opens.
  auto chunk = [&](auto sc, int kc) {
    constexpr int d = decltype(sc)::value;
    issue(std::integral_constant<int, d ^ 1>{}, min(kc + 1, KC - 1), kc + 1 < KC);
    const uint8_t* buf = s_q + d * Q_STAGE_BYTES;
    uint32_t sb[TL_NS];
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns)
      sb[ns] = w4a4_block_scale<FMT>(ws[d][ns], kc, bad);
#pragma unroll
    for (int ms = 0; ms < NSUB; ++ms) {
      const int row = ms * 16 + r;
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(buf + row * 64 + g * 16);
      const uint32_t sdw = *reinterpret_cast<const uint32_t*>(buf + Q_CODE_BYTES + (row >> 5) * 256 + (row & 31) * 4);
      const uint32_t sa = (sdw >> (8 * g)) & 0xFFu;
#pragma unroll
      for (int ns = 0; ns < TL_NS; ++ns) acc[ms][ns] = mfma_fp4(a, sa, cs[d][ns], sb[ns], acc[ms][ns]);
    }
    vm_wait_barrier<0>();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  issue(S0{}, 0, true);
  vm_wait_barrier<0>();
  int k0 = 0;
  for (; k0 + 2 <= KC; k0 += 2) {
    chunk(S0{}, k0);
    chunk(S1{}, k0 + 1);
  }
  if (k0 < KC) chunk(S0{}, k0);
}

template <int FMT, bool OBF16, int ACT>
__global__ __launch_bounds__(256, 2) void gmm_w4a4_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                          const uint8_t* __restrict__ qcodes,
                                                          const uint8_t* __restrict__ qscales, int32_t x_rows,
                                                          const int32_t* __restrict__ row_index,
                                                          const int32_t* __restrict__ goff, int E,
                                                          void* __restrict__ y, int NB,
                                                          int32_t* __restrict__ err_count) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_q[Q_STAGES * Q_STAGE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TileScan ts = scan_tiles(goff, E, TL_BM);
  const int item = work_item(ts.total * NB, true);
  if (item < 0) return;
  const int t = item / NB;
  const int nb = item - t * NB;
  const Tile tile = locate_tile(E, TL_BM, ts, t);
  const int K = (int)L.K;
  const int KC = (int)L.KC;
  const int groups = (int)L.groups;
  const int n0 = ACT == 1 ? nb * (TL_BN / 2) + wave * 32 : nb * TL_BN + wave * 16 * TL_NS;
  const bool wave_active = n0 < (ACT == 1 ? L.N / 2 : L.N);
  const int h16 = ACT == 1 ? (int)(L.N / 32) : 0;
  const int span = ACT == 1 ? h16 + 2 : TL_NS;
  const int r = lane & 15;
  const int nsub = (tile.rows + 15) >> 4;

  // Staging sources: code load j of wave w covers rows 16(Q_LOADS w + j) + l/4,
  // 16-byte segment l & 3 of the row's 64 code bytes per chunk; the scale load
  // of wave w covers rows 32w + l for lanes l < 32.  Rows past the band read
  // zeros (their accumulator rows are never stored).
  uint32_t cvo[Q_LOADS];
#pragma unroll
  for (int j = 0; j < Q_LOADS; ++j) {
    const int rl = 16 * (wave * Q_LOADS + j) + (lane >> 2);
    cvo[j] = BUF_OOB;
    if (rl < tile.rows) {
      const int64_t src = row_index ? row_index[tile.m0 + rl] : tile.m0 + rl;
      cvo[j] = (uint32_t)(src * (K / 2) + (lane & 3) * 16);
    }
  }
  uint32_t svo = BUF_OOB;
  {
    const int rl = 32 * wave + lane;
    if (lane < 32 && rl < tile.rows) {
      const int64_t src = row_index ? row_index[tile.m0 + rl] : tile.m0 + rl;
      svo = (uint32_t)(src * (K / 32));
    }
  }
  // The sizes go through readfirstlane: K / 32 also feeds the divergent svo
  // above, and the compiler would otherwise build the descriptor in vector
  // registers and wrap every load through it in a waterfall loop.
  const __amdgpu_buffer_rsrc_t qcr =
      buffer_rsrc(qcodes, (uint32_t)__builtin_amdgcn_readfirstlane((int)((int64_t)x_rows * (K / 2))));
  const __amdgpu_buffer_rsrc_t qsr =
      buffer_rsrc(qscales, (uint32_t)__builtin_amdgcn_readfirstlane((int)((int64_t)x_rows * (K / 32))));
  const int64_t et = (int64_t)tile.e * L.NT + (wave_active ? (n0 >> 4) : 0);
  const __amdgpu_buffer_rsrc_t cr =
      buffer_rsrc(packed + ((et * L.KC) << 10), wave_active ? (uint32_t)(span * KC) << 10 : 0u);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(packed + L.scales_off + et * L.groups * 256,
                                                wave_active ? (uint32_t)(span * groups) * 256 : 0u);

  f32x4_t acc[TL_MS][TL_NS];
#pragma unroll
  for (int ms = 0; ms < TL_MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < TL_NS; ++ns) acc[ms][ns] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int bad = 0;
  switch (nsub) {
    case 1: w4a4_k_walk<1, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
    case 2: w4a4_k_walk<2, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
    case 3: w4a4_k_walk<3, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
    case 4: w4a4_k_walk<4, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
    case 5: w4a4_k_walk<5, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
    case 6: w4a4_k_walk<6, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
    case 7: w4a4_k_walk<7, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
    default: w4a4_k_walk<8, FMT, ACT>(s_q, qcr, qsr, cvo, svo, cr, sr, KC, groups, h16, wave, acc, bad); break;
  }

  if (!wave_active) return;
  if (FMT == 1 && err_count && tile.first) {
    // each weight block is counted once: by its expert's first tile
    for (int d = 32; d > 0; d >>= 1) bad += __shfl_xor(bad, d, 64);
    if (lane == 0 && bad) atomicAdd(err_count, bad);
  }
  const float post = FMT == 1 ? reinterpret_cast<const float*>(packed + L.tscale_off)[tile.e] : 1.0f;
#pragma unroll
  for (int ms = 0; ms < TL_MS; ++ms) {
    if (ms < nsub) {
      if (ACT == 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          store_tile_silu_mul<OBF16>(y, L.N / 2, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + j * 16 + r,
                                     acc[ms][j], acc[ms][j + 2], post);
      } else {
#pragma unroll
        for (int ns = 0; ns < TL_NS; ++ns)
          store_tile<OBF16>(y, L.N, tile.m0 + ms * 16, tile.rows - ms * 16, n0 + ns * 16 + r,
                            acc[ms][ns], post);
      }
    }
  }
}

// Grids.  The host launches an upper bound on the tiles (the band sizes are
// on the device) times the column groups; workgroups past the real tiles exit
// at once.  A dispatch counts its work-items in 32 bits, so the host checks
// these counts (gmm_workgroups) before it launches anything.
struct TiledGrid {
  int NB;           // column groups of TL_BN columns (TL_BN / 2 gated columns)
  int64_t groups;
};

static TiledGrid tiled_grid(int act, int64_t N, int64_t E, int64_t M) {
  const int64_t em = E < M ? E : M;
  const int64_t cols = act == 1 ? N / 2 : N;
  const int64_t bn = act == 1 ? TL_BN / 2 : TL_BN;
  const int64_t NB = (cols + bn - 1) / bn;
  return {(int)NB, ((M + TL_BM - 1) / TL_BM + em) * NB};
}

struct StreamGrid {
  bool split;       // the split kernel (MXFP4, no activation, mean band >= 4 rows)
  bool narrow;      // two-subtile waves with a deep ring (a grid of at most one wave per SIMD)
  int NB;           // column groups of one streaming workgroup
  int HB;           // split kernel: workgroups reserved for tiled units
  int TBM;          // split kernel: rows of a tiled unit
  int64_t groups;
};

// Split-kernel workgroups that run at once (two per CU on 256 CUs).
constexpr int64_t SPLIT_ROUND = 512;
// Waves of a grid that gets at most one wave per SIMD (4 SIMDs on 256 CUs).
constexpr int64_t NARROW_WAVES = 1024;

// Stream-kernel shape: four 16-column subtiles per wave (64 columns, fewer
// and longer waves amortise the tile lookup and activation loads), and tiles
// of up to 32 rows: a popular expert's band streams its codes once per 32
// rows instead of once per 16.  bf16 weights (fmt 2) carry four times the
// bytes per column, so their waves own two subtiles (32 columns).
//
// With a mean band of 4 rows or more the activation loads (one 16-row
// subtile of 16-byte loads per wave and chunk, whatever the weight count)
// fetch real rows and cost as much load issue as the codes: eight subtiles
// per wave (two waves per SIMD) halve them per weight byte, and such problems
// can hold bands long enough for the tiled units of the split kernel.  That
// kernel takes bands of more than SPLIT_TH rows (at most min(E, M /
// (SPLIT_TH + 1)) of them) as tiled units, one workgroup each, and the other
// bands as streaming tiles of SPLIT_BM rows.  Its tiled units cover 128 rows,
// or 64 when the whole grid is one round of workgroups: 64-row units spread
// the few thick bands of a small problem over twice the CUs (one GPU's share
// of the w2 decode under 8-way expert parallelism: 40.9 -> 36.8 us, while
// 32-row units gave 40.4 and every band as streaming tiles 49.5).  Thinner
// bands keep four subtiles and three waves per SIMD (two with NVFP4 weights).
//
// A grid whose bound gives at most one wave per SIMD even with two subtiles
// per wave (a batch-1 decode: six rows) is bound by each wave's serial walk:
// its MFMAs on a one-row band and the load latency with two chunks in
// flight each take about 0.4 us a chunk.  MXFP4 waves then own two
// subtiles and keep four chunks in flight (two waves
// per SIMD of registers): batch-1 w13 decode 20.5 -> 16.4 us, batch-1 w2
// 14.5 -> 11.9 us.  With more waves than SIMDs the same shape was slower
// (two tokens: 24.2 -> 26.5 us).  With the fused activation such a wave
// owns one gate and one up subtile.
static StreamGrid stream_grid(int fmt, int act, int64_t N, int64_t E, int64_t M) {
  const int64_t cols = act == 1 ? N / 2 : N;
  const int64_t em = E < M ? E : M;
  if (act == 0 && fmt == 0 && M >= 4 * E && N % 128 == 0) {
    const int64_t NB = (cols + 512 - 1) / 512;
    const int64_t NBT = (cols + TL_BN - 1) / TL_BN;
    const int64_t thick = M / (SPLIT_TH + 1) < em ? M / (SPLIT_TH + 1) : em;
    const int64_t thin = (M / SPLIT_BM + em + 7) / 8 * 8;
    // the bands of more than SPLIT_TH rows hold at most M / TBM more tiles
    // than bands
    auto reserve = [&](int64_t tbm) { return ((M / tbm + thick) * NBT + 7) / 8 * 8; };
    const int64_t HB = reserve(TL_BM);
    if (HB + thin * NB <= SPLIT_ROUND) {
      const int64_t HS = reserve(TL_BM / 2);
      return {true, false, (int)NB, (int)HS, TL_BM / 2, HS + thin * NB};
    }
    return {true, false, (int)NB, (int)HB, TL_BM, HB + thin * NB};
  }
  const int64_t BM = 32;
  const int64_t tiles = ((M + BM - 1) / BM + em + 7) / 8 * 8;   // whole rounds of 8 tiles
  if (fmt == 0) {
    // two-subtile waves: 32 output columns, or 16 gate and 16 up columns
    const int64_t per2 = act == 1 ? 64 : 128;
    const int64_t NB2 = (cols + per2 - 1) / per2;
    if (4 * tiles * NB2 <= NARROW_WAVES) return {false, true, (int)NB2, 0, TL_BM, tiles * NB2};
  }
  // a workgroup covers 4 * 64 output columns (4 * 32 with bf16 weights), or
  // 4 * 32 activation columns
  const int64_t per = act == 1 ? 128 : (fmt == 2 ? 128 : 256);
  const int64_t NB = (cols + per - 1) / per;
  return {false, false, (int)NB, 0, TL_BM, tiles * NB};
}

int64_t gmm_workgroups(int fmt, int32_t E, int32_t N, int32_t M, int act, int kernel) {
  return kernel == 1 ? stream_grid(fmt, act, N, E, M).groups : tiled_grid(act, N, E, M).groups;
}

template <int FMT, bool OBF16, int ACT>
static void launch_w4a4_t(const uint8_t* packed, const Layout& L, const uint8_t* qcodes, const uint8_t* qscales,
                          int32_t x_rows, const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                          void* y, int32_t* err_count, hipStream_t stream) {
  const TiledGrid g = tiled_grid(ACT, L.N, E, M);
  hipLaunchKernelGGL((gmm_w4a4_kernel<FMT, OBF16, ACT>), dim3((unsigned)g.groups), dim3(64 * TL_WAVES), 0,
                     stream, packed, L, qcodes, qscales, x_rows, row_index, goff, E, y, g.NB, err_count);
}

template <int FMT>
static void launch_w4a4_f(const uint8_t* packed, const Layout& L, const uint8_t* qcodes, const uint8_t* qscales,
                          int32_t x_rows, const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                          void* y, int y_bf16, int act, int32_t* err_count, hipStream_t stream) {
  if (act == 1) {
    if (y_bf16) launch_w4a4_t<FMT, true, 1>(packed, L, qcodes, qscales, x_rows, row_index, goff, E, M, y, err_count, stream);
    else launch_w4a4_t<FMT, false, 1>(packed, L, qcodes, qscales, x_rows, row_index, goff, E, M, y, err_count, stream);
  } else {
    if (y_bf16) launch_w4a4_t<FMT, true, 0>(packed, L, qcodes, qscales, x_rows, row_index, goff, E, M, y, err_count, stream);
    else launch_w4a4_t<FMT, false, 0>(packed, L, qcodes, qscales, x_rows, row_index, goff, E, M, y, err_count, stream);
  }
}

hipError_t launch_gmm_w4a4(const uint8_t* packed, int fmt, int32_t E, int32_t N, int32_t K, const uint8_t* qcodes,
                           const uint8_t* qscales, int32_t x_rows, const int32_t* row_index,
                           const int32_t* group_offsets, int32_t M, void* y, int y_bf16, int act,
                           int32_t* err_count, hipStream_t stream) {
  const Layout L = make_layout(fmt, E, N, K);
  if (err_count) launch_zero_i32(err_count, 1, stream);
  if (fmt == 1)
    launch_w4a4_f<1>(packed, L, qcodes, qscales, x_rows, row_index, group_offsets, E, M, y, y_bf16, act, err_count,
                     stream);
  else
    launch_w4a4_f<0>(packed, L, qcodes, qscales, x_rows, row_index, group_offsets, E, M, y, y_bf16, act, err_count,
                     stream);
  return hipGetLastError();
}

template <int FMT, bool OBF16, int ACT>
static void launch_stream(const uint8_t* packed, const Layout& L, const uint16_t* x, uint32_t x_bytes,
                          const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                          void* y, hipStream_t stream) {
  // two chunks in flight for one-subtile tiles; the two-subtile walk keeps
  // one so that both walks fit three workgroups per CU (two with NVFP4
  // weights, whose walks for general E4M3 scales need more registers: at
  // three they spilled and ran 3 % slower)
  constexpr int NS = FMT == 2 ? 2 : 4, D = 2, MS = 2;
  const StreamGrid g = stream_grid(FMT, ACT, L.N, E, M);
  if constexpr (ACT == 0 && FMT == 0) {
    if (g.split) {
      hipLaunchKernelGGL((gmm_split_kernel<OBF16>), dim3((unsigned)g.groups), dim3(256), 0, stream, packed,
                         L, x, x_bytes, row_index, goff, E, y, g.NB, g.HB, g.TBM);
      return;
    }
  }
  if constexpr (FMT == 0) {
    if (g.narrow) {
      hipLaunchKernelGGL((gmm_stream_kernel<2, 4, MS, FMT, OBF16, ACT>), dim3((unsigned)g.groups), dim3(256), 0,
                         stream, packed, L, x, x_bytes, row_index, goff, E, y, g.NB);
      return;
    }
  }
  hipLaunchKernelGGL((gmm_stream_kernel<NS, D, MS, FMT, OBF16, ACT>), dim3((unsigned)g.groups),
                     dim3(256), 0, stream, packed, L, x, x_bytes, row_index, goff, E, y, g.NB);
}

template <int FMT, bool OBF16, int ACT>
static void launch_tiled(const uint8_t* packed, const Layout& L, const uint16_t* x, uint32_t x_bytes,
                         const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                         void* y, hipStream_t stream) {
  const TiledGrid g = tiled_grid(ACT, L.N, E, M);
  hipLaunchKernelGGL((gmm_tiled_kernel<FMT, OBF16, ACT>), dim3((unsigned)g.groups), dim3(64 * TL_WAVES), 0,
                     stream, packed, L, x, x_bytes, row_index, goff, E, y, g.NB);
}

template <int FMT, bool OBF16, int ACT>
static void launch_gmm_t(const uint8_t* packed, const Layout& L, const uint16_t* x, int32_t x_rows,
                         const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                         void* y, int kernel, hipStream_t stream) {
  const uint32_t x_bytes = (uint32_t)((int64_t)x_rows * L.K * 2);
  if (kernel == 1) launch_stream<FMT, OBF16, ACT>(packed, L, x, x_bytes, row_index, goff, E, M, y, stream);
  else launch_tiled<FMT, OBF16, ACT>(packed, L, x, x_bytes, row_index, goff, E, M, y, stream);
}

template <int FMT, bool OBF16>
static void launch_gmm_a(const uint8_t* packed, const Layout& L, const uint16_t* x, int32_t x_rows,
                         const int32_t* row_index, const int32_t* goff, int32_t E, int32_t M,
                         void* y, int act, int kernel, hipStream_t stream) {
  if constexpr (FMT == 2) {
    launch_gmm_t<FMT, OBF16, 0>(packed, L, x, x_rows, row_index, goff, E, M, y, kernel, stream);
  } else {
    if (act == 1) launch_gmm_t<FMT, OBF16, 1>(packed, L, x, x_rows, row_index, goff, E, M, y, kernel, stream);
    else launch_gmm_t<FMT, OBF16, 0>(packed, L, x, x_rows, row_index, goff, E, M, y, kernel, stream);
  }
}

hipError_t launch_gmm(const uint8_t* packed, int fmt, int32_t E, int32_t N, int32_t K,
                      const uint16_t* x, int32_t x_rows, const int32_t* row_index,
                      const int32_t* group_offsets, int32_t M, void* y, int y_bf16, int act,
                      int kernel, hipStream_t stream) {
  const Layout L = make_layout(fmt, E, N, K);
  if (fmt == 0) {
    if (y_bf16) launch_gmm_a<0, true>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, act, kernel, stream);
    else launch_gmm_a<0, false>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, act, kernel, stream);
  } else if (fmt == 1) {
    if (y_bf16) launch_gmm_a<1, true>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, act, kernel, stream);
    else launch_gmm_a<1, false>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, act, kernel, stream);
  } else {
    if (y_bf16) launch_gmm_a<2, true>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, act, kernel, stream);
    else launch_gmm_a<2, false>(packed, L, x, x_rows, row_index, group_offsets, E, M, y, act, kernel, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
