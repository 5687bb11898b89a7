/*
 * moe_gmm.h - routed-expert W4A16 grouped matmul for AMD MI355X (gfx950).
 *
 * C ABI of libmoegmm.so: the routed-expert matmuls of one MoE layer
 * (source: "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that
 * v6e can't hold").  moe_route_sort groups the (token, slot) pairs by expert;
 * moe_gmm multiplies each expert's group of rows by that expert's 4-bit
 * weights, which it decodes exactly to bf16 on chip as they stream in and
 * feeds to the bf16 matrix cores with f32 accumulation; moe_combine weighs
 * and sums each token's k results.  Weights are MXFP4 (e2m1 codes, one E8M0
 * power-of-two scale per 32 weights along K) or NVFP4 (e2m1 codes, one E4M3
 * scale per 16 weights along K, one f32 scale per expert); activations stay
 * bf16.
 *
 * Conventions for every call below:
 *  - Every data pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *    tensor's data_ptr()).  The caller owns every buffer; the library
 *    allocates nothing and keeps no state, so calls are reentrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously; results are valid after the caller
 *    synchronises that stream.  No call synchronises the device.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    non-zero moe_status_t is returned and nothing is launched.  A launch
 *    failure reported by the runtime returns MOE_ERR_HIP.
 *  - bf16 values are passed as uint16_t bit patterns; f32 as float.
 *  - Array shapes are row-major, written [d0, d1, ...].
 */
#ifndef MOE_GMM_H
#define MOE_GMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                      */
  MOE_ERR_SHAPE = 2,       /* a size is non-positive, too large or misaligned */
  MOE_ERR_FORMAT = 3,      /* unknown weight format or dtype enum             */
  MOE_ERR_UNSUPPORTED = 4, /* valid request this build does not implement     */
  MOE_ERR_HIP = 5          /* the HIP runtime reported a launch error         */
} moe_status_t;

typedef enum {
  MOE_W_MXFP4 = 0,  /* e2m1 codes, E8M0 scale per 32 along K                  */
  MOE_W_NVFP4 = 1,  /* e2m1 codes, E4M3 scale per 16 along K, f32 per expert  */
  MOE_W_BF16 = 2    /* bf16 weights: the comparison arm (moe_bf16_encode)     */
} moe_wfmt_t;
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Epilogue of moe_gmm_act. */
typedef enum {
  MOE_ACT_NONE = 0,     /* y = the [M, N] matmul output                        */
  MOE_ACT_SILU_MUL = 1  /* y = [M, N/2] silu(out[:, :N/2]) * out[:, N/2:]      */
} moe_act_t;

/* Kernel configuration of moe_gmm_ex.  AUTO picks from the problem shape. */
typedef enum {
  MOE_GMM_AUTO = 0,
  MOE_GMM_STREAM = 1,  /* weight-streaming waves, no LDS: few rows per expert  */
  MOE_GMM_TILED = 2    /* LDS-staged activation tiles: many rows per expert    */
} moe_gmm_kernel_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/*
 * moe_route_sort_workspace_bytes - bytes of device workspace moe_route_sort
 * needs for T tokens of k slots over E experts: 0 when the pairs are sorted
 * by one workgroup (T*k <= 4096), else 4 * E * G, with G = ceil(T*k / S)
 * segments of S = max(1024, ceil(T*k / 64) rounded up to 512) pairs
 * (G <= 64, so at most 256 KiB).  Also 0 for sizes moe_route_sort rejects.
 */
size_t moe_route_sort_workspace_bytes(int32_t T, int32_t k, int32_t E);

/*
 * moe_route_sort - counting sort of token-expert pairs into expert bands.
 *
 * Source: "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that
 * v6e can't hold": the activations are ordered by expert into one band of
 * rows each, and the grouped matmul walks the band sizes.  Inside a band,
 * pairs keep ascending flat pair order p = t*k + j (stable), so the result is
 * unique and deterministic; positions are decided by counts and scans, never
 * by atomics.
 *
 * topk_ids       [T, k] int32  expert of slot j of token t.
 * group_offsets  [E+1]  int32  out: band e is rows [off[e], off[e+1]).
 * sorted_token   [T*k]  int32  out: token of each band row; -1 past off[E].
 * sorted_pair    [T*k]  int32  out: pair p of each band row; -1 past off[E].
 * pair_row       [T*k]  int32  out: band row of pair p; -1 if dropped.
 * err_count      [1]    int32  out, may be NULL: number of pairs whose id is
 *                              outside [0, E); they are dropped from every
 *                              band (the device-side data error).
 * ws, ws_bytes   caller-owned device workspace of at least
 *                moe_route_sort_workspace_bytes(T, k, E) bytes, 4-byte
 *                aligned; it holds the per-segment expert counts between
 *                the count and place kernels, needs no clearing and may be
 *                reused once the stream has passed this call.  May be NULL
 *                when that size is 0.
 * Errors: NULL ws with a non-zero need -> MOE_ERR_NULL; ws_bytes below the
 * need or ws misaligned -> MOE_ERR_SHAPE.
 * Limits: 1 <= T, 1 <= k, 1 <= E <= 1024, T*k <= 2^24.
 */
int moe_route_sort(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                   int32_t* group_offsets, int32_t* sorted_token,
                   int32_t* sorted_pair, int32_t* pair_row, int32_t* err_count,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_sort_noalloc - moe_route_sort for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, results and errors as moe_route_sort without ws/ws_bytes.
 * The count table lives in a library-owned array of 256 KiB per GPU (the
 * largest moe_route_sort_workspace_bytes of any accepted size), resolved on
 * the first call on each device and held until the process ends; the call
 * allocates nothing.  It uses the array of the current device, which must be
 * the device of `stream`.  Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (on different streams, or from several
 * host threads without ordering) race on it and must be serialised by the
 * caller.  The table is written in full before it is read, so nothing needs
 * clearing between calls.  A size needing more than the array returns
 * MOE_ERR_SHAPE (none of the accepted sizes does); a failure to resolve the
 * array returns MOE_ERR_HIP.
 */
int moe_route_sort_noalloc(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                           int32_t* group_offsets, int32_t* sorted_token,
                           int32_t* sorted_pair, int32_t* pair_row, int32_t* err_count,
                           void* stream);

/*
 * moe_packed_weight_bytes - size in bytes of the packed buffer that
 * mxfp4_encode writes for E experts of an [N, K] weight (0 on bad sizes).
 * Codes stay 4 bits per weight; scales stay one byte per block (padded to
 * whole 256-byte groups), plus, for NVFP4, 4*E bytes of tensor scales and a
 * 4-byte flag per 16 columns of each expert (whether all of their E4M3
 * scales are powers of two), each part padded to 256 bytes.
 */
size_t moe_packed_weight_bytes(int fmt, int32_t E, int32_t N, int32_t K);

/*
 * mxfp4_encode - load-time repack of canonical expert weights into the
 * packed layout moe_gmm streams.
 *
 * Source: "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that
 * v6e can't hold": the expert weights are re-laid-out once when the model
 * loads and stay 4 bits per weight in HBM; the grouped matmul streams them in
 * BK x BN tiles.  On gfx950 the e2m1 codes are decoded natively, so the
 * repack is a pure permutation of 16-byte code runs and scale bytes (the
 * pages' signed re-encoding was needed only by hardware without 4-bit
 * vectors).
 *
 * fmt            MOE_W_MXFP4 or MOE_W_NVFP4.
 * codes          [E, N, K/2] uint8: two e2m1 codes per byte, the even K index
 *                in the low nibble (bit 3 of a code = sign).
 * scales         MXFP4: [E, N, K/32] E8M0 bytes (2^(b-127));
 *                NVFP4: [E, N, K/16] E4M3FN bytes.
 * tensor_scale   NVFP4: [E] float, the per-expert scale; MXFP4: must be NULL.
 * packed         out, moe_packed_weight_bytes(fmt, E, N, K) bytes, 256-aligned.
 * err_count      out [1] int32, may be NULL: the number of scale values
 *                outside the exact-decode domain (the scale sanity sweep of
 *                "DeepSeek-V4-Flash-0731-NVFP4", section "Verification"):
 *                MXFP4 E8M0 bytes other than 2..252 (0 and 1 are below the
 *                bf16-normal range of the decode, 253 and 254 overflow bf16
 *                for the larger codes, 255 is NaN), NVFP4 E4M3 NaN bytes
 *                (0x7F, 0xFF) and non-finite tensor scales.  Such values are
 *                packed as given; the weights they scale do not decode to the
 *                format's values, so every output they feed is unspecified.
 *                A zero count means every packed weight decodes exactly.
 * Limits: K % 128 == 0, K <= 33,553,408 (a wave's code range of eight
 * 16-column subtiles stays below 2^31 - 64 KiB), N % 64 == 0, E >= 1,
 * E*N*K/2 < 2^40.
 */
int mxfp4_encode(int fmt, const uint8_t* codes, const uint8_t* scales,
                 const float* tensor_scale, int32_t E, int32_t N, int32_t K,
                 void* packed, int32_t* err_count, void* stream);

/*
 * moe_bf16_encode - load-time repack of bf16 expert weights for the bf16
 * comparison arm.
 *
 * Source: "Running DeepSeek V4 Flash on TPU v6", section "Grouped matmul
 * performance vs bf16": the MXFP4 grouped matmul is measured against the same
 * grouped matmul with bf16 weights.  The packed layout has the chunks and the
 * K assignment of the 4-bit layout, each 16-bit weight in place of its code,
 * so moe_gmm with fmt MOE_W_BF16 on the decoded weights of an MXFP4 matrix
 * issues the same MFMAs on the same operands and returns the same bits.
 *
 * weights   [E, N, K] bf16 bit patterns, K contiguous, 16-byte aligned.
 * packed    out, moe_packed_weight_bytes(MOE_W_BF16, E, N, K) = E*N*K*2
 *           bytes, 256-aligned.
 * Limits as mxfp4_encode, and K <= 16,776,704.  (mxfp4_encode rejects MOE_W_BF16
 * with MOE_ERR_FORMAT.)
 */
int moe_bf16_encode(const uint16_t* weights, int32_t E, int32_t N, int32_t K, void* packed,
                    void* stream);

/*
 * moe_gmm - routed-expert grouped matmul, W4A16 on bf16 MFMA.
 *
 * Source: "Running DeepSeek V4 Flash on TPU v6", section "1. Four bits that
 * v6e can't hold" (the loop nest over N tiles and (expert, M-tile) pairs, K
 * walked with the weight tile decoded to bf16 then block-scaled, f32
 * accumulation on the bf16 matrix unit, ragged and empty groups) and section
 * "Grouped matmul performance vs bf16" (the NVFP4 variant with per-16 E4M3
 * block scales).
 *
 * For every row r of band e:  y[r, n] = sum_k x[src(r), k] * W_e[n, k]
 * with W_e[n, k] = e2m1(code) * blockscale (* tensor_scale[e] for NVFP4),
 * each decoded weight exact in bf16, products exact, sums in f32.
 *
 * packed         mxfp4_encode output for (fmt, E, N, K).
 * x              bf16 [x_rows, K]: the token rows when row_index != NULL
 *                (band row r reads x[row_index[r]]), else the band-ordered
 *                rows (x_rows >= M).
 * row_index      [M] int32 (moe_route_sort's sorted_token) or NULL.
 * group_offsets  [E+1] int32 device array from moe_route_sort.
 * M              rows of y (T*k).  Rows [group_offsets[E], M) are not written.
 * y              out [M, N], f32 or bf16 (round-to-nearest-even of the f32 sum).
 * Preconditions not checked: row_index values lie in [0, x_rows); group_offsets
 * is non-decreasing with group_offsets[0] = 0 and group_offsets[E] <= M.
 * Exact-decode domain: MXFP4 scale bytes 2..252 (block exponent -125..125).
 * Limits as mxfp4_encode; E <= 1024; M <= 2^24; K <= 33,553,408 and
 * x_rows * K * 2 <= 2^31 - 64 KiB bytes (every buffer range a kernel builds
 * stays below the lane offset its bounded loads use to read zeros).  The
 * grid, an upper bound on the row tiles times the column groups, stays within
 * the 2^32 - 1 work-items a dispatch counts (16,777,215 workgroups): about
 * (M/32 + min(E, M)) * N/256 workgroups for the streaming kernel (N/128 with
 * bf16 weights or the fused activation) and (M/128 + min(E, M)) * N/256 for
 * the tiled one; larger grids return MOE_ERR_SHAPE.
 */
int moe_gmm(const void* packed, int fmt, int32_t E, int32_t N, int32_t K,
            const uint16_t* x, int32_t x_rows, const int32_t* row_index,
            const int32_t* group_offsets, int32_t M, void* y, int y_dtype,
            void* stream);

/* moe_gmm_ex - moe_gmm with an explicit kernel configuration
 * (moe_gmm_kernel_t).  AUTO takes the LDS-tiled kernel when M >= 24 * E (a
 * mean band of 24 rows or more) and the weight-streaming one otherwise.  With
 * MXFP4 weights, no fused activation and M >= 4 * E, the streaming choice
 * runs bands of more than 64 rows as LDS-tiled units inside the same launch.
 * Every configuration computes the same sums in the same order, so all of
 * them return bitwise identical y; this holds for MOE_W_BF16 weights too. */
int moe_gmm_ex(const void* packed, int fmt, int32_t E, int32_t N, int32_t K,
               const uint16_t* x, int32_t x_rows, const int32_t* row_index,
               const int32_t* group_offsets, int32_t M, void* y, int y_dtype,
               int kernel, void* stream);

/*
 * moe_gmm_act - moe_gmm_ex with the gate/up activation fused into the
 * epilogue.
 *
 * Source: "Running DeepSeek V4 Flash on TPU v6", section "Grouped matmul
 * performance vs bf16", names the gate/up activation that follows the fused
 * gate+up (w13) matmul; the "DeepSeek-V4-Flash-0731-NVFP4" model card,
 * section "The lossless weight cast", calls that matmul the fused w1/w3
 * GEMM1.  Neither page writes the activation out; this library takes the
 * SiLU-gated product of the two column halves (gate = w1 = the first N/2
 * weight rows, up = w3 = the last N/2).
 *
 * act = MOE_ACT_NONE: exactly moe_gmm_ex.
 * act = MOE_ACT_SILU_MUL: y is [M, N/2] (f32 or bf16, row stride N/2) with
 *   y[r, j] = silu(g) * u,  g = out[r, j],  u = out[r, N/2 + j],
 *   silu(g) = g / (1 + e^-g), out the f32 matmul sums of moe_gmm (times the
 *   NVFP4 tensor scale), evaluated in f32; the [M, N] sums are never written.
 *   Requires N % 128 == 0 and (N/32 + 2) * (K/128) KiB <= 2^31 - 64 KiB.
 * Every kernel configuration returns bitwise identical y.  Other arguments,
 * limits and errors as moe_gmm; an unknown act returns MOE_ERR_FORMAT, and
 * MOE_ACT_SILU_MUL with MOE_W_BF16 weights MOE_ERR_UNSUPPORTED.
 */
int moe_gmm_act(const void* packed, int fmt, int32_t E, int32_t N, int32_t K,
                const uint16_t* x, int32_t x_rows, const int32_t* row_index,
                const int32_t* group_offsets, int32_t M, void* y, int y_dtype,
                int act, int kernel, void* stream);

/*
 * moe_mxfp4_quantize - MXFP4 quantization of bf16 activation rows, for the
 * W4A4 variant.
 *
 * Source: "DeepSeek-V4-Flash-0731-NVFP4" (model card) runs the routed experts
 * W4A4 (its table row for the routed experts and its "Performance"
 * discussion: activations quantized to 4-bit floats too).  That card uses
 * NVFP4 with calibrated per-tensor scales; gfx950's scaled matrix
 * instructions take power-of-two block scales, so this library quantizes to
 * MXFP4: for each block of 32 consecutive K values of a row,
 *   X = floor(log2(max |v|)) - 2, scale byte = X + 127 clamped to [0, 254]
 *   (an all-zero block: byte 0), code = the e2m1 value nearest to v / 2^X
 *   (a tie to the even mantissa bit, magnitudes past 6 to 6), sign kept.
 *
 * x        bf16 [R, K], K contiguous, 16-byte aligned; finite values.
 * codes    out [R, K/2] uint8, the even K index in the low nibble, 16-byte aligned.
 * scales   out [R, K/32] uint8 E8M0.
 * Limits: K % 32 == 0, R * K < 2^40.
 */
int moe_mxfp4_quantize(const uint16_t* x, int32_t R, int32_t K, uint8_t* codes, uint8_t* scales,
                       void* stream);

/*
 * moe_gmm_w4a4 - the grouped matmul with 4-bit weights and MXFP4-quantized
 * activations, on the scaled FP4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
 *
 * Source: the grouped matmul of moe_gmm ("Running DeepSeek V4 Flash on TPU
 * v6", section "1. Four bits that v6e can't hold") with the W4A4 execution of
 * "DeepSeek-V4-Flash-0731-NVFP4" (sections "What was quantized" and
 * "Performance"), whose NVFP4 weights come from MXFP4 by the scale mapping of
 * its section "The lossless weight cast".
 *
 * For every row r of band e:  y[r, n] = sum_k A[src(r), k] * W_e[n, k] with
 * A = e2m1(code) * 2^(scale - 127) of the quantized activations; the products
 * are exact, the sums f32 (the matrix unit adds each 128-deep chunk, then
 * the running sum).  act as moe_gmm_act.
 *
 * packed         mxfp4_encode output for (fmt, E, N, K).
 * fmt            MOE_W_MXFP4, or MOE_W_NVFP4 whose two E4M3 scales of every
 *                32-weight block are one equal power of two (2^-9 .. 2^8; true
 *                of every pack made by moe_mxfp4_to_nvfp4): that scale is
 *                given to the instruction as the block's E8M0 byte and the
 *                per-expert tensor scale multiplies the f32 sums, so the
 *                output equals, bit for bit, that of the MXFP4 weights the
 *                cast came from.  MOE_W_BF16 returns MOE_ERR_UNSUPPORTED.
 * xq_codes       [x_rows, K/2] from moe_mxfp4_quantize, 16-byte aligned.
 * xq_scales      [x_rows, K/32].
 * err_count      out [1] int32, may be NULL: with NVFP4 weights, the number
 *                of (expert, column, 32-block) weight blocks this call used
 *                whose scales do not qualify (whether they do is known only
 *                on the device); outputs that read such a block are
 *                unspecified.  Always 0 for MXFP4.
 * Other arguments, limits and errors as moe_gmm_act, with
 * x_rows * K/2 <= 2^31 - 64 KiB and the tiled kernel's grid.  LDS-tiled
 * kernel (meant for prefill bands).
 */
int moe_gmm_w4a4(const void* packed, int fmt, int32_t E, int32_t N, int32_t K, const uint8_t* xq_codes,
                 const uint8_t* xq_scales, int32_t x_rows, const int32_t* row_index,
                 const int32_t* group_offsets, int32_t M, void* y, int y_dtype, int act,
                 int32_t* err_count, void* stream);

/*
 * moe_combine - top-k weighted unpermute back to token order.
 *
 * Source: the band layout of "Running DeepSeek V4 Flash on TPU v6", section
 * "1. Four bits that v6e can't hold", and the deterministic expert reduction
 * of "DeepSeek-V4-Flash" (PocketLLM docs), section "Correctness and
 * precision": out[t, n] = sum over j = 0..k-1, in that order, of
 * topk_weights[t, j] * y[pair_row[t*k + j], n], accumulated in f32 with
 * fused multiply-adds; no atomics.  pair_row < 0 contributes nothing.
 *
 * y              [rows, N] f32 or bf16 (y_dtype), rows >= every pair_row + 1.
 * topk_weights   [T, k] float.
 * pair_row       [T*k] int32 (moe_route_sort output).
 * out            [T, N] f32 or bf16 (out_dtype; bf16 = RNE of the f32 sum).
 * Limits: N % 4 == 0, 1 <= k <= 64, T*k <= 2^24, T*N < 2^40.
 */
int moe_combine(const void* y, int y_dtype, const float* topk_weights,
                const int32_t* pair_row, int32_t T, int32_t k, int32_t N,
                void* out, int out_dtype, void* stream);

/*
 * moe_mxfp4_to_nvfp4 - the lossless MXFP4 -> NVFP4 scale cast.
 *
 * Source: "DeepSeek-V4-Flash-0731-NVFP4", section "The lossless weight cast":
 * per expert, with k_j the unbiased exponent of block j and k_max their
 * maximum, the tensor scale is 2^(k_max - 8) and both 16-halves of block j
 * get the E4M3 scale 2^(k_j - k_max + 8); codes are unchanged.
 *
 * scales         [E, N, K/32] E8M0 bytes of one expert tensor per expert.
 * block_scales   out [E, N, K/16] E4M3FN bytes.
 * tensor_scale   out [E] float (a subnormal f32 when k_max < -118; exact).
 * err_count      out [1] int32, may be NULL: blocks that cannot be held
 *                exactly (k_j < k_max - 17, or a NaN byte 0xFF); such a
 *                block's bytes are written as 0.
 * Limits: K % 32 == 0, N >= 1, E >= 1.
 */
int moe_mxfp4_to_nvfp4(const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                       uint8_t* block_scales, float* tensor_scale,
                       int32_t* err_count, void* stream);

/*
 * moe_debug_decode - decode a packed buffer back to dense bf16 weights
 * [E, N, K] (test support).  Same decode as moe_gmm: e2m1 x block scale,
 * exact in bf16; NVFP4 output excludes the per-expert tensor scale.
 */
int moe_debug_decode(const void* packed, int fmt, int32_t E, int32_t N,
                     int32_t K, uint16_t* w_bf16, void* stream);

/*
 * moe_calib_mfma_bf16 - measurement support: the bf16 matrix-unit rate this
 * part sustains with no memory traffic.  The published dense bf16 peak
 * assumes the full shader clock on every cycle; this loop measures what the
 * matrix cores hold under the part's power limit, for reading the tiled
 * grouped matmul's MFMA-bound fraction against.
 *
 * a    [blocks*256*8] 16-byte A fragments (8 bf16 each), lane-major: lane g
 *      of the grid holds a[8g .. 8g+7].
 * b    [blocks*256*4] 16-byte B fragments, b[4g .. 4g+3] for lane g.
 * out  [blocks*256] f32, out: a sum of each lane's accumulators.
 * Each wave keeps its fragments in registers and issues iters * 128
 * v_mfma_f32_16x16x32_bf16 over a 128 x 64 accumulator tile (the tiled
 * kernel's wave tile), rotating the fragments so that every instruction's
 * operands differ from the previous one's.  FLOPs per call:
 * blocks * 4 waves * iters * 128 * 16384.
 * Limits: 1 <= blocks <= 65535, 1 <= iters <= 2^20; a and b 16-byte aligned.
 */
int moe_calib_mfma_bf16(const uint16_t* a, const uint16_t* b, int32_t blocks,
                        int32_t iters, float* out, void* stream);

/*
 * moe_calib_mfma_parts - measurement support: the bf16 matrix-unit rate of
 * the tiled grouped matmul's wave tile (rows16 row subtiles, 6 or 8, x 4
 * column subtiles of v_mfma_f32_16x16x32_bf16; 128-deep chunks of 4 steps)
 * with chosen parts of that kernel's data movement beside it, so that the
 * rate each part costs can be read off one at a time.  parts is one of:
 *   0                          operands in registers only;
 *   MOE_PARTS_LDS_A            A fragments read from LDS (one 1 KiB read per
 *                              wave, row subtile and step);
 *   MOE_PARTS_CODES            B decoded (scaled e2m1 convert) from codes
 *                              streamed from HBM, 4 KiB per wave and chunk,
 *                              one chunk ahead;
 *   MOE_PARTS_STAGE            an 8 KiB activation chunk per wave copied
 *                              into LDS by direct-to-LDS loads, then a wait
 *                              for all loads and a workgroup barrier;
 *   MOE_PARTS_BARRIER          a workgroup barrier per chunk only;
 *   MOE_PARTS_REG_DECODE       B decoded from register-held codes that change
 *                              every chunk;
 *   MOE_PARTS_CODES_XOR        the code stream, only XOR-ed into a register;
 *   MOE_PARTS_LDS_A | MOE_PARTS_CODES | MOE_PARTS_STAGE   all of the kernel's.
 *
 * a      [blocks*256*8] 16-byte A fragments (8 bf16), lane-major as in
 *        moe_calib_mfma_bf16; the first 4096 fragments from workgroup g's
 *        start also fill its LDS.
 * b      [blocks*256*4] 16-byte B fragments (used when B is not decoded).
 * codes  [codes_bytes] e2m1 codes, cut into blocks*4 equal regions (one per
 *        wave, a multiple of 4 KiB, at least 4 KiB); a wave reads its region
 *        as four streams that wrap.  Make it larger than the 256 MiB
 *        last-level cache for HBM reads.
 * x      [x_bytes] staging source, a multiple of 1 KiB; the copies wrap at
 *        x_bytes (1 MiB stays in L2, 32 MiB does not).
 * scale  decode scale; only its exponent is applied (a power of two is exact).
 * out    [blocks*256] f32: each lane's sum of its accumulators (+1 if the
 *        XOR of the codes it read is odd, MOE_PARTS_CODES_XOR only).
 * FLOPs per call: blocks * 4 * chunks * 4 * rows16 * 4 * 16384.  Limits:
 * 1 <= blocks <= 65535, 2 <= chunks <= 2^24 and even, a wave region below
 * 2^31 bytes, 8 KiB <= x_bytes < 2^31; every pointer 16-byte aligned (out 4).
 * An unsupported parts value or rows16 returns MOE_ERR_SHAPE.
 */
#define MOE_PARTS_LDS_A 1
#define MOE_PARTS_CODES 2
#define MOE_PARTS_STAGE 4
#define MOE_PARTS_BARRIER 8
#define MOE_PARTS_REG_DECODE 16
#define MOE_PARTS_CODES_XOR 32
int moe_calib_mfma_parts(int32_t parts, int32_t rows16, const uint16_t* a, const uint16_t* b,
                         const void* codes, size_t codes_bytes, const uint16_t* x, size_t x_bytes,
                         float scale, int32_t blocks, int32_t chunks, float* out, void* stream);

/*
 * moe_calib_hbm_read - measurement support: the HBM read rate this part
 * sustains with the weight-streaming kernel's access pattern (each wave walks
 * its own contiguous region of src in 1 KiB runs, one 16-byte non-temporal
 * buffer load per lane, eight runs in flight), for reading the decode
 * kernels' HBM-bound fraction against.
 *
 * src    [bytes] device buffer, 16-byte aligned; bytes a multiple of 16.
 *        Make it larger than the 256 MiB last-level cache (the bench uses
 *        2 GiB) so the reads come from HBM.
 * out    [blocks * 256] uint32, out: each thread's XOR of the 32-bit words it
 *        read; the XOR over all of out equals the XOR of every 32-bit word
 *        of src.
 * Bytes per call: bytes.  Limits: 1 <= blocks <= 65535, and at most 2^22
 * runs of 1 KiB per wave (bytes < blocks * 2^34).
 */
int moe_calib_hbm_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GMM_H */
