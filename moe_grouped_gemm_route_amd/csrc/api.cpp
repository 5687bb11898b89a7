// C ABI of libmoegmm.so (declared in include/moe_gmm.h): host-side argument
// checks, kernel-configuration choice, and the launches.  Every check runs
// before the first HIP call, so a rejected call enqueues nothing.
#include "moe_gmm.h"

#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxRows = int64_t(1) << 24;
constexpr int64_t kMaxCodeBytes = int64_t(1) << 40;

bool fmt_ok(int fmt) { return fmt == MOE_W_MXFP4 || fmt == MOE_W_NVFP4 || fmt == MOE_W_BF16; }
bool dtype_ok(int d) { return d == MOE_F32 || d == MOE_BF16; }

// Weight sizes the packed layout and the kernels support.
int check_weight_shape(int fmt, int32_t E, int32_t N, int32_t K) {
  if (!fmt_ok(fmt)) return MOE_ERR_FORMAT;
  if (E < 1 || N < 1 || K < 1) return MOE_ERR_SHAPE;
  if (K % 128 != 0 || N % 64 != 0) return MOE_ERR_SHAPE;
  if ((int64_t)E * N * (K / 2) >= kMaxCodeBytes) return MOE_ERR_SHAPE;
  // a wave's code range (up to eight 16-column subtiles of 1 KiB per chunk)
  // stays below the lane offset that reads zeros
  if ((int64_t)8 * (K / 128) * 1024 > (int64_t)moe::kLaneOob) return MOE_ERR_SHAPE;
  // bf16 weights: a wave's (up to four) 4 KiB-per-chunk subtiles likewise
  if (fmt == MOE_W_BF16 && (int64_t)4 * (K / 128) * 4096 > (int64_t)moe::kLaneOob) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// The matmul kernels find their tiles from the band offsets with 64 lanes
// of at most 16 experts each.
constexpr int32_t kMaxGmmExperts = 1024;
// A dispatch packet counts the work-items of each grid dimension in 32 bits:
// at 256 work-items per workgroup, at most this many workgroups.
constexpr int64_t kMaxWorkgroups = 0xFFFFFFFFll / 256;

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Route-sort sizes: ids fit the 10 id bits the placement ballots, and every
// pair and row index fits int32.
int route_sort_shape(int32_t T, int32_t k, int32_t E) {
  if (T < 1 || k < 1 || E < 1 || E > 1024) return MOE_ERR_SHAPE;
  if ((int64_t)T * k > kMaxRows) return MOE_ERR_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case MOE_ERR_FORMAT: return "unknown weight format or dtype";
    case MOE_ERR_UNSUPPORTED: return "not supported by this build";
    case MOE_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

size_t moe_route_sort_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (route_sort_shape(T, k, E) != MOE_OK) return 0;
  return moe::route_plan((int64_t)T * k, E).ws_bytes;
}

int moe_route_sort(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                   int32_t* group_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                   int32_t* pair_row, int32_t* err_count, void* ws, size_t ws_bytes, void* stream) {
  if (!topk_ids || !group_offsets || !sorted_token || !sorted_pair || !pair_row) return MOE_ERR_NULL;
  const int st = route_sort_shape(T, k, E);
  if (st != MOE_OK) return st;
  const size_t need = moe::route_plan((int64_t)T * k, E).ws_bytes;
  if (need > 0) {
    if (!ws) return MOE_ERR_NULL;
    if (ws_bytes < need || ((uintptr_t)ws & 3)) return MOE_ERR_SHAPE;
  }
  return hip_status(moe::launch_route_sort(topk_ids, T, k, E, group_offsets, sorted_token,
                                           sorted_pair, pair_row, err_count, static_cast<int32_t*>(ws),
                                           static_cast<hipStream_t>(stream)));
}

int moe_route_sort_noalloc(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                           int32_t* group_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                           int32_t* pair_row, int32_t* err_count, void* stream) {
  if (!topk_ids || !group_offsets || !sorted_token || !sorted_pair || !pair_row) return MOE_ERR_NULL;
  const int st = route_sort_shape(T, k, E);
  if (st != MOE_OK) return st;
  const size_t need = moe::route_plan((int64_t)T * k, E).ws_bytes;
  int32_t* ws = nullptr;
  if (need > 0) {
    size_t have = 0;
    if (moe::route_sort_scratch(&ws, &have) != hipSuccess) return MOE_ERR_HIP;
    if (need > have) return MOE_ERR_SHAPE;
  }
  return hip_status(moe::launch_route_sort(topk_ids, T, k, E, group_offsets, sorted_token,
                                           sorted_pair, pair_row, err_count, ws,
                                           static_cast<hipStream_t>(stream)));
}

size_t moe_packed_weight_bytes(int fmt, int32_t E, int32_t N, int32_t K) {
  if (check_weight_shape(fmt, E, N, K) != MOE_OK) return 0;
  return (size_t)moe::make_layout(fmt, E, N, K).total_bytes;
}

int mxfp4_encode(int fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                 int32_t E, int32_t N, int32_t K, void* packed, int32_t* err_count, void* stream) {
  const int st = check_weight_shape(fmt, E, N, K);
  if (st != MOE_OK) return st;
  if (!codes || !scales || !packed) return MOE_ERR_NULL;
  if (fmt == MOE_W_BF16) return MOE_ERR_FORMAT;          /* moe_bf16_encode packs those */
  if (fmt == MOE_W_NVFP4 && !tensor_scale) return MOE_ERR_NULL;
  if (fmt == MOE_W_MXFP4 && tensor_scale) return MOE_ERR_FORMAT;
  if (((uintptr_t)codes & 15) || ((uintptr_t)packed & 255)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_encode(fmt, codes, scales, tensor_scale, E, N, K,
                                       static_cast<uint8_t*>(packed), err_count,
                                       static_cast<hipStream_t>(stream)));
}

int moe_bf16_encode(const uint16_t* weights, int32_t E, int32_t N, int32_t K, void* packed,
                    void* stream) {
  const int st = check_weight_shape(MOE_W_BF16, E, N, K);
  if (st != MOE_OK) return st;
  if (!weights || !packed) return MOE_ERR_NULL;
  if (((uintptr_t)weights & 15) || ((uintptr_t)packed & 255)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_bf16_encode(weights, E, N, K, static_cast<uint8_t*>(packed),
                                            static_cast<hipStream_t>(stream)));
}

int moe_gmm_act(const void* packed, int fmt, int32_t E, int32_t N, int32_t K, const uint16_t* x,
                int32_t x_rows, const int32_t* row_index, const int32_t* group_offsets, int32_t M, void* y,
                int y_dtype, int act, int kernel, void* stream) {
  const int st = check_weight_shape(fmt, E, N, K);
  if (st != MOE_OK) return st;
  if (E > kMaxGmmExperts) return MOE_ERR_SHAPE;
  if (!dtype_ok(y_dtype)) return MOE_ERR_FORMAT;
  if (kernel < MOE_GMM_AUTO || kernel > MOE_GMM_TILED) return MOE_ERR_FORMAT;
  if (act != MOE_ACT_NONE && act != MOE_ACT_SILU_MUL) return MOE_ERR_FORMAT;
  if (!packed || !x || !group_offsets || !y) return MOE_ERR_NULL;
  if (M < 1 || M > kMaxRows) return MOE_ERR_SHAPE;
  if (x_rows < 1 || x_rows > kMaxRows || (!row_index && x_rows < M)) return MOE_ERR_SHAPE;
  // activation rows are addressed with 32-bit byte offsets, below the lane
  // offset that reads zeros
  if ((int64_t)x_rows * K * 2 > (int64_t)moe::kLaneOob) return MOE_ERR_SHAPE;
  if (((uintptr_t)packed & 255) || ((uintptr_t)x & 15)) return MOE_ERR_SHAPE;
  // the bf16 comparison arm has no fused activation
  if (fmt == MOE_W_BF16 && act != MOE_ACT_NONE) return MOE_ERR_UNSUPPORTED;
  if (act == MOE_ACT_SILU_MUL) {
    // gate and up halves of 64-column multiples; one wave's code range spans
    // both halves of an expert and stays below the lane offset that reads zeros
    if (N % 128 != 0) return MOE_ERR_SHAPE;
    if ((int64_t)(N / 32 + 2) * (K / 128) * 1024 > (int64_t)moe::kLaneOob) return MOE_ERR_SHAPE;
  }
  if (kernel == MOE_GMM_AUTO) {
    // Bands averaging 24 rows or more keep the matrix cores busy enough for
    // the LDS-tiled kernel; thinner bands are pure weight streaming.  (A
    // token sweep of the w13 and w2 shapes puts the crossover between a mean
    // band of 18 rows, where streaming is 5-8 % faster, and 24.)
    kernel = ((int64_t)M >= 24 * (int64_t)E) ? MOE_GMM_TILED : MOE_GMM_STREAM;
  }
  if (moe::gmm_workgroups(fmt, E, N, M, act, kernel) > kMaxWorkgroups) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_gmm(static_cast<const uint8_t*>(packed), fmt, E, N, K, x, x_rows,
                                    row_index, group_offsets, M, y, y_dtype == MOE_BF16, act, kernel,
                                    static_cast<hipStream_t>(stream)));
}

int moe_gmm_ex(const void* packed, int fmt, int32_t E, int32_t N, int32_t K, const uint16_t* x,
               int32_t x_rows, const int32_t* row_index, const int32_t* group_offsets, int32_t M, void* y,
               int y_dtype, int kernel, void* stream) {
  return moe_gmm_act(packed, fmt, E, N, K, x, x_rows, row_index, group_offsets, M, y, y_dtype,
                     MOE_ACT_NONE, kernel, stream);
}

int moe_mxfp4_quantize(const uint16_t* x, int32_t R, int32_t K, uint8_t* codes, uint8_t* scales,
                       void* stream) {
  if (!x || !codes || !scales) return MOE_ERR_NULL;
  if (R < 1 || K < 32 || K % 32 != 0 || (int64_t)R * K >= (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 15)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_quantize_mxfp4(x, R, K, codes, scales, static_cast<hipStream_t>(stream)));
}

int moe_gmm_w4a4(const void* packed, int fmt, int32_t E, int32_t N, int32_t K, const uint8_t* xq_codes,
                 const uint8_t* xq_scales, int32_t x_rows, const int32_t* row_index,
                 const int32_t* group_offsets, int32_t M, void* y, int y_dtype, int act, int32_t* err_count,
                 void* stream) {
  if (fmt == MOE_W_BF16) return MOE_ERR_UNSUPPORTED;
  const int st = check_weight_shape(fmt, E, N, K);
  if (st != MOE_OK) return st;
  if (E > kMaxGmmExperts) return MOE_ERR_SHAPE;
  if (!dtype_ok(y_dtype)) return MOE_ERR_FORMAT;
  if (act != MOE_ACT_NONE && act != MOE_ACT_SILU_MUL) return MOE_ERR_FORMAT;
  if (!packed || !xq_codes || !xq_scales || !group_offsets || !y) return MOE_ERR_NULL;
  if (M < 1 || M > kMaxRows) return MOE_ERR_SHAPE;
  if (x_rows < 1 || x_rows > kMaxRows || (!row_index && x_rows < M)) return MOE_ERR_SHAPE;
  // activation codes are addressed with 32-bit byte offsets, below the lane
  // offset that reads zeros
  if ((int64_t)x_rows * (K / 2) > (int64_t)moe::kLaneOob) return MOE_ERR_SHAPE;
  if (((uintptr_t)packed & 255) || ((uintptr_t)xq_codes & 15)) return MOE_ERR_SHAPE;
  if (act == MOE_ACT_SILU_MUL) {
    if (N % 128 != 0) return MOE_ERR_SHAPE;
    if ((int64_t)(N / 32 + 2) * (K / 128) * 1024 > (int64_t)moe::kLaneOob) return MOE_ERR_SHAPE;
  }
  if (moe::gmm_workgroups(fmt, E, N, M, act, MOE_GMM_TILED) > kMaxWorkgroups) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_gmm_w4a4(static_cast<const uint8_t*>(packed), fmt, E, N, K, xq_codes, xq_scales,
                                         x_rows, row_index, group_offsets, M, y, y_dtype == MOE_BF16, act,
                                         err_count, static_cast<hipStream_t>(stream)));
}

int moe_gmm(const void* packed, int fmt, int32_t E, int32_t N, int32_t K, const uint16_t* x,
            int32_t x_rows, const int32_t* row_index, const int32_t* group_offsets, int32_t M,
            void* y, int y_dtype, void* stream) {
  return moe_gmm_ex(packed, fmt, E, N, K, x, x_rows, row_index, group_offsets, M, y, y_dtype,
                    MOE_GMM_AUTO, stream);
}

int moe_combine(const void* y, int y_dtype, const float* topk_weights, const int32_t* pair_row,
                int32_t T, int32_t k, int32_t N, void* out, int out_dtype, void* stream) {
  if (!dtype_ok(y_dtype) || !dtype_ok(out_dtype)) return MOE_ERR_FORMAT;
  if (!y || !topk_weights || !pair_row || !out) return MOE_ERR_NULL;
  if (T < 1 || k < 1 || k > 64 || N < 4 || N % 4 != 0) return MOE_ERR_SHAPE;
  if ((int64_t)T * k > kMaxRows || (int64_t)T * N >= (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  if (((uintptr_t)y & 15) || ((uintptr_t)out & 15)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_combine(y, y_dtype == MOE_BF16, topk_weights, pair_row, T, k, N,
                                        out, out_dtype == MOE_BF16,
                                        static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_to_nvfp4(const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                       uint8_t* block_scales, float* tensor_scale, int32_t* err_count,
                       void* stream) {
  if (!scales || !block_scales || !tensor_scale) return MOE_ERR_NULL;
  if (E < 1 || N < 1 || K < 32 || K % 32 != 0) return MOE_ERR_SHAPE;
  if ((int64_t)N * (K / 32) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if ((uintptr_t)block_scales & 1) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_mxfp4_to_nvfp4(scales, E, N, K, block_scales, tensor_scale,
                                               err_count, static_cast<hipStream_t>(stream)));
}

int moe_debug_decode(const void* packed, int fmt, int32_t E, int32_t N, int32_t K,
                     uint16_t* w_bf16, void* stream) {
  const int st = check_weight_shape(fmt, E, N, K);
  if (st != MOE_OK) return st;
  if (!packed || !w_bf16) return MOE_ERR_NULL;
  if (((uintptr_t)packed & 255) || ((uintptr_t)w_bf16 & 1)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_debug_decode(static_cast<const uint8_t*>(packed), fmt, E, N, K,
                                             w_bf16, static_cast<hipStream_t>(stream)));
}

int moe_calib_mfma_bf16(const uint16_t* a, const uint16_t* b, int32_t blocks, int32_t iters, float* out,
                        void* stream) {
  if (!a || !b || !out) return MOE_ERR_NULL;
  if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 20)) return MOE_ERR_SHAPE;
  if (((uintptr_t)a & 15) || ((uintptr_t)b & 15) || ((uintptr_t)out & 3)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_calib_mfma(a, b, blocks, iters, out, static_cast<hipStream_t>(stream)));
}

int moe_calib_mfma_parts(int32_t parts, int32_t rows16, const uint16_t* a, const uint16_t* b,
                         const void* codes, size_t codes_bytes, const uint16_t* x, size_t x_bytes,
                         float scale, int32_t blocks, int32_t chunks, float* out, void* stream) {
  if (!a || !b || !codes || !x || !out) return MOE_ERR_NULL;
  if (!moe::calib_parts_supported(parts) || (rows16 != 6 && rows16 != 8)) return MOE_ERR_SHAPE;
  if (blocks < 1 || blocks > 65535 || chunks < 2 || chunks > (1 << 24) || chunks % 2 != 0) return MOE_ERR_SHAPE;
  const uint64_t region = (uint64_t)codes_bytes / ((uint64_t)blocks * 4) / 4096 * 4096;
  if (region < 4096 || region >= (1ull << 31)) return MOE_ERR_SHAPE;
  if (x_bytes < 8192 || x_bytes % 1024 != 0 || x_bytes >= (1ull << 31)) return MOE_ERR_SHAPE;
  if (((uintptr_t)a & 15) || ((uintptr_t)b & 15) || ((uintptr_t)codes & 15) || ((uintptr_t)x & 15) ||
      ((uintptr_t)out & 3))
    return MOE_ERR_SHAPE;
  return hip_status(moe::launch_calib_parts(parts, rows16, a, b, codes, (uint32_t)region, x,
                                            (uint32_t)(x_bytes / 1024), scale, blocks, chunks, out,
                                            static_cast<hipStream_t>(stream)));
}

int moe_calib_hbm_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out, void* stream) {
  if (!src || !out) return MOE_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > 65535) return MOE_ERR_SHAPE;
  // a wave's region of whole 1 KiB runs is addressed with 32-bit offsets
  if (bytes / 1024 / ((uint64_t)blocks * 4) >= (1u << 22)) return MOE_ERR_SHAPE;
  if (((uintptr_t)src & 15) || ((uintptr_t)out & 3)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_calib_hbm_read(src, bytes, blocks, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
