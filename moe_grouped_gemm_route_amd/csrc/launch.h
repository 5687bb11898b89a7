// Internal launchers behind the C ABI.  Arguments are validated by api.cpp
// before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Route-sort plan for M pairs: G segments of S pairs, one workgroup each.
// Small M: one workgroup, no workspace (fused); else a count kernel and a
// place kernel with a [G][E] int32 count table in the workspace.
struct RoutePlan {
  int fused;
  int S, G;
  size_t ws_bytes;
};
RoutePlan route_plan(int64_t M, int32_t E);

// Device address and size of the current device's route-sort count table
// (the no-allocation entry point's scratch array).
hipError_t route_sort_scratch(int32_t** ptr, size_t* bytes);

hipError_t launch_route_sort(const int32_t* ids, int32_t T, int32_t k, int32_t E,
                             int32_t* group_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                             int32_t* pair_row, int32_t* err_count, int32_t* ws, hipStream_t stream);

hipError_t launch_encode(int fmt, const uint8_t* codes, const uint8_t* scales,
                         const float* tensor_scale, int32_t E, int32_t N, int32_t K,
                         uint8_t* packed, int32_t* err_count, hipStream_t stream);

hipError_t launch_bf16_encode(const uint16_t* w, int32_t E, int32_t N, int32_t K, uint8_t* packed,
                              hipStream_t stream);

hipError_t launch_debug_decode(const uint8_t* packed, int fmt, int32_t E, int32_t N, int32_t K,
                               uint16_t* w, hipStream_t stream);

hipError_t launch_mxfp4_to_nvfp4(const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                                 uint8_t* block_scales, float* tensor_scale, int32_t* err_count,
                                 hipStream_t stream);

// kernel: 1 = weight-streaming waves, 2 = LDS-tiled activations.
// act: 0 = the [M, N] matmul output, 1 = the [M, N/2] SiLU-gated gate/up
// activation of it.
hipError_t launch_gmm(const uint8_t* packed, int fmt, int32_t E, int32_t N, int32_t K,
                      const uint16_t* x, int32_t x_rows, const int32_t* row_index,
                      const int32_t* group_offsets,
                      int32_t M, void* y, int y_bf16, int act, int kernel, hipStream_t stream);

// Workgroups that launch_gmm launches for these sizes (kernel 1 or 2; the
// W4A4 kernel's grid is kernel 2's).
int64_t gmm_workgroups(int fmt, int32_t E, int32_t N, int32_t M, int act, int kernel);

// W4A4: MXFP4 (fmt 0) or NVFP4 (fmt 1, power-of-two block scales) weights
// times MXFP4-quantized activations (codes [x_rows, K/2], E8M0 scales
// [x_rows, K/32]) on the scaled FP4 MFMA; err_count (may be NULL) receives the
// NVFP4 blocks whose scales do not qualify.
hipError_t launch_gmm_w4a4(const uint8_t* packed, int fmt, int32_t E, int32_t N, int32_t K, const uint8_t* qcodes,
                           const uint8_t* qscales, int32_t x_rows, const int32_t* row_index,
                           const int32_t* group_offsets, int32_t M, void* y, int y_bf16, int act,
                           int32_t* err_count, hipStream_t stream);

// Sets n int32 to zero with a kernel (no memset node, so the call stays safe
// to record into a HIP graph).
void launch_zero_i32(int32_t* p, int n, hipStream_t stream);

hipError_t launch_quantize_mxfp4(const uint16_t* x, int32_t R, int32_t K, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);

// Matrix-unit calibration: blocks workgroups of 4 waves, each wave issuing
// iters * 128 bf16 MFMAs on register-resident fragments (a: 8, b: 4 per lane).
hipError_t launch_calib_mfma(const uint16_t* a, const uint16_t* b, int32_t blocks, int32_t iters, float* out,
                             hipStream_t stream);

// Matrix-unit build-up: the tiled kernel's wave tile (rows16 row subtiles,
// 6 or 8) with the data movement named by parts (a supported combination of
// the PARTS_* bits in calib.hip), chunks 128-deep chunks per wave.
bool calib_parts_supported(int32_t parts);
hipError_t launch_calib_parts(int32_t parts, int32_t rows16, const uint16_t* a, const uint16_t* b,
                              const void* codes, uint32_t region, const uint16_t* x, uint32_t x_blocks,
                              float scale, int32_t blocks, int32_t chunks, float* out, hipStream_t stream);

// HBM read calibration: blocks workgroups of 256 threads XOR-reduce the
// 16-byte words of src (bytes a multiple of 16) into out[blocks * 256].
hipError_t launch_calib_hbm_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out,
                                 hipStream_t stream);

hipError_t launch_combine(const void* y, int y_bf16, const float* w, const int32_t* pair_row,
                          int32_t T, int32_t k, int32_t N, void* out, int out_bf16,
                          hipStream_t stream);

}  // namespace moe
