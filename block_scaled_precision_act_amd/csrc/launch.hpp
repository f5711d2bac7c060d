// launch.hpp - internal launchers behind the C ABI (argument checks live in api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// MXFP4 quantizer: rows x K values (K % 32 == 0) -> codes [rows, K/2], scales [rows, K/32].
hipError_t launch_quant_mx_bf16(const void* x, int64_t rows, int64_t K, void* q, void* s, hipStream_t st);
hipError_t launch_quant_mx_f32(const void* x, int64_t rows, int64_t K, void* q, void* s, hipStream_t st);

// PTPC FP8 quantizer: rows x K values (K % 8 == 0) -> E4M3 codes [rows, K], FP32 scales [rows].
hipError_t launch_quant_ptpc_bf16(const void* x, int64_t rows, int64_t K, void* q, float* s, hipStream_t st);
hipError_t launch_quant_ptpc_f32(const void* x, int64_t rows, int64_t K, void* q, float* s, hipStream_t st);

// GEMMs (K % 128 == 0, M, N > 0).
hipError_t launch_gemm_a4w4(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                            int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t st);
size_t gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K);
// The same GEMM with its workspace in a static per-device array of kGemmScratchBytes (no allocation):
// the largest workspace of any split-K plan (256 workgroups); the caller rejects shapes that need more.
constexpr size_t kGemmScratchBytes = (size_t)8 << 20;
hipError_t launch_gemm_a4w4_noalloc(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                                    int64_t M, int64_t N, int64_t K, hipStream_t st);
// A4W4 layer: BF16 X -> MXFP4 -> BF16 Y, in one launch for M <= 8 (quantization inside the split-K
// GEMM's workgroups), else the quantizer and the GEMM.
hipError_t launch_linear_a4w4(const void* x, const void* qw, const void* sw, void* y, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t st);
size_t linear_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Grouped A4W4 GEMM over MoE experts (decode-sized groups, see mx_gemm_a4w4_grouped_bf16).
hipError_t launch_a4w4_grouped(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                               const int32_t* offsets, int64_t G, int64_t max_rows, int64_t N, int64_t K,
                               hipStream_t st);
hipError_t launch_gemm_a8w8(const void* qa, const float* sa, const void* qw, const float* sw, void* y,
                            int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t st);
size_t gemm_a8w8_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Compute units of the current device (cached per device); 0 if the query fails.
int device_cus();

}  // namespace mx
