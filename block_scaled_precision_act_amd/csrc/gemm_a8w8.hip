// gemm_a8w8.hip - PTPC FP8 A8W8 GEMM entry (E4M3 operands with per-token and
// per-output-channel FP32 scales: "Kimi-K3-DSpark-FP8-PTPC", section "Phase 1
// FP8 PTPC Quantization").  Same kernels as the A4W4 path, FP8 operands, unit
// MFMA scales and the two FP32 scales applied in the epilogue.
#include "gemm_kernels.hpp"
#include "launch.hpp"

namespace mx {

hipError_t launch_gemm_a8w8(const void* qa, const float* sa, const void* qw, const float* sw, void* y, int64_t M,
                            int64_t N, int64_t K, hipStream_t st) {
    return launch_gemm<true>(qa, sa, qw, sw, y, M, N, K, st);
}

}  // namespace mx
