// gemm_a4w4.hip - MXFP4 A4W4 GEMM entry ("A4W4 dispatch" of "Kimi-K3 DSpark
// O-Proj-only MXFP4", section "Exact quantization coverage").  The kernels are
// in gemm_kernels.hpp; M <= 128 takes the decode path (K split over the waves
// of a workgroup), larger M the LDS-tiled path.
#include "gemm_kernels.hpp"
#include "launch.hpp"

namespace mx {

hipError_t launch_gemm_a4w4(const void* qa, const void* sa, const void* qw, const void* sw, void* y, int64_t M,
                            int64_t N, int64_t K, void* /*workspace: no kernel needs one*/, hipStream_t st) {
    return launch_gemm<false>(qa, sa, qw, sw, y, M, N, K, st);
}

hipError_t launch_a4w4_grouped(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                               const int32_t* offsets, int64_t G, int64_t max_rows, int64_t N, int64_t K,
                               hipStream_t st) {
    return launch_gemm_a4w4_grouped(qa, sa, qw, sw, y, offsets, G, max_rows, N, K, st);
}

// No kernel of the A4W4 path needs device scratch memory.
size_t gemm_a4w4_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

}  // namespace mx
