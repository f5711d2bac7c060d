// api.cpp - the C ABI of libmxgemm (see include/mxgemm.h): argument checks on
// the host, then one launcher per call.  Nothing here allocates, synchronizes
// or keeps per-call state; the only state is a per-device "is this a gfx950"
// cache filled on first use.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/mxgemm.h"
#include "launch.hpp"

#define MX_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kAbiVersion = 1;
constexpr int kMaxDevices = 64;
int g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mx_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MX_ERROR_DEVICE;
    if (dev < kMaxDevices && g_device_ok[dev] != 0) return g_device_ok[dev] == 1 ? MX_SUCCESS : MX_ERROR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MX_ERROR_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_device_ok[dev] = ok ? 1 : 2;
    return ok ? MX_SUCCESS : MX_ERROR_DEVICE;
}

mx_status launched(hipError_t e) { return e == hipSuccess ? MX_SUCCESS : MX_ERROR_LAUNCH; }

// rows >= 0, 0 < K <= 2^31-1, K % kmod == 0, rows * K fits comfortably in int64
mx_status check_rows(int64_t rows, int64_t K, int64_t kmod) {
    if (rows < 0) return MX_ERROR_INVALID_VALUE;
    if (K <= 0 || K > INT32_MAX || K % kmod != 0) return MX_ERROR_UNSUPPORTED_SHAPE;
    if (rows > (INT64_C(1) << 40) / K) return MX_ERROR_UNSUPPORTED_SHAPE;
    return MX_SUCCESS;
}

mx_status check_gemm(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0) return MX_ERROR_INVALID_VALUE;
    if (K <= 0 || K % 128 != 0 || K > INT32_MAX) return MX_ERROR_UNSUPPORTED_SHAPE;
    if (M > INT32_MAX || N > INT32_MAX) return MX_ERROR_UNSUPPORTED_SHAPE;
    // 256 x 256 output tiles must fit one 1-D grid
    if (((M + 255) / 256) * ((N + 255) / 256) > INT32_MAX) return MX_ERROR_UNSUPPORTED_SHAPE;
    if (M > (INT64_C(1) << 40) / K || N > (INT64_C(1) << 40) / K) return MX_ERROR_UNSUPPORTED_SHAPE;
    return MX_SUCCESS;
}

}  // namespace

MX_API int mx_abi_version(void) { return kAbiVersion; }

MX_API const char* mx_status_string(mx_status status) {
    switch (status) {
        case MX_SUCCESS: return "MX_SUCCESS";
        case MX_ERROR_INVALID_VALUE: return "MX_ERROR_INVALID_VALUE: null pointer or negative size";
        case MX_ERROR_UNSUPPORTED_SHAPE: return "MX_ERROR_UNSUPPORTED_SHAPE: K (or a size) outside the supported rules";
        case MX_ERROR_MISALIGNED: return "MX_ERROR_MISALIGNED: a pointer misses its required alignment";
        case MX_ERROR_WORKSPACE: return "MX_ERROR_WORKSPACE: workspace smaller than the size query";
        case MX_ERROR_LAUNCH: return "MX_ERROR_LAUNCH: kernel launch failed";
        case MX_ERROR_DEVICE: return "MX_ERROR_DEVICE: current device is not a gfx950 GPU";
    }
    return "MX_ERROR_UNKNOWN";
}

static mx_status quant_mx(bool f32, const void* x, int64_t rows, int64_t K, void* q, void* s, void* stream) {
    mx_status st = check_rows(rows, K, 32);
    if (st != MX_SUCCESS) return st;
    if (rows == 0) return MX_SUCCESS;
    if (!x || !q || !s) return MX_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || !aligned(q, 16)) return MX_ERROR_MISALIGNED;
    if ((st = check_device()) != MX_SUCCESS) return st;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    return launched(f32 ? mx::launch_quant_mx_f32(x, rows, K, q, s, hs) : mx::launch_quant_mx_bf16(x, rows, K, q, s, hs));
}

MX_API mx_status mx_quant_act_bf16(const void* x_bf16, int64_t M, int64_t K, void* q, void* s, void* stream) {
    return quant_mx(false, x_bf16, M, K, q, s, stream);
}

MX_API mx_status mx_quant_weight_f32(const float* w, int64_t N, int64_t K, void* q, void* s, void* stream) {
    return quant_mx(true, w, N, K, q, s, stream);
}

MX_API size_t mx_gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_gemm(M, N, K) != MX_SUCCESS || M == 0 || N == 0) return 0;
    return mx::gemm_a4w4_workspace_bytes(M, N, K);
}

MX_API mx_status mx_gemm_a4w4_bf16(const void* qa, const void* sa, const void* qw, const void* sw, void* y_bf16,
                                   int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    mx_status st = check_gemm(M, N, K);
    if (st != MX_SUCCESS) return st;
    if (M == 0 || N == 0) return MX_SUCCESS;
    if (!qa || !sa || !qw || !sw || !y_bf16) return MX_ERROR_INVALID_VALUE;
    const size_t need = mx_gemm_a4w4_workspace_bytes(M, N, K);
    if (workspace_bytes < need || (need && !workspace)) return MX_ERROR_WORKSPACE;
    if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(sa, 4) || !aligned(sw, 4) || !aligned(y_bf16, 2) ||
        (need && !aligned(workspace, 16)))
        return MX_ERROR_MISALIGNED;
    if ((st = check_device()) != MX_SUCCESS) return st;
    return launched(mx::launch_gemm_a4w4(qa, sa, qw, sw, y_bf16, M, N, K, workspace, reinterpret_cast<hipStream_t>(stream)));
}

MX_API mx_status mx_gemm_a4w4_bf16_noalloc(const void* qa, const void* sa, const void* qw, const void* sw,
                                           void* y_bf16, int64_t M, int64_t N, int64_t K, void* stream) {
    mx_status st = check_gemm(M, N, K);
    if (st != MX_SUCCESS) return st;
    if (M == 0 || N == 0) return MX_SUCCESS;
    if (!qa || !sa || !qw || !sw || !y_bf16) return MX_ERROR_INVALID_VALUE;
    if (mx_gemm_a4w4_workspace_bytes(M, N, K) > mx::kGemmScratchBytes) return MX_ERROR_WORKSPACE;
    if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(sa, 4) || !aligned(sw, 4) || !aligned(y_bf16, 2))
        return MX_ERROR_MISALIGNED;
    if ((st = check_device()) != MX_SUCCESS) return st;
    return launched(mx::launch_gemm_a4w4_noalloc(qa, sa, qw, sw, y_bf16, M, N, K, reinterpret_cast<hipStream_t>(stream)));
}

MX_API size_t mx_linear_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_gemm(M, N, K) != MX_SUCCESS || M == 0 || N == 0) return 0;
    return mx::linear_a4w4_workspace_bytes(M, N, K);
}

MX_API mx_status mx_linear_a4w4_bf16(const void* x_bf16, const void* qw, const void* sw, void* y_bf16, int64_t M,
                                     int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
    mx_status st = check_gemm(M, N, K);
    if (st != MX_SUCCESS) return st;
    if (M == 0 || N == 0) return MX_SUCCESS;
    if (!x_bf16 || !qw || !sw || !y_bf16) return MX_ERROR_INVALID_VALUE;
    const size_t need = mx_linear_a4w4_workspace_bytes(M, N, K);
    if (workspace_bytes < need || (need && !workspace)) return MX_ERROR_WORKSPACE;
    if (!aligned(x_bf16, 16) || !aligned(qw, 16) || !aligned(sw, 4) || !aligned(y_bf16, 2) ||
        (need && !aligned(workspace, 256)))
        return MX_ERROR_MISALIGNED;
    if ((st = check_device()) != MX_SUCCESS) return st;
    return launched(mx::launch_linear_a4w4(x_bf16, qw, sw, y_bf16, M, N, K, workspace,
                                           reinterpret_cast<hipStream_t>(stream)));
}

MX_API mx_status mx_gemm_a4w4_grouped_bf16(const void* qa, const void* sa, const void* qw, const void* sw,
                                           void* y_bf16, const int32_t* offsets, int64_t G, int64_t max_rows,
                                           int64_t N, int64_t K, void* stream) {
    if (G < 0 || N < 0 || max_rows < 0) return MX_ERROR_INVALID_VALUE;
    if (max_rows > INT32_MAX || G > 65535 || N > INT32_MAX || K <= 0 || K % 512 != 0 || K > 16384)
        return MX_ERROR_UNSUPPORTED_SHAPE;
    if (N > (INT64_C(1) << 40) / K / (G > 0 ? G : 1)) return MX_ERROR_UNSUPPORTED_SHAPE;
    if (G == 0 || N == 0 || max_rows == 0) return MX_SUCCESS;
    if (!qa || !sa || !qw || !sw || !y_bf16 || !offsets) return MX_ERROR_INVALID_VALUE;
    if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(sa, 16) || !aligned(sw, 16) || !aligned(y_bf16, 2) ||
        !aligned(offsets, 4))
        return MX_ERROR_MISALIGNED;
    mx_status st;
    if ((st = check_device()) != MX_SUCCESS) return st;
    return launched(mx::launch_a4w4_grouped(qa, sa, qw, sw, y_bf16, offsets, G, max_rows, N, K,
                                            reinterpret_cast<hipStream_t>(stream)));
}

static mx_status quant_ptpc(bool f32, const void* x, int64_t rows, int64_t K, void* q, float* s, void* stream) {
    mx_status st = check_rows(rows, K, 8);
    if (st != MX_SUCCESS) return st;
    if (rows == 0) return MX_SUCCESS;
    if (!x || !q || !s) return MX_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(s, 4)) return MX_ERROR_MISALIGNED;
    if ((st = check_device()) != MX_SUCCESS) return st;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    return launched(f32 ? mx::launch_quant_ptpc_f32(x, rows, K, q, s, hs)
                        : mx::launch_quant_ptpc_bf16(x, rows, K, q, s, hs));
}

MX_API mx_status ptpc_quant_act_fp8(const void* x_bf16, int64_t M, int64_t K, void* q, float* s, void* stream) {
    return quant_ptpc(false, x_bf16, M, K, q, s, stream);
}

MX_API mx_status ptpc_quant_weight_f32(const float* w, int64_t N, int64_t K, void* q, float* s, void* stream) {
    return quant_ptpc(true, w, N, K, q, s, stream);
}

MX_API size_t gemm_a8w8_ptpc_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_gemm(M, N, K) != MX_SUCCESS || M == 0 || N == 0) return 0;
    return mx::gemm_a8w8_workspace_bytes(M, N, K);
}

MX_API mx_status gemm_a8w8_ptpc_bf16(const void* qa, const float* sa, const void* qw, const float* sw, void* y_bf16,
                                     int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    mx_status st = check_gemm(M, N, K);
    if (st != MX_SUCCESS) return st;
    if (M == 0 || N == 0) return MX_SUCCESS;
    if (!qa || !sa || !qw || !sw || !y_bf16) return MX_ERROR_INVALID_VALUE;
    const size_t need = gemm_a8w8_ptpc_workspace_bytes(M, N, K);
    if (workspace_bytes < need || (need && !workspace)) return MX_ERROR_WORKSPACE;
    if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(sa, 4) || !aligned(sw, 4) || !aligned(y_bf16, 2) ||
        (need && !aligned(workspace, 16)))
        return MX_ERROR_MISALIGNED;
    if ((st = check_device()) != MX_SUCCESS) return st;
    return launched(mx::launch_gemm_a8w8(qa, sa, qw, sw, y_bf16, M, N, K, workspace,
                                         reinterpret_cast<hipStream_t>(stream)));
}
