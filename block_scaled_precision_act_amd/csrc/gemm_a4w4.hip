// gemm_a4w4.hip - MXFP4 A4W4 GEMM and one-launch layer entries ("A4W4 dispatch"
// with dynamic MXFP4 activations: "Kimi-K3 DSpark O-Proj-only MXFP4", section
// "Exact quantization coverage").
//
// GEMM.  Decode sizes (M <= 64) whose 32-column tiles would occupy at most half
// of the 256 CUs, with K long enough for parts of 2048 K-values, take the
// split-K kernel (gemm_splitk.hpp), which needs the caller's workspace.  Other
// shapes take the kernels of gemm_kernels.hpp: the decode rings for M <= 128
// (K split over the waves of a workgroup) and the LDS-tiled kernels above.
// Measured (N, K, M = 64 unless noted; graph-replayed): split-K is faster at
// (4096, 8192) 9.7 vs 10.3 us and (2048, 16384, M = 32) 9.5 vs 12.5 us, slower
// at (7168, 8192) 11.7 vs 11.3 us, (2048, 8192) and (7168, 4096): there its
// cross-workgroup reduction (partial stores, count, partial loads: about 3 us
// of round trips) costs more than the activation re-reads it saves.
//
// Layer.  mx_linear_a4w4_bf16 runs the split-K kernel with its activation block
// quantized from BF16 X inside each workgroup (one launch) whenever a split-K
// plan exists (M <= 64), else the quantizer and the GEMM in two launches.
#include <mutex>

#include "gemm_kernels.hpp"
#include "gemm_splitk.hpp"
#include "launch.hpp"

namespace mx {

namespace {

// The split-K plan of a shape: slabs (K = 256) per part, parts, tiles, fragments; nsl == 0 if none.
// layer: the one-launch layer's plan (any split that keeps half the CUs busy); else the GEMM's (only
// where the split was measured faster than the decode rings).
struct SplitPlan {
    int nsl = 0, kp = 0, tiles = 0, mf = 0;
    int grid() const { return 8 * kp * ((tiles + 7) / 8); }
};

SplitPlan split_plan(int64_t M, int64_t N, int64_t K, bool layer) {
    SplitPlan p;
    if (M < 1 || M > 64 || K % 1024 != 0 || N < 1 || N > (int64_t)sk::kTN * sk::kMaxTiles) return p;
    const int tiles = (int)((N + sk::kTN - 1) / sk::kTN);
    if (!layer && (N + 31) / 32 > 128) return p;  // the decode rings fill more than half the CUs
    for (int nsl : {8, 4}) {
        if (K % (256 * nsl) != 0) continue;
        const int64_t kp = K / (256 * nsl);
        if (kp != 2 && kp != 4 && kp != 8) continue;
        if (!layer && (nsl != 8 || kp < 4)) continue;
        // at least half the 256 CUs busy, at most two rounds of workgroups
        if ((int64_t)tiles * kp < 128 || 8 * kp * ((tiles + 7) / 8) > 512) continue;
        p.nsl = nsl;
        p.kp = (int)kp;
        p.tiles = tiles;
        p.mf = M <= 32 ? 1 : 2;
        return p;
    }
    return p;
}

template <int MF, int S, int NSL, bool FUSED>
hipError_t launch_split_nsl(const SplitPlan& p, const uint8_t* a, const uint8_t* sa, const uint8_t* w,
                            const uint8_t* sw, uint16_t* y, int m, int n, int k, uint8_t* ws, hipStream_t st) {
    const dim3 grid((unsigned)p.grid()), block(256);
    switch (p.kp) {
        case 2: hipLaunchKernelGGL((gemm_splitk_fp4<MF, S, NSL, 2, FUSED>), grid, block, 0, st, a, sa, w, sw, y, m, n, k, p.tiles, ws); break;
        case 4: hipLaunchKernelGGL((gemm_splitk_fp4<MF, S, NSL, 4, FUSED>), grid, block, 0, st, a, sa, w, sw, y, m, n, k, p.tiles, ws); break;
        default: hipLaunchKernelGGL((gemm_splitk_fp4<MF, S, NSL, 8, FUSED>), grid, block, 0, st, a, sa, w, sw, y, m, n, k, p.tiles, ws); break;
    }
    return hipGetLastError();
}

// FUSED: qa is BF16 X [M, K] and sa is unused.
template <bool FUSED>
hipError_t launch_split(const SplitPlan& p, const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                        int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t st) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    const int m = (int)M, n = (int)N, k = (int)K;
    // ring depth: 4 slots with 64 activation rows (140 KB of LDS), 5 with 32 (122 KB); 4 at 4 slabs per part
    if (p.mf == 1)
        return p.nsl == 8 ? launch_split_nsl<1, 5, 8, FUSED>(p, a, sa8, w, sw8, out, m, n, k, ws, st)
                          : launch_split_nsl<1, 4, 4, FUSED>(p, a, sa8, w, sw8, out, m, n, k, ws, st);
    return p.nsl == 8 ? launch_split_nsl<2, 4, 8, FUSED>(p, a, sa8, w, sw8, out, m, n, k, ws, st)
                      : launch_split_nsl<2, 4, 4, FUSED>(p, a, sa8, w, sw8, out, m, n, k, ws, st);
}

bool aligned16(const void* a, const void* b) {
    return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) == 0;
}

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const SplitPlan p = split_plan(M, N, K, false);
    return p.nsl ? sk::workspace_bytes(p.tiles, p.kp, p.mf) : 0;
}

hipError_t launch_gemm_a4w4(const void* qa, const void* sa, const void* qw, const void* sw, void* y, int64_t M,
                            int64_t N, int64_t K, void* workspace, hipStream_t st) {
    const SplitPlan p = split_plan(M, N, K, false);
    if (p.nsl && workspace && aligned16(sa, sw))
        return launch_split<false>(p, qa, sa, qw, sw, y, M, N, K, workspace, st);
    return launch_gemm<false>(qa, sa, qw, sw, y, M, N, K, st);
}

// Either path fits: the one-launch split-K layer (counter area, then partials), or - when no plan applies or
// the weight scales are not 16-byte aligned - the activation codes and scales, placed after the counter area
// so that they never disturb the counters a later one-launch call relies on.  (The GEMM of the two-launch
// path never needs a workspace: a GEMM split-K plan implies a layer plan, and the only other reason to take
// two launches, unaligned weight scales, also rules the GEMM's split out.)
size_t linear_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const SplitPlan p = split_plan(M, N, K, true);
    const size_t fused = p.nsl ? sk::workspace_bytes(p.tiles, p.kp, p.mf) : 0;
    const size_t two = sk::kCounterBytes + align256((size_t)M * K / 2) + align256((size_t)M * K / 32);
    return fused > two ? fused : two;
}

hipError_t launch_linear_a4w4(const void* x, const void* qw, const void* sw, void* y, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t st) {
    const SplitPlan p = split_plan(M, N, K, true);
    if (p.nsl && aligned16(qw, sw)) return launch_split<true>(p, x, nullptr, qw, sw, y, M, N, K, workspace, st);
    uint8_t* qa = reinterpret_cast<uint8_t*>(workspace) + sk::kCounterBytes;
    uint8_t* sa = qa + align256((size_t)M * K / 2);
    hipError_t e = launch_quant_mx_bf16(x, M, K, qa, sa, st);
    if (e != hipSuccess) return e;
    return launch_gemm_a4w4(qa, sa, qw, sw, y, M, N, K, nullptr, st);
}

// ---------------------------------------------------------------------------------------------------------
// Allocation-free GEMM: the split-K workspace lives in a static device array (zero-filled when the code
// object is loaded; every call leaves its counters at zero again), one copy per GPU.  In host code the
// array's name is only a stand-in: its device address is looked up once per device, with that device
// current, and only that address is ever passed to a kernel.
namespace {
__device__ __align__(256) uint8_t scratch[kGemmScratchBytes];
constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];
std::once_flag g_scratch_once[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
}  // namespace

hipError_t gemm_scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    *out = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

hipError_t launch_gemm_a4w4_noalloc(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                                    int64_t M, int64_t N, int64_t K, hipStream_t st) {
    void* ws = nullptr;
    if (gemm_a4w4_workspace_bytes(M, N, K) > 0) {
        hipError_t e = gemm_scratch_ptr(&ws);
        if (e != hipSuccess) return e;
    }
    return launch_gemm_a4w4(qa, sa, qw, sw, y, M, N, K, ws, st);
}

hipError_t launch_a4w4_grouped(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                               const int32_t* offsets, int64_t G, int64_t max_rows, int64_t N, int64_t K,
                               hipStream_t st) {
    return launch_gemm_a4w4_grouped(qa, sa, qw, sw, y, offsets, G, max_rows, N, K, st);
}

}  // namespace mx
