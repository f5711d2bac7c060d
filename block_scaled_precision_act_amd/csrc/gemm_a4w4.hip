// gemm_a4w4.hip - MXFP4 A4W4 GEMM, one-call layer and grouped entries ("A4W4 dispatch" with
// dynamic MXFP4 activations: "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact quantization
// coverage"; expert weights and activations in OCP MXFP4: "Kimi-K3-Quark-MXFP4-AttnFP8", section
// "Model Quantization").
//
// GEMM.  Decode sizes with K = 8192 or 16384 take the split-K kernels of gemm_splitk.hpp (128-column
// tiles, the partials summed across the tile's workgroups in the caller's workspace): M <= 64 in K
// parts of 2048, and 64 < M <= 128 in two 64-row halves with K parts of 4096 or 8192 (M = 128,
// N = 7168, K = 8192: 12.9 vs 17.3 us for the two-row-halves ring).  A plan is taken when its grid
// keeps at least half of the CUs busy and fits the device at once; otherwise (a device with fewer CUs,
// say) the ring kernels run and the workspace is not touched.  Other shapes take the kernels of
// gemm_kernels.hpp: the decode rings for M <= 128 (K split over the waves of a workgroup) and the
// LDS-tiled kernels above, whose 128 x 128 tile kernel with copy and MFMA waves also splits K in two parts
// over 2 x tiles workgroups when there are at most 128 tiles (M = 136 / 256, N = 7168, K = 8192: 16.7 /
// 17.9-18.7 us against 19.4 / 21.0 us with full K; the 4-wave kernel's two parts took 20.6 / 20.9 us and
// full K 26.5 / 26.9 us).  Past 128 tiles, two 4-wave workgroups per CU on a 2-slot ring gained 3% at
// M = 384 and nothing at M = 512, and K parts of 256 x 224 tiles lost: their partials overflow the L2s.  Measured (graph-replayed, rotated weights, us), split-K vs ring: K = 8192,
// N = 7168: M = 64 10.4 vs 12.4, M = 1 7.8 vs 8.4; K = 8192, N = 2048, M = 64: 6.6 vs 9.9; K = 16384,
// N = 4096, M = 64: 11.1 vs 17.7.  At K = 4096 the rings are as fast or faster (N = 7168, M = 64: 7.4
// vs 7.2), so they keep it.
//
// Layer.  mx_linear_a4w4_bf16 quantizes inside the split-K workgroups (one launch) for M <= 8, where
// that beat the quantizer + GEMM pair (N = 7168, K = 8192, M = 1: 8.6 vs 9.9 us); above that every
// workgroup quantizing its K part of all M rows costs more than the second launch (M = 16: 11.4 vs
// 10.4 us), so the layer runs the quantizer and the GEMM.
//
// Grouped.  gemm_grouped_fp4 (128-column tiles, K walked in parts) for K % 1024 == 0 where it measured
// faster (see launch_a4w4_grouped), else the grouped decode ring (K % 2048 == 0) or the grouped LDS-staged
// decode kernel (other K % 512 == 0).
#include <mutex>

#include "gemm_kernels.hpp"
#include "gemm_splitk.hpp"
#include "launch.hpp"

namespace mx {

int device_cus() {
    constexpr int kMaxDevices = 64;
    static int cus[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(once[dev], [dev] {
        int n = 0;
        cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
    });
    return cus[dev];
}

namespace {

// The split-K plan of a shape: slabs (K = 256) per part, parts, tiles, fragments; nsl == 0 if none.  Every
// plan keeps at least half of the 256 CUs busy with at most 256 workgroups (it depends on the shape only, so
// the workspace queries do too).  layer: the one-launch layer's plan (parts of 1024 or 2048 K-values); else
// the GEMM's (parts of 2048, at least 4: measured faster than the decode rings there).
struct SplitPlan {
    int nsl = 0, kp = 0, tiles = 0, mf = 0;
    int grid() const { return 8 * kp * ((tiles + 7) / 8); }
    // The kernel's tail needs every workgroup resident at once (one per CU: its LDS block rules out two).
    bool fits_device() const { return nsl != 0 && grid() <= device_cus(); }
};

SplitPlan split_plan(int64_t M, int64_t N, int64_t K, bool layer) {
    SplitPlan p;
    if (M < 1 || M > 64 || K % 1024 != 0 || N < 1 || N > (int64_t)sk::kTN * sk::kMaxGrid) return p;
    const int tiles = (int)((N + sk::kTN - 1) / sk::kTN);
    for (int nsl : {8, 4}) {
        if (K % (256 * nsl) != 0) continue;
        const int64_t kp = K / (256 * nsl);
        if (kp != 2 && kp != 4 && kp != 8) continue;
        if (!layer && (nsl != 8 || kp < 4)) continue;
        if ((int64_t)tiles * kp < 128 || 8 * kp * ((tiles + 7) / 8) > sk::kMaxGrid) continue;
        p.nsl = nsl;
        p.kp = (int)kp;
        p.tiles = tiles;
        p.mf = M <= 32 ? 1 : 2;
        return p;
    }
    return p;
}

// 64 < M <= 128: the split-K plan over two row halves (gemm_splitk_fp4_rh): parts of 4096 or 8192 K-values,
// 2 x parts x tiles between 128 and 256 workgroups; kp == 0 if none.
struct RhPlan {
    int nsl = 0, kp = 0, tiles = 0;
    int grid() const { return 8 * 2 * kp * ((tiles + 7) / 8); }
    bool fits_device() const { return kp != 0 && grid() <= device_cus(); }
};

RhPlan rh_plan(int64_t M, int64_t N, int64_t K) {
    RhPlan p;
    if (M <= 64 || M > 128 || N < 1 || N > (int64_t)sk::kTN * sk::kMaxGrid) return p;
    const int tiles = (int)((N + sk::kTN - 1) / sk::kTN);
    for (int nsl : {16, 32}) {
        if (K % (256 * nsl) != 0) continue;
        const int64_t kp = K / (256 * nsl);
        if (kp != 2 && kp != 4) continue;
        if (2 * kp * tiles < 128 || 8 * 2 * kp * ((tiles + 7) / 8) > sk::kMaxGrid) continue;
        p.nsl = nsl;
        p.kp = (int)kp;
        p.tiles = tiles;
        return p;
    }
    return p;
}

// M > 128 with at most 128 output tiles of 128 x 128 (M <= 256 at N = 7168): one tile per workgroup would
// leave half of the CUs idle or more, so K is split in two parts over 2 x tiles workgroups
// (gemm_tile128_pc_fp4<VEC, 2>, one per CU) whose partials meet in the workspace (compact slots, 64 KB per
// tile, at most 8 MiB).  K % 2048 == 0 (parts of whole scale blocks); tile t's two workgroups share an XCD.
struct TilePlan {
    int tiles_m = 0, tiles_n = 0;
    int tiles() const { return tiles_m * tiles_n; }
    int grid() const { return 16 * ((tiles() + 7) / 8); }
    bool fits_device() const { return tiles_m != 0 && grid() <= device_cus(); }
};

TilePlan tile_plan(int64_t M, int64_t N, int64_t K) {
    TilePlan p;
    if (M <= 128 || N < 1 || K % 2048 != 0) return p;
    const int64_t tm = (M + 127) / 128, tn = (N + 127) / 128;
    if (tm * tn > 128) return p;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    return p;
}

hipError_t launch_tile_split(const TilePlan& p, const void* qa, const void* sa, const void* qw, const void* sw,
                             void* y, int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
    const dim3 grid((unsigned)p.grid()), block(512);
    const int m = (int)M, n = (int)N, k = (int)K;
    if (N % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0)
        hipLaunchKernelGGL((gemm_tile128_pc_fp4<true, 2>), grid, block, 0, st, a, sa8, w, sw8, out, m, n, k,
                           p.tiles_m, p.tiles_n, w8);
    else
        hipLaunchKernelGGL((gemm_tile128_pc_fp4<false, 2>), grid, block, 0, st, a, sa8, w, sw8, out, m, n, k,
                           p.tiles_m, p.tiles_n, w8);
    return hipGetLastError();
}

template <int NSL>
hipError_t launch_rh_nsl(const RhPlan& p, const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                         int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
    const dim3 grid((unsigned)p.grid()), block(256);
    // a 4-slot ring (measured against 3 and 5 slots: within 1%)
    if (p.kp == 2)
        hipLaunchKernelGGL((gemm_splitk_fp4_rh<4, NSL, 2>), grid, block, 0, st, a, sa8, w, sw8, out, (int)M, (int)N,
                           (int)K, p.tiles, w8);
    else
        hipLaunchKernelGGL((gemm_splitk_fp4_rh<4, NSL, 4>), grid, block, 0, st, a, sa8, w, sw8, out, (int)M, (int)N,
                           (int)K, p.tiles, w8);
    return hipGetLastError();
}

template <int MF, int S, int NSL, int KP, bool FUSED>
hipError_t launch_split_kp(const SplitPlan& p, const uint8_t* a, const uint8_t* sa, const uint8_t* w,
                           const uint8_t* sw, uint16_t* y, int m, int n, int k, uint8_t* ws, hipStream_t st) {
    hipLaunchKernelGGL((gemm_splitk_fp4<MF, S, NSL, KP, FUSED>), dim3((unsigned)p.grid()), dim3(256), 0, st, a, sa, w,
                       sw, y, m, n, k, p.tiles, ws);
    return hipGetLastError();
}

template <int MF, int S, int NSL, bool FUSED>
hipError_t launch_split_nsl(const SplitPlan& p, const uint8_t* a, const uint8_t* sa, const uint8_t* w,
                            const uint8_t* sw, uint16_t* y, int m, int n, int k, uint8_t* ws, hipStream_t st) {
    switch (p.kp) {
        case 2: return launch_split_kp<MF, S, NSL, 2, FUSED>(p, a, sa, w, sw, y, m, n, k, ws, st);
        case 4: return launch_split_kp<MF, S, NSL, 4, FUSED>(p, a, sa, w, sw, y, m, n, k, ws, st);
        default: return launch_split_kp<MF, S, NSL, 8, FUSED>(p, a, sa, w, sw, y, m, n, k, ws, st);
    }
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
    // ring depth: 4 slots with 64 activation rows (140 KB of LDS), 5 with 32 (122 KB); 4 at 4 slabs per part.
    // The one-launch layer (FUSED) runs only for M <= 8: one fragment.
    if constexpr (FUSED) {
        return p.nsl == 8 ? launch_split_nsl<1, 5, 8, true>(p, a, sa8, w, sw8, out, m, n, k, ws, st)
                          : launch_split_nsl<1, 4, 4, true>(p, a, sa8, w, sw8, out, m, n, k, ws, st);
    } else {
        // the GEMM's plans: parts of 2048 (8 slabs), 4 or 8 of them
        if (p.mf == 1)
            return p.kp == 4 ? launch_split_kp<1, 5, 8, 4, false>(p, a, sa8, w, sw8, out, m, n, k, ws, st)
                             : launch_split_kp<1, 5, 8, 8, false>(p, a, sa8, w, sw8, out, m, n, k, ws, st);
        return p.kp == 4 ? launch_split_kp<2, 4, 8, 4, false>(p, a, sa8, w, sw8, out, m, n, k, ws, st)
                         : launch_split_kp<2, 4, 8, 8, false>(p, a, sa8, w, sw8, out, m, n, k, ws, st);
    }
}

bool aligned16(const void* a, const void* b) {
    return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) == 0;
}

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t gemm_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const SplitPlan p = split_plan(M, N, K, false);
    if (p.nsl) return sk::workspace_bytes(p.tiles, p.kp, p.mf);
    const RhPlan r = rh_plan(M, N, K);
    if (r.kp) return sk::workspace_bytes(2 * r.tiles, r.kp, 2);
    const TilePlan t = tile_plan(M, N, K);
    return t.tiles_m ? sk::workspace_bytes_compact(t.tiles(), 2, 4) : 0;
}

hipError_t launch_gemm_a4w4(const void* qa, const void* sa, const void* qw, const void* sw, void* y, int64_t M,
                            int64_t N, int64_t K, void* workspace, hipStream_t st) {
    const SplitPlan p = split_plan(M, N, K, false);
    if (workspace && aligned16(sa, sw) && p.fits_device())
        return launch_split<false>(p, qa, sa, qw, sw, y, M, N, K, workspace, st);
    const RhPlan r = rh_plan(M, N, K);
    if (workspace && aligned16(sa, sw) && r.fits_device())
        return r.nsl == 16 ? launch_rh_nsl<16>(r, qa, sa, qw, sw, y, M, N, K, workspace, st)
                           : launch_rh_nsl<32>(r, qa, sa, qw, sw, y, M, N, K, workspace, st);
    const TilePlan t = tile_plan(M, N, K);
    if (workspace && aligned16(sa, sw) && t.fits_device())
        return launch_tile_split(t, qa, sa, qw, sw, y, M, N, K, workspace, st);
    return launch_gemm<false>(qa, sa, qw, sw, y, M, N, K, st);
}

// The layer's workspace holds either path: the one-launch split-K layer's partial slots, or the quantizer's
// codes and scales placed past the largest partial area of any split-K launch (the split-K kernels read a 0
// word there as "not written yet", so nothing else may leave data in that area of a shared workspace),
// followed through by the GEMM, whose own split-K plan then uses the partial area.
constexpr int kLinearOneLaunchMaxM = 8;
constexpr size_t kLinearCodesOffset = sk::kMaxWorkspaceBytes;

size_t linear_a4w4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const SplitPlan p = split_plan(M, N, K, true);
    const size_t one = p.nsl ? sk::workspace_bytes(p.tiles, p.kp, p.mf) : 0;
    const size_t two = kLinearCodesOffset + align256((size_t)M * K / 2) + align256((size_t)M * K / 32);
    return one > two ? one : two;
}

hipError_t launch_linear_a4w4(const void* x, const void* qw, const void* sw, void* y, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t st) {
    const SplitPlan p = split_plan(M, N, K, true);
    if (M <= kLinearOneLaunchMaxM && aligned16(qw, sw) && p.fits_device())
        return launch_split<true>(p, x, nullptr, qw, sw, y, M, N, K, workspace, st);
    uint8_t* qa = reinterpret_cast<uint8_t*>(workspace) + kLinearCodesOffset;
    uint8_t* sa = qa + align256((size_t)M * K / 2);
    hipError_t e = launch_quant_mx_bf16(x, M, K, qa, sa, st);
    if (e != hipSuccess) return e;
    return launch_gemm_a4w4(qa, sa, qw, sw, y, M, N, K, workspace, st);
}

// ---------------------------------------------------------------------------------------------------------
// Allocation-free GEMM: the split-K workspace lives in a static device array (zero-filled when the code
// object is loaded; every call leaves its counters at zero again), one copy per GPU.  In host code the
// array's name is only a stand-in: its device address is looked up once per device, with that device
// current, and only that address is ever passed to a kernel.
namespace {
static_assert(kGemmScratchBytes >= sk::kMaxWorkspaceBytes, "the static workspace holds every split-K plan");
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

// Grouped GEMM.  gemm_grouped_fp4 (one 128-column tile per workgroup and expert, K walked in parts of 8 or
// 4 slabs) where it measured faster than the 32-column kernels of gemm_kernels.hpp (graph-replayed, two
// rotated weight sets, 64 tokens x top-8 routed over the experts; us, this kernel vs the other):
//   K = 2048, 32 experts of [7168, 2048]: 47.9 vs 57.4 (the ring), parts of 8 slabs, a 2-slot ring, two
//             workgroups per CU for 32-row chunks (50.3 us with a 5-slot ring, one per CU);
//   K = 7168, 32 experts of [2048, 7168]: 43.0 vs 56.7 (the LDS-staged kernel); 64-row chunks (256
//             tokens): 83.6 vs 152;
//   K = 4096, 32 experts of [7168, 4096]: 86 vs 97 (the ring); 64-row chunks: 153 vs 229;
//   K = 16384, 32 experts of [2048, 16384], 64-row chunks: 193 vs 212.
// The ring stays faster for 32-row chunks over few 128-column tiles (32 experts of [2048, 8192]: 65 vs 53;
// 16 of [4096, 16384]: 180 vs 160): with under 1024 workgroups the tiles leave CUs idle.  K % 1024 != 0
// (parts of 4 slabs do not fit) takes the LDS-staged kernel.
hipError_t launch_a4w4_grouped(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                               const int32_t* offsets, int64_t G, int64_t max_rows, int64_t N, int64_t K,
                               hipStream_t st) {
    const int64_t tiles = (N + sk::kTN - 1) / sk::kTN;
    const bool wide = max_rows > 32;
    const bool tile_path = K == 2048 || (K % 1024 == 0 && (wide || K % 2048 != 0 || tiles * G >= 1024));
    if (!tile_path) return launch_gemm_a4w4_grouped(qa, sa, qw, sw, y, offsets, G, max_rows, N, K, st);
    // the entry point has checked the 16-byte alignment of every operand
    const dim3 grid((unsigned)tiles, (unsigned)G);
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    const int n = (int)N, k = (int)K, t = (int)tiles;
    if (K == 2048 && !wide)
        hipLaunchKernelGGL((gemm_grouped_fp4<1, 2, 8>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, n, k, t, offsets);
    else if (K == 2048)
        hipLaunchKernelGGL((gemm_grouped_fp4<2, 4, 8>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, n, k, t, offsets);
    else if (!wide)
        hipLaunchKernelGGL((gemm_grouped_fp4<1, 2, 4>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, n, k, t, offsets);
    else
        hipLaunchKernelGGL((gemm_grouped_fp4<2, 2, 4>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, n, k, t, offsets);
    return hipGetLastError();
}

}  // namespace mx
