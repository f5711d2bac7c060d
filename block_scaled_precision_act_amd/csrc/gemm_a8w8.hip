// gemm_a8w8.hip - PTPC FP8 A8W8 GEMM entry (E4M3 operands with per-token and
// per-output-channel FP32 scales: "Kimi-K3-DSpark-FP8-PTPC", section "Phase 1
// FP8 PTPC Quantization").  E4M3 codes are widened exactly to FP16 for the
// MFMAs; the two FP32 scales are applied in the epilogue.
//
// 33 <= M <= 64 with K = 8192 or 16384 (4 or 8 K parts of 2048) takes the
// split-K kernel (gemm_splitk_fp8 in gemm_splitk.hpp), which needs the caller's
// workspace, when its grid (128 .. 256 workgroups) fits the device at once.
// Measured (graph-replayed, rotated weights, N = 7168, K = 8192): M = 64 15.7
// vs 18.6 us for the decode ring, M = 48 14.6 vs 17.2 us; at M <= 32 the ring
// is as fast or faster (M = 1 11.4 vs 13.0, M = 32 13.4 vs 13.1 us), so it
// keeps those.
//
// M > 128 with at most 256 output tiles of 128 x 128 (M <= 512 at N = 7168):
// gemm_tile128_pc_fp8 (copy waves beside the MFMA waves), one tile per
// workgroup, and with at most 128 tiles K in two parts over 2 x tiles
// workgroups summed in the caller's workspace (64 KB per tile).  Otherwise, where
// the 256 x 224 tiles number at most 128 (M <= 1024 at N = 7168), K is split
// into two parts of them (parts of at least 1024), summed in the caller's
// workspace (gemm_tile224_fp8<VEC, 2>): one workgroup takes about 133 us per
// tile at K = 8192 (the FP16 MFMAs bound it), so few tiles left most CUs idle.
// More parts would fit only at most 64 such tiles, which the 128 x 128 tiles
// always take.  Measured (graph-replayed, rotated weights, N = 7168, K = 8192):
// one 256 x 224 workgroup per tile took 133-135 us at every M from 129 to 1024;
// its two K parts M = 768 / 1024 93.0 / 103.8 us (before the 128 x 128 tile took
// the smaller M: 8 parts at M = 136 / 256 48.8 / 51.6 us, 4 at M = 512 70.4 us);
// the 128 x 128 tile M = 136 / 200 / 256 35.4 / 35.1 / 35.5 us (two parts),
// M = 384 / 512 55.8 / 60.8-65.2 us.
// Everything else runs the kernels of gemm_kernels.hpp.
#include "gemm_kernels.hpp"
#include "gemm_splitk.hpp"
#include "launch.hpp"

namespace mx {

namespace {

constexpr int kNsl8 = 16;  // slabs (K = 128) per K part

// parts and tiles of the FP8 split-K plan; kp == 0 if none (depends on the shape only)
struct Split8 {
    int kp = 0, tiles = 0;
    int grid() const { return 8 * kp * ((tiles + 7) / 8); }
    bool fits_device() const { return kp != 0 && grid() <= device_cus(); }
};

Split8 split8_plan(int64_t M, int64_t N, int64_t K) {
    Split8 p;
    if (M < 33 || M > 64 || K % (128 * kNsl8) != 0 || N < 1 || N > (int64_t)sk::kTN * sk::kMaxGrid) return p;
    const int64_t kp = K / (128 * kNsl8);
    if (kp != 4 && kp != 8) return p;
    const int tiles = (int)((N + sk::kTN - 1) / sk::kTN);
    if ((int64_t)tiles * kp < 128 || 8 * kp * ((tiles + 7) / 8) > sk::kMaxGrid) return p;
    p.kp = (int)kp;
    p.tiles = tiles;
    return p;
}

// M > 128 on 128 x 128 tiles, two K parts when kp == 2 (see the file comment); kp == 0 if none
struct Pc8 {
    int kp = 0, tiles_m = 0, tiles_n = 0;
    int tiles() const { return tiles_m * tiles_n; }
    int grid() const { return kp == 1 ? tiles() : 8 * kp * ((tiles() + 7) / 8); }
    bool fits_device() const { return kp == 2 && grid() <= device_cus(); }
};

Pc8 pc8_plan(int64_t M, int64_t N, int64_t K) {
    Pc8 p;
    if (M <= 128 || N < 1) return p;
    const int64_t tm = (M + 127) / 128, tn = (N + 127) / 128;
    if (tm * tn > 256) return p;
    p.kp = tm * tn <= 128 && K % 256 == 0 && K / 2 >= 1024 ? 2 : 1;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    return p;
}

template <int KP>
hipError_t launch_pc8(const Pc8& p, const void* qa, const float* sa, const void* qw, const float* sw, void* y,
                      int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
    const dim3 grid((unsigned)(KP == 1 ? p.tiles() : p.grid())), block(512);
    if (N % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0)
        hipLaunchKernelGGL((gemm_tile128_pc_fp8<true, KP>), grid, block, 0, st, a, sa, w, sw, out, (int)M, (int)N,
                           (int)K, p.tiles_m, p.tiles_n, w8);
    else
        hipLaunchKernelGGL((gemm_tile128_pc_fp8<false, KP>), grid, block, 0, st, a, sa, w, sw, out, (int)M, (int)N,
                           (int)K, p.tiles_m, p.tiles_n, w8);
    return hipGetLastError();
}

// M > 128 on 256 x 224 tiles with K in parts (see the file comment); kp == 0 if none
struct Tile8 {
    int kp = 0, tiles_m = 0, tiles_n = 0;
    int tiles() const { return tiles_m * tiles_n; }
    int grid() const { return 8 * kp * ((tiles() + 7) / 8); }
    bool fits_device() const { return kp != 0 && grid() <= device_cus(); }
};

Tile8 tile8_plan(int64_t M, int64_t N, int64_t K) {
    Tile8 p;
    if (M <= 128 || N < 1 || (M > N ? M : N) * K >= ((int64_t)1 << 31)) return p;
    const int64_t tm = (M + tile224_fp8::kTM - 1) / tile224_fp8::kTM, tn = (N + tile224_fp8::kTN - 1) / tile224_fp8::kTN;
    // Two K parts.  More never fit: this plan runs only past 256 tiles of 128 x 128 (the copy/MFMA-wave
    // kernel takes fewer), which means more than 64 of these tiles (128 tn128 tm128 <= 2 tm ceil(1.75 tn),
    // at most 256 when tm tn <= 64), and 4 parts of more than 64 tiles would exceed 256 workgroups.
    if (tm * tn > 128 || K % 256 != 0 || K / 2 < 1024 || 16 * ((tm * tn + 7) / 8) > sk::kMaxGrid) return p;
    p.kp = 2;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    return p;
}

template <int KP>
hipError_t launch_tile8(const Tile8& p, const void* qa, const float* sa, const void* qw, const float* sw, void* y,
                        int64_t M, int64_t N, int64_t K, void* ws, hipStream_t st) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
    const dim3 grid((unsigned)p.grid()), block(256);
    if (N % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0)
        hipLaunchKernelGGL((gemm_tile224_fp8<true, KP>), grid, block, 0, st, a, sa, w, sw, out, (int)M, (int)N, (int)K,
                           p.tiles_m, p.tiles_n, w8);
    else
        hipLaunchKernelGGL((gemm_tile224_fp8<false, KP>), grid, block, 0, st, a, sa, w, sw, out, (int)M, (int)N,
                           (int)K, p.tiles_m, p.tiles_n, w8);
    return hipGetLastError();
}

}  // namespace

size_t gemm_a8w8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const Split8 p = split8_plan(M, N, K);
    if (p.kp) return sk::workspace_bytes(p.tiles, p.kp, 2);
    const Pc8 c = pc8_plan(M, N, K);
    if (c.kp) return c.kp == 2 ? sk::workspace_bytes_compact(c.tiles(), 2, 4) : 0;
    const Tile8 t = tile8_plan(M, N, K);
    return t.kp ? sk::workspace_bytes_chunked(t.tiles(), t.kp, tile224_fp8::kMf) : 0;
}

hipError_t launch_gemm_a8w8(const void* qa, const float* sa, const void* qw, const float* sw, void* y, int64_t M,
                            int64_t N, int64_t K, void* workspace, hipStream_t st) {
    const Split8 p = split8_plan(M, N, K);
    if (workspace && p.fits_device()) {
        const dim3 grid((unsigned)p.grid()), block(256);
        const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
        const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
        uint16_t* out = reinterpret_cast<uint16_t*>(y);
        uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
        // a 3-slot ring: 2 slabs in flight per wave measured faster than 3 or 5 (M = 64: 15.7, 16.3, 18.6 us)
        if (p.kp == 4)
            hipLaunchKernelGGL((gemm_splitk_fp8<2, 3, kNsl8, 4>), grid, block, 0, st, a, sa, w, sw, out, (int)M, (int)N,
                               (int)K, p.tiles, ws);
        else
            hipLaunchKernelGGL((gemm_splitk_fp8<2, 3, kNsl8, 8>), grid, block, 0, st, a, sa, w, sw, out, (int)M, (int)N,
                               (int)K, p.tiles, ws);
        return hipGetLastError();
    }
    const Pc8 c = pc8_plan(M, N, K);
    if (c.kp) {
        if (workspace && c.fits_device()) return launch_pc8<2>(c, qa, sa, qw, sw, y, M, N, K, workspace, st);
        return launch_pc8<1>(c, qa, sa, qw, sw, y, M, N, K, nullptr, st);
    }
    const Tile8 t = tile8_plan(M, N, K);
    if (workspace && t.fits_device()) return launch_tile8<2>(t, qa, sa, qw, sw, y, M, N, K, workspace, st);
    return launch_gemm<true>(qa, sa, qw, sw, y, M, N, K, st);
}

}  // namespace mx
