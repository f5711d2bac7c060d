// gemm_kernels.hpp - block-scaled GEMM kernels for gfx950 (CDNA4 scaled MFMA).
//
// Y[m, n] = sum_k A[m, k] * W[n, k], BF16 out, where
//   FP4 (A4W4): A, W are MXFP4 - E2M1 codes, one E8M0 scale per 32 K-values
//     ("Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact quantization
//     coverage"); the scales are applied inside the MFMA
//     (v_mfma_scale_f32_*_f8f6f4, FP4 operands, one scale byte per lane).
//   FP8 (A8W8): A, W are E4M3 codes with one FP32 scale per row
//     ("Kimi-K3-DSpark-FP8-PTPC", section "Phase 1 FP8 PTPC Quantization").
//     The codes are widened exactly to FP16 in registers and multiplied with
//     FP16 MFMAs; the epilogue multiplies by sA[m] * sW[n].  (gfx950's FP8
//     MFMA sums each group of 8 products with a short internal adder - a
//     small product next to a large one in the same group is dropped - which
//     misses the 1e-6 * sum|a*w| accuracy this layer is held to; its FP16 and
//     FP4 MFMAs sum exactly up to FP32 rounding.)
// Both operands are K-contiguous, which is exactly the MFMA operand layout:
// in a 16x16x128 (32x32x64) MFMA, lane l supplies row l%16 (l%32) and 32
// consecutive K-values; for FP4 the lane's scale byte covers exactly those 32
// values (one MX block).
//
// K permutation (FP4).  An MFMA sums over whatever K-values its lanes supply,
// as long as A and W lanes agree.  So across the 4 MFMAs of one step, lane
// group q reads 64 contiguous code bytes (4 blocks) and one dword of 4
// consecutive scale bytes; MFMA t takes the t-th 16 bytes and selects scale
// byte t with op_sel.  Every lane then does wide contiguous loads and needs
// no scale shuffling.
#pragma once

#include "mx_device.hpp"

namespace mx {

// ============================================================================
// Decode path (small M, HBM-bound on the weight stream).
// One workgroup per 32 output columns; its NW waves split K and each streams
// its own slice of W (and of A) straight into registers; the partial tiles are
// summed through LDS in a fixed wave order (deterministic) and written as BF16.
// ============================================================================
template <bool FP8, int MF, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_decode_kernel(const uint8_t* __restrict__ qa,
                                                              const void* __restrict__ sa_,
                                                              const uint8_t* __restrict__ qw,
                                                              const void* __restrict__ sw_,
                                                              uint16_t* __restrict__ y, int M, int N, int K) {
    constexpr int NF = 2;  // 16-column fragments per workgroup
    __shared__ float red[NW][MF * NF * 4][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * (16 * NF);
    const int64_t KB = FP8 ? (int64_t)K : (int64_t)K / 2;  // code bytes per row
    const int64_t KS = (int64_t)K / 32;                     // FP4 scale bytes per row
    const int chunks = K / 128;
    const int c0 = (int)((int64_t)chunks * wave / NW), c1 = (int)((int64_t)chunks * (wave + 1) / NW);

    const uint8_t* arow[MF];
    const uint8_t* wrow[NF];
    const uint8_t* asrow[MF];
    const uint8_t* wsrow[NF];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        const int m = min(16 * i + r16, M - 1);  // rows past M are read (in bounds) and never stored
        arow[i] = qa + m * KB;
        asrow[i] = reinterpret_cast<const uint8_t*>(sa_) + m * KS;
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        const int n = min(n0 + 16 * j + r16, N - 1);
        wrow[j] = qw + n * KB;
        wsrow[j] = reinterpret_cast<const uint8_t*>(sw_) + n * KS;
    }

    v4f acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if constexpr (!FP8) {
        int c = c0;
        for (; c + 4 <= c1; c += 4) {
            // lane group q takes chunk c+q (64 code bytes = 4 blocks, one scale dword)
            uint4 a[MF][4], b[NF][4];
            int sa[MF], sb[NF];
            const int64_t off = 64 * (int64_t)(c + q);
#pragma unroll
            for (int j = 0; j < NF; ++j) {
#pragma unroll
                for (int t = 0; t < 4; ++t) b[j][t] = ldg16(wrow[j] + off + 16 * t);
                sb[j] = ldg4(wsrow[j] + 4 * (c + q));
            }
#pragma unroll
            for (int i = 0; i < MF; ++i) {
#pragma unroll
                for (int t = 0; t < 4; ++t) a[i][t] = ldg16(arow[i] + off + 16 * t);
                sa[i] = ldg4(asrow[i] + 4 * (c + q));
            }
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j) {
                    acc[i][j] = mfma16<kFmtFP4, 0>(fp4_operand(a[i][0]), fp4_operand(b[j][0]), acc[i][j], sa[i], sb[j]);
                    acc[i][j] = mfma16<kFmtFP4, 1>(fp4_operand(a[i][1]), fp4_operand(b[j][1]), acc[i][j], sa[i], sb[j]);
                    acc[i][j] = mfma16<kFmtFP4, 2>(fp4_operand(a[i][2]), fp4_operand(b[j][2]), acc[i][j], sa[i], sb[j]);
                    acc[i][j] = mfma16<kFmtFP4, 3>(fp4_operand(a[i][3]), fp4_operand(b[j][3]), acc[i][j], sa[i], sb[j]);
                }
        }
        for (; c < c1; ++c) {
            // single chunk: lane group q takes block 4c+q (16 code bytes, one scale byte)
            const int64_t off = 64 * (int64_t)c + 16 * q;
            uint4 a[MF], b[NF];
            int sa[MF], sb[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                b[j] = ldg16(wrow[j] + off);
                sb[j] = wsrow[j][4 * c + q];
            }
#pragma unroll
            for (int i = 0; i < MF; ++i) {
                a[i] = ldg16(arow[i] + off);
                sa[i] = asrow[i][4 * c + q];
            }
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j)
                    acc[i][j] = mfma16<kFmtFP4, 0>(fp4_operand(a[i]), fp4_operand(b[j]), acc[i][j], sa[i], sb[j]);
        }
    } else {
        // FP8: chunk c is 128 code bytes per row; lane group q takes bytes [32q, 32q+32).  The
        // codes are widened exactly to FP16 and run through FP16 MFMAs (K = 32 each): operand u
        // of a lane is its bytes [8u, 8u+8), so MFMA u covers bytes {32q + 8u + [0, 8)} over q.
        for (int c = c0; c < c1; ++c) {
            const int64_t off = 128 * (int64_t)c + 32 * q;
            uint4 a[MF][2], b[NF][2];
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                b[j][0] = ldg16(wrow[j] + off);
                b[j][1] = ldg16(wrow[j] + off + 16);
            }
#pragma unroll
            for (int i = 0; i < MF; ++i) {
                a[i][0] = ldg16(arow[i] + off);
                a[i][1] = ldg16(arow[i] + off + 16);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v8h bh[NF];
#pragma unroll
                for (int j = 0; j < NF; ++j) {
                    const uint4 v = b[j][u >> 1];
                    bh[j] = (u & 1) ? e4m3x8_to_f16x8(v.z, v.w) : e4m3x8_to_f16x8(v.x, v.y);
                }
#pragma unroll
                for (int i = 0; i < MF; ++i) {
                    const uint4 v = a[i][u >> 1];
                    const v8h ah = (u & 1) ? e4m3x8_to_f16x8(v.z, v.w) : e4m3x8_to_f16x8(v.x, v.y);
#pragma unroll
                    for (int j = 0; j < NF; ++j) acc[i][j] = mfma16_f16(ah, bh[j], acc[i][j]);
                }
            }
        }
    }

    // fixed-order cross-wave sum through LDS
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][(i * NF + j) * 4 + r][lane] = acc[i][j][r];
    __syncthreads();
    constexpr int kOut = MF * NF * 4 * 64;
    for (int e = threadIdx.x; e < kOut; e += 64 * NW) {
        const int v = e >> 6, l = e & 63;
        float sum = red[0][v][l];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += red[w][v][l];
        const int r = v & 3, ij = v >> 2, j = ij % NF, i = ij / NF;
        const int m = 16 * i + 4 * (l >> 4) + r, n = n0 + 16 * j + (l & 15);
        if (m < M && n < N) {
            if constexpr (FP8)
                sum = sum * reinterpret_cast<const float*>(sa_)[m] * reinterpret_cast<const float*>(sw_)[n];
            y[(int64_t)m * N + n] = (uint16_t)bf16_rne(sum);
        }
    }
}

// ============================================================================
// Tile path (large M, MFMA-bound).
// 256 x 256 output tile per workgroup of 4 waves (2 x 2, 128 x 128 each, 4 x 4
// fragments of 32 x 32).  Each K-stage moves 128 code bytes per row of both
// operands (K = 256 FP4 or 128 FP8) from global memory through registers into
// a padded LDS tile (row pitch 144 B keeps ds_read_b128 conflict-free), double
// buffered: the loads of stage s+1 are in flight while stage s computes.
// MFMA operand A is the weight tile (rows n), operand B the activation tile
// (rows m), so each lane ends up with 4 consecutive n of one m per register
// quad and writes 8-byte BF16 groups.
// ============================================================================
constexpr int kTileM = 256, kTileN = 256, kStageBytes = 128, kLdsPitch = 144;
constexpr int kTileLds = 2 * 2 * 256 * kLdsPitch;  // [buffer][operand][row][pitch]

__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
    // Workgroups are dealt to the 8 XCDs round-robin; renumber them so each XCD
    // owns a contiguous run of tiles, then walk that run in groups of 4 tile
    // rows so concurrently resident tiles share weight and activation panels
    // in the XCD's L2.
    const int T = tiles_m * tiles_n;
    const int T8 = T & ~7;
    const int L = b < T8 ? (b & 7) * (T8 >> 3) + (b >> 3) : b;
    constexpr int GM = 4;
    const int group = L / (GM * tiles_n);
    const int tm0 = group * GM;
    const int gsz = min(tiles_m - tm0, GM);
    const int rem = L - group * GM * tiles_n;
    tm = tm0 + rem % gsz;
    tn = rem / gsz;
}

template <bool FP8>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(const uint8_t* __restrict__ qa, const void* __restrict__ sa_,
                                                           const uint8_t* __restrict__ qw, const void* __restrict__ sw_,
                                                           uint16_t* __restrict__ y, int M, int N, int K, int tiles_m,
                                                           int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kTileLds];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kTileM, n0 = tn * kTileN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = FP8 ? (int64_t)K : (int64_t)K / 2;
    const int64_t KS = (int64_t)K / 32;
    const int nst = (int)((KB + kStageBytes - 1) / kStageBytes);

    // global -> LDS copy assignment: thread covers rows (tid>>3) + 32i, 16-byte column tid&7
    const int crow = tid >> 3, ccol = tid & 7;
    const uint8_t* wsrc[8];
    const uint8_t* xsrc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        wsrc[i] = qw + (int64_t)min(n0 + crow + 32 * i, N - 1) * KB + ccol * 16;
        xsrc[i] = qa + (int64_t)min(m0 + crow + 32 * i, M - 1) * KB + ccol * 16;
    }
    // FP4 scale rows of this lane's fragments
    const uint8_t* wsc[4];
    const uint8_t* xsc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        wsc[f] = reinterpret_cast<const uint8_t*>(sw_) + (int64_t)min(n0 + 128 * wn + 32 * f + l32, N - 1) * KS;
        xsc[f] = reinterpret_cast<const uint8_t*>(sa_) + (int64_t)min(m0 + 128 * wm + 32 * f + l32, M - 1) * KS;
    }

    uint4 pw[8], px[8];
    int psw[4], psx[4], csw[4], csx[4];

    auto gload = [&](int s) {
        const int64_t koff = (int64_t)s * kStageBytes;
        const bool kin = koff + ccol * 16 < KB;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pw[i] = kin ? ldg16(wsrc[i] + koff) : make_uint4(0, 0, 0, 0);
            px[i] = kin ? ldg16(xsrc[i] + koff) : make_uint4(0, 0, 0, 0);
        }
        if constexpr (!FP8) {
            const int64_t sidx = 8 * (int64_t)s + 4 * h;
            const bool sin = sidx < KS;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                psw[f] = sin ? ldg4(wsc[f] + sidx) : 0x7f7f7f7f;
                psx[f] = sin ? ldg4(xsc[f] + sidx) : 0x7f7f7f7f;
            }
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* wd = lds + (buf * 2 + 0) * 256 * kLdsPitch + crow * kLdsPitch + ccol * 16;
        uint8_t* xd = lds + (buf * 2 + 1) * 256 * kLdsPitch + crow * kLdsPitch + ccol * 16;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *reinterpret_cast<uint4*>(wd + 32 * i * kLdsPitch) = pw[i];
            *reinterpret_cast<uint4*>(xd + 32 * i * kLdsPitch) = px[i];
        }
        if constexpr (!FP8) {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                csw[f] = psw[f];
                csx[f] = psx[f];
            }
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int s = 0; s < nst; ++s) {
        const int cur = s & 1;
        if (s + 1 < nst) gload(s + 1);
        const uint8_t* wb = lds + (cur * 2 + 0) * 256 * kLdsPitch + (128 * wn + l32) * kLdsPitch;
        const uint8_t* xb = lds + (cur * 2 + 1) * 256 * kLdsPitch + (128 * wm + l32) * kLdsPitch;
        if constexpr (!FP8) {
            // lane group h holds bytes [64h, 64h+64) of the stage (blocks 4h..4h+3); MFMA t takes block 4h+t
#define MX_TILE_FP4_STEP(T)                                                                                     \
    {                                                                                                           \
        uint4 wa[4], xv[4];                                                                                     \
        _Pragma("unroll") for (int f = 0; f < 4; ++f) wa[f] =                                                  \
            *reinterpret_cast<const uint4*>(wb + 32 * f * kLdsPitch + 64 * h + 16 * (T));                      \
        _Pragma("unroll") for (int g = 0; g < 4; ++g) xv[g] =                                                  \
            *reinterpret_cast<const uint4*>(xb + 32 * g * kLdsPitch + 64 * h + 16 * (T));                      \
        _Pragma("unroll") for (int f = 0; f < 4; ++f) _Pragma("unroll") for (int g = 0; g < 4; ++g) acc[f][g] = \
            mfma32<kFmtFP4, (T)>(fp4_operand(wa[f]), fp4_operand(xv[g]), acc[f][g], csw[f], csx[g]);           \
    }
            MX_TILE_FP4_STEP(0)
            MX_TILE_FP4_STEP(1)
            MX_TILE_FP4_STEP(2)
            MX_TILE_FP4_STEP(3)
#undef MX_TILE_FP4_STEP
        } else {
            // FP8 codes are widened exactly to FP16 and run through 32x32x16 FP16 MFMAs.  Lane group
            // h holds bytes [64h, 64h+64) of the stage; sub-step t reads 16 of them (two operands).
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v8h wa[4][2], xv[4][2];
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const uint4 v = *reinterpret_cast<const uint4*>(wb + 32 * f * kLdsPitch + 64 * h + 16 * t);
                    wa[f][0] = e4m3x8_to_f16x8(v.x, v.y);
                    wa[f][1] = e4m3x8_to_f16x8(v.z, v.w);
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint4 v = *reinterpret_cast<const uint4*>(xb + 32 * g * kLdsPitch + 64 * h + 16 * t);
                    xv[g][0] = e4m3x8_to_f16x8(v.x, v.y);
                    xv[g][1] = e4m3x8_to_f16x8(v.z, v.w);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int f = 0; f < 4; ++f)
#pragma unroll
                        for (int g = 0; g < 4; ++g) acc[f][g] = mfma32_f16(wa[f][u], xv[g][u], acc[f][g]);
            }
        }
        if (s + 1 < nst) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds, per fragment (f, g) and j, Y[m][n .. n+3] with
    // m = m0 + 128wm + 32g + l32 and n = n0 + 128wn + 32f + 8j + 4h
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int m = m0 + 128 * wm + 32 * g + l32;
        if (m >= M) continue;
        float sxm = 1.f;
        if constexpr (FP8) sxm = reinterpret_cast<const float*>(sa_)[m];
        uint16_t* yrow = y + (int64_t)m * N;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + 128 * wn + 32 * f + 8 * j + 4 * h;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[f][g][4 * j + e];
                    if constexpr (FP8) v[e] = v[e] * sxm * reinterpret_cast<const float*>(sw_)[min(n + e, N - 1)];
                }
                if (vec_ok && n + 3 < N) {
                    uint2 pk;
                    pk.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
                    pk.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
                    *reinterpret_cast<uint2*>(yrow + n) = pk;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) yrow[n + e] = (uint16_t)bf16_rne(v[e]);
                }
            }
    }
}

// ----------------------------------------------------------------------------
// Host-side dispatch shared by the FP4 and FP8 entry points.
// ----------------------------------------------------------------------------
template <bool FP8>
inline hipError_t launch_gemm(const void* qa, const void* sa, const void* qw, const void* sw, void* y, int64_t M,
                              int64_t N, int64_t K, hipStream_t st) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    const int m = (int)M, n = (int)N, k = (int)K;
    if (M <= 128) {
        const dim3 grid((unsigned)((N + 31) / 32));
        if (M <= 16)
            hipLaunchKernelGGL((gemm_decode_kernel<FP8, 1, 8>), grid, dim3(512), 0, st, a, sa, w, sw, out, m, n, k);
        else if (M <= 32)
            hipLaunchKernelGGL((gemm_decode_kernel<FP8, 2, 8>), grid, dim3(512), 0, st, a, sa, w, sw, out, m, n, k);
        else if (M <= 64)
            hipLaunchKernelGGL((gemm_decode_kernel<FP8, 4, 8>), grid, dim3(512), 0, st, a, sa, w, sw, out, m, n, k);
        else
            hipLaunchKernelGGL((gemm_decode_kernel<FP8, 8, 4>), grid, dim3(256), 0, st, a, sa, w, sw, out, m, n, k);
    } else {
        const int tiles_m = (int)((M + kTileM - 1) / kTileM), tiles_n = (int)((N + kTileN - 1) / kTileN);
        hipLaunchKernelGGL((gemm_tile_kernel<FP8>), dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, a, sa, w,
                           sw, out, m, n, k, tiles_m, tiles_n);
    }
    return hipGetLastError();
}

}  // namespace mx
