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
//     FP16 MFMAs; the epilogue multiplies by sA[m] * sW[n] in FP64.  (gfx950's FP8
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

#include "gemm_splitk.hpp"
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
                sum = ptpc_scaled(sum, reinterpret_cast<const float*>(sa_)[m], reinterpret_cast<const float*>(sw_)[n]);
            y[(int64_t)m * N + n] = (uint16_t)bf16_rne(sum);
        }
    }
}

// ============================================================================
// Decode path, LDS-staged (FP4, K % 512 == 0).
// One workgroup (4 waves) per 32 output columns.  A stage is a 512-K slab of
// the workgroup's operands: the 32 weight rows and the 16*MF activation rows,
// 256 code bytes each, plus their 16 scale bytes.  Each wave instruction loads
// 1 KB = 4 rows x 256 contiguous bytes (fully coalesced); kInFlight stages of
// loads are kept in registers, each is written to a double-buffered LDS tile
// just before it is consumed.  In LDS the 16-byte chunks of a row are XOR-
// swizzled by (row % 16), so the MFMA-layout ds_read_b128 (16 rows, same
// logical chunk) touches 16 distinct bank groups.  Wave w multiplies chunk w
// (128 K) of every slab; the four partial tiles are summed through LDS in a
// fixed order at the end (deterministic).
// ============================================================================
template <int MF>
struct DecodeLds {
    static constexpr int kNT = 32;                      // output columns per workgroup
    static constexpr int kSlab = 256;                   // code bytes per row per stage
    static constexpr int kRows = kNT + 16 * MF;         // weight rows, then activation rows
    static constexpr int kCode = kRows * kSlab;
    static constexpr int kStage = kCode + kRows * 16;   // + 16 scale bytes per row
    static constexpr int kCodeLoads = kRows / 16;       // 16-byte loads per lane per stage
    static constexpr int kScaleRows = kRows / 4;        // scale rows loaded per wave
    static constexpr int kInFlight = 3;                 // stages of loads in registers
    static_assert(kRows % 16 == 0 && kScaleRows <= 64, "stage shape");
    static_assert((kStage % 256) == 0, "stage alignment");
};

template <int MF>
struct DecodeRegs {
    uint4 code[DecodeLds<MF>::kCodeLoads];
    uint4 scale;
};

// LDS bytes of the kernel: two stages, or the four waves' partial tiles for the final sum
template <int MF>
constexpr int decode_lds_bytes() {
    constexpr int V = MF * 2 * 4;
    return 2 * DecodeLds<MF>::kStage > 4 * V * 64 * 4 ? 2 * DecodeLds<MF>::kStage : 4 * V * 64 * 4;
}

// One workgroup's work: the 32 output columns of blockIdx.x for rows 0 .. M - 1 (M <= 16 MF) of qa / sa / y,
// with the workgroup's LDS block.
template <int MF>
__device__ __forceinline__ void decode_lds_rows(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                uint16_t* __restrict__ y, int M, int N, int K, uint8_t* lds) {
    using C = DecodeLds<MF>;
    constexpr int NF = 2;
    constexpr int V = MF * NF * 4;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * C::kNT;
    const int64_t KB = (int64_t)K / 2, KS = (int64_t)K / 32;
    const int nslab = K / 512;

    // load i of this lane covers row group g (4 rows): the first kWLoads loads of every wave
    // are weight rows (streamed once: non-temporal, so they do not push the shared
    // activations out of L2), the rest activation rows; lane -> row 4g + lane/16,
    // logical chunk lane%16
    constexpr int kWLoads = C::kNT / 16;
    const uint8_t* src[C::kCodeLoads];
    int dst[C::kCodeLoads];
#pragma unroll
    for (int i = 0; i < C::kCodeLoads; ++i) {
        const int g = i < kWLoads ? wave * kWLoads + i : C::kNT / 4 + wave * (C::kCodeLoads - kWLoads) + (i - kWLoads);
        const int rho = 4 * g + (lane >> 4);
        const uint8_t* row = rho < C::kNT ? qw + (int64_t)min(n0 + rho, N - 1) * KB
                                          : qa + (int64_t)min(rho - C::kNT, M - 1) * KB;
        src[i] = row + 16 * (lane & 15);
        dst[i] = rho * C::kSlab + 16 * ((lane & 15) ^ (rho & 15));
    }
    // scale load: lane < kScaleRows fetches the 16 scale bytes of row wave*kScaleRows + lane;
    // the other lanes repeat the last row's load (never stashed), so the load is issued
    // unconditionally and the compiler's vmcnt bookkeeping stays exact
    const bool s_on = lane < C::kScaleRows;
    const int srho = wave * C::kScaleRows + (s_on ? lane : C::kScaleRows - 1);
    const uint8_t* ssrc = srho < C::kNT ? sw + (int64_t)min(n0 + srho, N - 1) * KS
                                        : sa + (int64_t)min(srho - C::kNT, M - 1) * KS;

    auto fetch = [&](DecodeRegs<MF>& r, int s) {
#pragma unroll
        for (int i = 0; i < C::kCodeLoads; ++i)
            r.code[i] = i < kWLoads ? ldg16_stream(src[i] + (int64_t)s * C::kSlab) : ldg16(src[i] + (int64_t)s * C::kSlab);
        r.scale = ldg16(ssrc + (int64_t)s * 16);
    };
    auto stash = [&](const DecodeRegs<MF>& r, int buf) {
        uint8_t* st = lds + buf * C::kStage;
#pragma unroll
        for (int i = 0; i < C::kCodeLoads; ++i) *reinterpret_cast<uint4*>(st + dst[i]) = r.code[i];
        if (s_on) *reinterpret_cast<uint4*>(st + C::kCode + srho * 16) = r.scale;
    };

    v4f acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // this lane's physical chunk in every row it reads: logical chunk 4*wave + q, swizzled
    const int pchunk = (4 * wave + q) ^ r16;
    auto consume = [&](int buf) {
        const uint8_t* st = lds + buf * C::kStage;
        uint4 wv[NF];
        int wsc[NF];
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int rho = 16 * j + r16;
            wv[j] = *reinterpret_cast<const uint4*>(st + rho * C::kSlab + 16 * pchunk);
            wsc[j] = st[C::kCode + rho * 16 + 4 * wave + q];
        }
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            const int rho = C::kNT + 16 * i + r16;
            const uint4 av = *reinterpret_cast<const uint4*>(st + rho * C::kSlab + 16 * pchunk);
            const int asc = st[C::kCode + rho * 16 + 4 * wave + q];
#pragma unroll
            for (int j = 0; j < NF; ++j)
                acc[i][j] = mfma16<kFmtFP4, 0>(fp4_operand(av), fp4_operand(wv[j]), acc[i][j], asc, wsc[j]);
        }
    };

    // Stage s: stash its registers into LDS buffer s%2, barrier (which also retires the
    // reads of that buffer from stage s-2), refill the registers with stage s+3, multiply.
    // The steady-state loop fetches unconditionally, so the compiler's vmcnt bookkeeping
    // stays exact (each stash waits only for its own stage); the tail is peeled.
    DecodeRegs<MF> r0, r1, r2;
    fetch(r0, 0);
    fetch(r1, min(1, nslab - 1));  // unconditional (a short K re-reads its last slab)
    fetch(r2, min(2, nslab - 1));
    int s = 0;
    for (; s + 5 < nslab; s += 3) {
        stash(r0, s & 1);
        __syncthreads();
        fetch(r0, s + 3);
        consume(s & 1);
        stash(r1, (s + 1) & 1);
        __syncthreads();
        fetch(r1, s + 4);
        consume((s + 1) & 1);
        stash(r2, s & 1);
        __syncthreads();
        fetch(r2, s + 5);
        consume(s & 1);
    }
    // tail: stages s .. nslab-1 (at most 5); r0, r1, r2 hold stages s, s+1, s+2 where they exist
    for (int t = 0; s + t < nslab; t += 3) {
        const int a = s + t;
        stash(r0, a & 1);
        __syncthreads();
        if (a + 3 < nslab) fetch(r0, a + 3);
        consume(a & 1);
        if (a + 1 >= nslab) break;
        stash(r1, (a + 1) & 1);
        __syncthreads();
        if (a + 4 < nslab) fetch(r1, a + 4);
        consume((a + 1) & 1);
        if (a + 2 >= nslab) break;
        stash(r2, a & 1);
        __syncthreads();
        consume(a & 1);
    }

    // fixed-order sum of the four waves' partial tiles
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(wave * V + (i * NF + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    __syncthreads();
    for (int e = threadIdx.x; e < V * 64; e += 256) {
        const int v = e >> 6, l = e & 63;
        const float sum = ((red[v * 64 + l] + red[(V + v) * 64 + l]) + red[(2 * V + v) * 64 + l]) + red[(3 * V + v) * 64 + l];
        const int r = v & 3, ij = v >> 2, j = ij % NF, i = ij / NF;
        const int m = 16 * i + 4 * (l >> 4) + r, n = n0 + 16 * j + (l & 15);
        if (m < M && n < N) y[(int64_t)m * N + n] = (uint16_t)bf16_rne(sum);
    }
}

// GROUPED (MoE experts, grid.y = expert e): the rows goff[e] .. goff[e+1] - 1 of the packed activations with
// weight e of the stacked weights ([G, N, K/2] codes, [G, N, K/32] scales) into the same rows of y, in chunks
// of 16 MF rows (a barrier between chunks, which reuse the LDS block), so every row of every group is
// written; an empty group's workgroups return before their first barrier.  Otherwise M rows (M <= 16 MF).
template <int MF, bool GROUPED = false>
__global__ __launch_bounds__(256) void gemm_decode_lds_fp4(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                           const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                           uint16_t* __restrict__ y, int M, int N, int K,
                                                           const int32_t* __restrict__ goff) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[decode_lds_bytes<MF>()];
    if constexpr (GROUPED) {
        const int e = blockIdx.y;
        const int r0 = __builtin_amdgcn_readfirstlane(goff[e]);
        const int rows = __builtin_amdgcn_readfirstlane(goff[e + 1]) - r0;  // uniform over the workgroup
        if (rows <= 0) return;  // the whole workgroup, before any barrier
        const int64_t KB = (int64_t)K / 2, KS = (int64_t)K / 32;
        qw += (int64_t)e * N * KB;
        sw += (int64_t)e * N * KS;
        for (int c = 0; c < rows; c += 16 * MF) {
            if (c > 0) __syncthreads();  // every wave has read the previous chunk's partial tiles
            const int64_t r = (int64_t)r0 + c;
            decode_lds_rows<MF>(qa + r * KB, sa + r * KS, qw, sw, y + r * N, min(rows - c, 16 * MF), N, K, lds);
        }
    } else {
        decode_lds_rows<MF>(qa, sa, qw, sw, y, M, N, K, lds);
    }
}

// ============================================================================
// Decode path, per-wave LDS rings (FP4, M <= 64, K % 2048 == 0, K <= 16384,
// 16-byte aligned scale rows; M <= 128 and K <= 8192 with two row halves).
// One workgroup (4 waves) per 32 output columns.  A slab is K = 256 of the
// 32*MF activation rows and the 32 weight rows: 128 code bytes per row, copied
// global -> LDS (global_load_lds) 8 whole rows (whole cache lines) per wave
// instruction.  Wave w owns the w-th quarter of K (nmine = K / 1024
// consecutive slabs, an even count) and a private ring of S slab slots, so it
// waits only for its own copies.  The workgroup's scale rows (K/32 bytes each:
// 64 activation rows, then 32 weight rows, contiguous in memory) are copied
// once, up front, as whole lines into one shared block; after that single
// barrier no wave waits for another until the end, when the four partial
// tiles are summed through LDS in a fixed order (deterministic).  With two
// row halves (RH = 2, M <= 128) waves 2h and 2h+1 share K half h, each with
// its own 64 activation rows, and two partial tiles meet per output.
// MFMA: 32 x 32 x 64, operand A = 32 weight rows (n), operand B = 32
// activation rows (m); k-step t of a slab uses the row's chunks 4h + t in lane
// group h (the K-permutation of the tile path; chunks are XOR-swizzled by
// (row % 8) ^ ((row / 8) % 2), conflict-free for the MFMA-layout reads), so
// one scale dword per row and slab serves all four k-steps.  In the
// scale block, row r's 16-byte pieces are rotated by r (position p holds piece
// (p + r) mod P), which spreads the 32 rows of a fragment over the LDS banks.
// ============================================================================
namespace dec4 {
constexpr int kNT = 32;             // output columns per workgroup
constexpr int kSlab = 128;          // code bytes per row per slab (K = 256)
constexpr int kMaxMine = 16;        // slabs per wave supported (K <= 16384)
// KSMAX: scale bytes per row the shared block holds (256: K <= 8192, 512: K <= 16384)
// RH: row halves.  RH = 1: wave w owns K quarter w of all 32 MF activation rows.  RH = 2: wave w
// owns K half w / 2 of activation rows 32 MF (w % 2) .. 32 MF (w % 2) + 32 MF - 1, so a slab still
// holds 32 MF activation rows and the workgroup covers 64 MF rows (both waves of a K half copy
// the same weight rows; the second copy is mostly an L2 hit).
template <int MF, int S, int KSMAX, int RH = 1>
struct Cfg {
    static constexpr int kArows = 32 * MF;                   // activation rows per slab
    static constexpr int kRows = kArows + kNT;              // activation rows, then weight rows
    static constexpr int kSlabBytes = kRows * kSlab;         // 12 KB (MF = 2) or 8 KB
    static constexpr int kCopies = kSlabBytes / 1024;        // copies per wave per slab
    static constexpr int kScArows = RH * kArows;             // activation rows of the workgroup
    static constexpr int kScRows = kScArows + kNT;           // rows of the shared scale block
    static constexpr int kScBytes = kScRows * KSMAX;         // shared scale block
    static constexpr int kScCopies = kScBytes / 1024 / 4;    // scale copies per wave
    static constexpr int kRing = 4 * S * kSlabBytes;
    static constexpr int kLds = kRing + kScBytes;
    static_assert(kScCopies * 4096 == kScBytes, "scale copies");
    static_assert(kScCopies + S * kCopies <= 63, "vmcnt");
    static_assert(kLds <= 160 * 1024, "LDS");
    static_assert(4 * MF * 16 * 64 * 4 <= kLds, "reduction staging");
    static_assert(RH == 1 || RH == 2, "row halves");
};
}  // namespace dec4

// The decode ring's work on one set of at most 32 MF RH activation rows (M of them) and the workgroup's
// 32 columns, in the workgroup's LDS block (the kernel below).
template <int MF, int S, int KSMAX, int RH>
__device__ __forceinline__ void decode_fp4_rows(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                uint16_t* __restrict__ y, int M, int N, int K, uint8_t* lds) {
    using C = dec4::Cfg<MF, S, KSMAX, RH>;
    using namespace dec4;
    const int n0 = blockIdx.x * kNT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = (int64_t)K / 2;
    const int KS = K / 32;                  // scale bytes per row
    const int kq = wave / RH, rh = wave % RH;  // K part and row half of this wave
    const int nmine = K * RH / 1024;        // slabs per wave (even)
    const int s0 = kq * nmine;              // first slab of this wave
    const int ra = rh * C::kArows;          // first activation row of this wave
    uint8_t* const ring = lds + wave * S * C::kSlabBytes;
    uint8_t* const scb = lds + C::kRing;

    // 1. the workgroup's scale rows, whole: P = K / 512 pieces of 16 bytes per row; piece q = 64 c +
    //    lane of copy c (wave w issues c = w kScCopies + e) is position q mod P of row q / P, which
    //    holds piece (position + row) mod P.  Pieces past the data read one address (never used).
    const int P = KS / 16;
#pragma unroll
    for (int e = 0; e < C::kScCopies; ++e) {
        const int c = wave * C::kScCopies + e;
        const int q = 64 * c + lane;
        const int r = q / P, p = q - r * P;
        const uint8_t* src = sa;
        if (r < C::kScRows) {
            const int64_t off = 16 * ((p + r) % P);
            src = r < C::kScArows ? sa + (int64_t)min(r, M - 1) * KS + off
                                  : sw + (int64_t)min(n0 + r - C::kScArows, N - 1) * KS + off;
        }
        g2lds16(src, scb + 1024 * c);
    }
    // 2. code copies: copy i moves rows 8i .. 8i+7 (lane / 8) of the slab, the lane filling chunk
    //    lane % 8 with logical chunk (lane % 8) ^ swz(row), swz(r) = (r % 8) ^ ((r / 8) % 2): any 8
    //    consecutive rows get 8 distinct chunks, so the 8 lanes an LDS cycle serves of a
    //    ds_read_b128 (32 four-byte banks) hit distinct banks, and so do 16 lanes over 64 banks.
    //    An activation copy whose 8 rows all lie at or past M reads one address in every lane (one
    //    cache line): those rows only
    //    feed output columns that are never stored.  Every wave issues the same copies (its nmine
    //    slabs, each in one batch), so the wait counts below are fixed.
    const uint8_t* rowp[C::kCopies];
#pragma unroll
    for (int i = 0; i < C::kCopies; ++i) {
        const int r = 8 * i + (lane >> 3);
        const int chunk = (lane & 7) ^ ((r & 7) ^ ((r >> 3) & 1));
        if (r < C::kArows)
            rowp[i] = ra + 8 * i < M ? qa + (int64_t)min(ra + r, M - 1) * KB + 16 * chunk : qa;
        else
            rowp[i] = qw + (int64_t)min(n0 + r - C::kArows, N - 1) * KB + 16 * chunk;
    }
    auto issue = [&](int j) {  // slab s0 + j into slot j % S
        uint8_t* slot = ring + (j % S) * C::kSlabBytes;
        const bool real = j < nmine;
        const int64_t koff = (int64_t)(s0 + (real ? j : 0)) * kSlab;
#pragma unroll
        for (int i = 0; i < C::kCopies; ++i) {
            const uint8_t* src = real ? rowp[i] + koff : qw;
            if (8 * i < C::kArows) g2lds16(src, slot + 1024 * i);    // activations: reused by every CU
            else g2lds16_nt(src, slot + 1024 * i);                   // weights: streamed once
        }
    };
#pragma unroll
    for (int j = 0; j < S; ++j) issue(j);
    wait_vmcnt<S * C::kCopies>();  // this wave's scale copies have landed (its slabs may not have)
    __builtin_amdgcn_s_barrier();  // and every other wave's

    // per-lane LDS offsets (rows: activation fragment g = 32 g + l32, weight rows kArows + l32)
    const uint32_t rbase = lds_addr(ring), sbase = lds_addr(scb);
    int xoff[MF], xsw[MF], xsr[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g) {
        const int r = 32 * g + l32;
        xoff[g] = r * kSlab;
        xsw[g] = (r & 7) ^ ((r >> 3) & 1);
        xsr[g] = ra + r;  // row of the scale block
    }
    const int wr = C::kArows + l32, wsr = C::kScArows + l32;
    const int woff = wr * kSlab, wsw = (wr & 7) ^ ((wr >> 3) & 1);
    auto scale_at = [&](int r, int j) -> uint32_t {  // dword of row r for local slab j, lane group h
        const int s = s0 + j;                            // slab index in K: bytes 8 s .. 8 s + 7 of the row
        int p = (s >> 1) - r % P;
        if (p < 0) p += P;
        return lds_read4(sbase + r * KS + 16 * p + 8 * (s & 1) + 4 * h);
    };

    v16f acc[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[g][r] = 0.f;

    // slab j; WAIT: the copies that may still be in flight (the later batches), REFILL: copy slab
    // j + S into the slot once it is read.  The last S slabs refill nothing, so no wave waits for
    // copies past its end before the reduction.  nmine >= S for every launch: K % 2048 == 0 gives
    // nmine >= 2, and S = 4 runs only for K > 8192.
    auto slab = [&](int j, auto WAIT, auto REFILL) __attribute__((always_inline)) {
        // slab j (and, for j = 0, the scale block) has landed once only the later batches may
        // still be in flight
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<decltype(WAIT)::value>();
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t sb = rbase + (j % S) * C::kSlabBytes;
        uint32_t ws = scale_at(wsr, j);
        uint32_t xs[MF];
#pragma unroll
        for (int g = 0; g < MF; ++g) xs[g] = scale_at(xsr[g], j);
        v4u wv[4], xv[4][MF];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            wv[t] = lds_read16(sb + woff + 16 * ((4 * h + t) ^ wsw));
#pragma unroll
            for (int g = 0; g < MF; ++g) xv[t][g] = lds_read16(sb + xoff[g] + 16 * ((4 * h + t) ^ xsw[g]));
        }
        lds_wait_dec<MF>(wv, xv, ws, xs);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(REFILL)::value) issue(j + S);  // the slot is read: refill it
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < MF; ++g) {
            acc[g] = mfma32<kFmtFP4, 0>(fp4_operand(wv[0]), fp4_operand(xv[0][g]), acc[g], (int)ws, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 1>(fp4_operand(wv[1]), fp4_operand(xv[1][g]), acc[g], (int)ws, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 2>(fp4_operand(wv[2]), fp4_operand(xv[2][g]), acc[g], (int)ws, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 3>(fp4_operand(wv[3]), fp4_operand(xv[3][g]), acc[g], (int)ws, (int)xs[g]);
        }
    };
    for (int j = 0; j < nmine - S; ++j)
        slab(j, std::integral_constant<int, (S - 1) * C::kCopies>{}, std::true_type{});
    static_for<S>([&](auto t) {
        slab(nmine - S + decltype(t)::value, std::integral_constant<int, (S - 1 - decltype(t)::value) * C::kCopies>{},
             std::false_type{});
    });

    // 3. fixed-order reduction of the partial tiles (four per output, or two with RH = 2) through LDS
    wait_vmcnt<0>();  // the trailing refills
    __syncthreads();  // every wave is done with its ring and scale block
    float* red = reinterpret_cast<float*>(lds);  // [wave][g][reg][lane]
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave * MF + g) * 16 + r) * 64 + lane] = acc[g][r];
    __syncthreads();
    // wave w finalizes register quad w of every fragment of every row half: D rows (n) 8w + 4h + e,
    // column (m) l32; the partials of K parts 0, 1, ... are added in that order
    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
#pragma unroll
    for (int fg = 0; fg < RH * MF; ++fg) {
        const int half = fg / MF, g = fg % MF;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * wave + e;
            float t = red[((half * MF + g) * 16 + r) * 64 + lane];
#pragma unroll
            for (int q = 1; q < 4 / RH; ++q) t += red[(((q * RH + half) * MF + g) * 16 + r) * 64 + lane];
            v[e] = t;
        }
        const int m = half * C::kArows + 32 * g + l32;
        const int n = n0 + 8 * wave + 4 * h;
        if (m >= M) continue;
        uint16_t* dst = y + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
            uint2 pk;
            pk.x = bf16x2_rne(v[0], v[1]);
            pk.y = bf16x2_rne(v[2], v[3]);
            *reinterpret_cast<uint2*>(dst) = pk;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = (uint16_t)(bf16x2_rne(v[e], 0.f) & 0xffffu);
        }
    }
}

// GROUPED: grid.y indexes groups (MoE experts).  Group e multiplies rows goff[e] .. goff[e+1]-1
// of the packed activations with weight e of the stacked weights ([G, N, K/2] codes, [G, N, K/32]
// scales) into the same rows of y.  The workgroup takes the group's rows in chunks of 32 MF (a
// barrier between chunks, which reuse the LDS block), so every row of every group is written whatever
// bound the caller passed; an empty group's workgroups return before their first barrier.
template <int MF, int S, int KSMAX, bool GROUPED = false, int RH = 1>
__global__ __launch_bounds__(256, 1) void gemm_decode_fp4(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                          const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                          uint16_t* __restrict__ y, int M, int N, int K,
                                                          const int32_t* __restrict__ goff) {
    using C = dec4::Cfg<MF, S, KSMAX, RH>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];
    if constexpr (GROUPED) {
        const int e = blockIdx.y;
        const int r0 = __builtin_amdgcn_readfirstlane(goff[e]);
        const int rows = __builtin_amdgcn_readfirstlane(goff[e + 1]) - r0;  // uniform over the workgroup
        if (rows <= 0) return;  // the whole workgroup, before any barrier
        qw += (int64_t)e * N * (K / 2);
        sw += (int64_t)e * N * (K / 32);
        for (int c = 0; c < rows; c += C::kScArows) {
            if (c > 0) __syncthreads();  // every wave has read the previous chunk's reduction staging
            const int64_t r = (int64_t)r0 + c;
            decode_fp4_rows<MF, S, KSMAX, RH>(qa + r * (K / 2), sa + r * (K / 32), qw, sw, y + r * N,
                                              min(rows - c, C::kScArows), N, K, lds);
        }
    } else {
        decode_fp4_rows<MF, S, KSMAX, RH>(qa, sa, qw, sw, y, M, N, K, lds);
    }
}

// ============================================================================
// Decode path, FP8 (E4M3 codes, FP32 per-row scales; M <= 64, K % 512 == 0;
// M <= 128 with two row halves, as in the FP4 decode kernel).
// The FP4 decode design above on byte codes: one workgroup (4 waves) per 32
// output columns, wave w owns a quarter of K and streams its K = 128 slabs
// (128 code bytes per row: the 32*MF activation rows, then the 32 weight rows)
// into a private ring of S slots with whole-line global -> LDS copies, waiting
// only for its own copies.  There are no block scales, so the ring is deeper.
// Each 16-byte chunk a lane reads is widened exactly to two 8 x FP16 MFMA
// operands (every E4M3 value is an FP16 normal) for v_mfma_f32_32x32x16_f16:
// lane group h takes chunks 4h .. 4h+3, chunk 4h+t half u feeding k-step
// (t, u) of both operands.  The four partial tiles are summed through LDS in a
// fixed order; the epilogue applies sum * sA[m] * sW[n] (in FP64) and rounds to BF16.
// ============================================================================
namespace dec8 {
constexpr int kNT = 32;             // output columns per workgroup
constexpr int kSlab = 128;          // code bytes per row per slab (K = 128)
// RH: row halves, as in the FP4 decode kernel (RH = 2: waves 2h and 2h+1 share K half h, each with
// its own 32 MF activation rows)
template <int MF, int S, int RH = 1>
struct Cfg {
    static constexpr int kArows = 32 * MF;
    static constexpr int kRows = kArows + kNT;              // activation rows, then weight rows
    static constexpr int kSlabBytes = kRows * kSlab;         // 12 KB (MF = 2) or 8 KB
    static constexpr int kCopies = kSlabBytes / 1024;        // copies per wave per slab
    static constexpr int kLds = 4 * S * kSlabBytes;
    static_assert(S * kCopies <= 63, "vmcnt");
    static_assert(kLds <= 160 * 1024, "LDS");
    static_assert(4 * MF * 16 * 64 * 4 <= kLds, "reduction staging");
    static_assert(RH == 1 || RH == 2, "row halves");
};
}  // namespace dec8

template <int MF, int S, int RH = 1>
__global__ __launch_bounds__(256, 1) void gemm_decode_fp8(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                          const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                          uint16_t* __restrict__ y, int M, int N, int K) {
    using C = dec8::Cfg<MF, S, RH>;
    using namespace dec8;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];
    const int n0 = blockIdx.x * kNT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int kq = wave / RH, rh = wave % RH;  // K part and row half of this wave
    const int nmine = K * RH / 512;         // slabs per wave
    const int s0 = kq * nmine;              // first slab of this wave
    const int ra = rh * C::kArows;          // first activation row of this wave
    uint8_t* const ring = lds + wave * S * C::kSlabBytes;

    // code copies: copy i moves rows 8i .. 8i+7 (lane / 8) of the slab, the lane filling chunk
    // lane % 8 with logical chunk (lane % 8) ^ (row % 8) ^ ((row / 8) % 2) (the conflict-free swizzle
    // of gemm_decode_fp4).  An activation copy whose 8 rows
    // all lie at or past M reads one address in every lane (one cache line): those rows only feed
    // outputs that are never stored.  A batch for a slab past the wave's last one also reads a
    // single address, so every wave issues the same number of copies and the waits are fixed.
    const uint8_t* rowp[C::kCopies];
#pragma unroll
    for (int i = 0; i < C::kCopies; ++i) {
        const int r = 8 * i + (lane >> 3);
        const int chunk = (lane & 7) ^ ((r & 7) ^ ((r >> 3) & 1));
        if (r < C::kArows)
            rowp[i] = ra + 8 * i < M ? qa + (int64_t)min(ra + r, M - 1) * K + 16 * chunk : qa;
        else
            rowp[i] = qw + (int64_t)min(n0 + r - C::kArows, N - 1) * K + 16 * chunk;
    }
    auto issue = [&](int j) {  // slab s0 + j into slot j % S
        uint8_t* slot = ring + (j % S) * C::kSlabBytes;
        const bool real = j < nmine;
        const int64_t koff = (int64_t)(s0 + (real ? j : 0)) * kSlab;
#pragma unroll
        for (int i = 0; i < C::kCopies; ++i) {
            const uint8_t* src = real ? rowp[i] + koff : qw;
            if (8 * i < C::kArows) g2lds16(src, slot + 1024 * i);    // activations: reused by every CU
            else g2lds16_nt(src, slot + 1024 * i);                   // weights: streamed once
        }
    };
#pragma unroll
    for (int j = 0; j < S; ++j) issue(j);

    const uint32_t rbase = lds_addr(ring);
    int xoff[MF], xsw[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g) {
        const int r = 32 * g + l32;
        xoff[g] = r * kSlab;
        xsw[g] = (r & 7) ^ ((r >> 3) & 1);
    }
    const int wr = C::kArows + l32;
    const int woff = wr * kSlab, wsw = (wr & 7) ^ ((wr >> 3) & 1);

    v16f acc[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[g][r] = 0.f;

    // slab j; WAIT: the copies that may still be in flight, REFILL: copy slab j + S into the slot
    // once it is read.  The last S slabs refill nothing, so the waits before the reduction find no
    // copies past the end in flight, except when a wave has fewer slabs than slots (small K): the
    // prologue's batches past the end then stay, the tail skips the missing slabs, and the waits
    // it keeps count at most those batches too many (they only wait longer).
    auto slab = [&](int j, auto WAIT, auto REFILL) __attribute__((always_inline)) {
        // slab j has landed once only the later batches may still be in flight
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<decltype(WAIT)::value>();
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t sb = rbase + (j % S) * C::kSlabBytes;
        v4u wv[4], xv[4][MF];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            wv[t] = lds_read16(sb + woff + 16 * ((4 * h + t) ^ wsw));
#pragma unroll
            for (int g = 0; g < MF; ++g) xv[t][g] = lds_read16(sb + xoff[g] + 16 * ((4 * h + t) ^ xsw[g]));
        }
        lds_wait_codes<MF>(wv, xv);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(REFILL)::value) issue(j + S);  // the slot is read: refill it
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v8h w0 = e4m3x8_to_f16x8(wv[t][0], wv[t][1]);
            const v8h w1 = e4m3x8_to_f16x8(wv[t][2], wv[t][3]);
#pragma unroll
            for (int g = 0; g < MF; ++g) {
                acc[g] = mfma32_f16(w0, e4m3x8_to_f16x8(xv[t][g][0], xv[t][g][1]), acc[g]);
                acc[g] = mfma32_f16(w1, e4m3x8_to_f16x8(xv[t][g][2], xv[t][g][3]), acc[g]);
            }
        }
    };
    for (int j = 0; j < nmine - S; ++j)
        slab(j, std::integral_constant<int, (S - 1) * C::kCopies>{}, std::true_type{});
    static_for<S>([&](auto t) {
        const int j = nmine - S + decltype(t)::value;
        if (j >= 0)
            slab(j, std::integral_constant<int, (S - 1 - decltype(t)::value) * C::kCopies>{}, std::false_type{});
    });

    // fixed-order reduction of the four partial tiles through LDS, then the row and column scales
    wait_vmcnt<0>();  // the trailing refills
    __syncthreads();  // every wave is done with its ring
    float* red = reinterpret_cast<float*>(lds);  // [wave][g][reg][lane]
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave * MF + g) * 16 + r) * 64 + lane] = acc[g][r];
    __syncthreads();
    // wave w finalizes register quad w of every fragment of every row half: D rows (n) 8w + 4h + e,
    // column (m) l32; the partials of K parts 0, 1, ... are added in that order
    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
    const int n = n0 + 8 * wave + 4 * h;
    float swn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) swn[e] = sw[min(n + e, N - 1)];
#pragma unroll
    for (int fg = 0; fg < RH * MF; ++fg) {
        const int half = fg / MF, g = fg % MF;
        const int m = half * C::kArows + 32 * g + l32;
        if (m >= M) continue;
        const float sam = sa[m];
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * wave + e;
            float t = red[((half * MF + g) * 16 + r) * 64 + lane];
#pragma unroll
            for (int q = 1; q < 4 / RH; ++q) t += red[(((q * RH + half) * MF + g) * 16 + r) * 64 + lane];
            v[e] = ptpc_scaled(t, sam, swn[e]);
        }
        uint16_t* dst = y + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
            uint2 pk;
            pk.x = bf16x2_rne(v[0], v[1]);
            pk.y = bf16x2_rne(v[2], v[3]);
            *reinterpret_cast<uint2*>(dst) = pk;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = (uint16_t)(bf16x2_rne(v[e], 0.f) & 0xffffu);
        }
    }
}

// ============================================================================
// Tile path (large M, MFMA-bound).
// 256 x 256 output tile per workgroup of 4 waves (2 x 2, 128 x 128 each, 4 x 4
// fragments of 32 x 32).  gemm_tile_kernel (FP4, the fallback for K % 256 != 0):
// each K-stage moves 128 code bytes per row of both operands (K = 256) from global memory through registers into
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

// VEC8: N % 4 == 0 and y 8-byte aligned (whole 8-byte output stores allowed).
template <bool VEC8>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                           const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                           uint16_t* __restrict__ y, int M, int N, int K, int tiles_m,
                                                           int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kTileLds];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kTileM, n0 = tn * kTileN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = (int64_t)K / 2;
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
    // scale rows of this lane's fragments
    const uint8_t* wsc[4];
    const uint8_t* xsc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        wsc[f] = sw + (int64_t)min(n0 + 128 * wn + 32 * f + l32, N - 1) * KS;
        xsc[f] = sa + (int64_t)min(m0 + 128 * wm + 32 * f + l32, M - 1) * KS;
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
        const int64_t sidx = 8 * (int64_t)s + 4 * h;
        const bool sin = sidx < KS;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            psw[f] = sin ? ldg4(wsc[f] + sidx) : 0x7f7f7f7f;
            psx[f] = sin ? ldg4(xsc[f] + sidx) : 0x7f7f7f7f;
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
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            csw[f] = psw[f];
            csx[f] = psx[f];
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
        if (s + 1 < nst) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds, per fragment (f, g) and j, Y[m][n .. n+3] with
    // m = m0 + 128wm + 32g + l32 and n = n0 + 128wn + 32f + 8j + 4h
    constexpr bool vec_ok = VEC8;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int m = m0 + 128 * wm + 32 * g + l32;
        if (m >= M) continue;
        uint16_t* yrow = y + (int64_t)m * N;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + 128 * wn + 32 * f + 8 * j + 4 * h;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[f][g][4 * j + e];
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

// ============================================================================
// Tile path, DMA-staged (FP4, K % 256 == 0).
// 256 x 256 output tile, 4 waves (2 x 2, 128 x 128 each, 4 x 4 fragments of
// 32 x 32).  A stage is K = 128 (64 code bytes per row) of both operands plus
// their scale dwords; stages are copied global -> LDS with global_load_lds
// (1 KB per wave instruction = 16 rows x 64 bytes, coalesced; 4-byte scale
// DMAs) into a ring of STAGES buffers, so STAGES - 1 stages are in flight while one is
// multiplied and no VGPRs are spent on staging (all 256 accumulators stay in
// AGPRs).  In LDS a row's four 16-byte chunks are XOR-swizzled by (row/4)%4,
// which spreads the 32 rows of an MFMA-layout ds_read_b128 over all banks.
// The LDS reads are inline asm and every wait is explicit: per wave vmcnt for
// its own DMAs of the stage, then a plain s_barrier.
// MFMA K-permutation within a stage: lane group h (lanes 32h..32h+31) holds
// chunks 2h and 2h+1 of its row; MFMA t multiplies chunk 2h+t, so the two
// MFMAs of a stage cover chunks {0,2} and {1,3}; the row's scale dword (4
// blocks) shifted right by 16h gives blocks 2h, 2h+1 in bytes 0, 1 (op_sel t).
// ============================================================================
namespace tile_dma {
constexpr int kRows = 256;
constexpr int kRowBytes = 64;                   // code bytes per row per stage (K = 128)
constexpr int kOpBytes = kRows * kRowBytes;     // 16 KB per operand per stage
constexpr int kScaleOff = 2 * kOpBytes;         // scale dwords: W then X, 1 KB each
constexpr int kStage = 2 * kOpBytes + 2 * kRows * 4;
constexpr int kLoadsPerStage = 10;              // per wave: 2 x 4 code DMAs + 2 scale DMAs
}  // namespace tile_dma

template <int STAGES>
__global__ __launch_bounds__(256, 1) void gemm_tile_dma_fp4(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                            const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                            uint16_t* __restrict__ y, int M, int N, int K, int tiles_m,
                                                            int tiles_n) {
    using namespace tile_dma;
    constexpr int kStages = STAGES;
    static_assert(kStages >= 3 && kStages * kStage <= 160 * 1024, "LDS ring");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStage];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kTileM, n0 = tn * kTileN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = (int64_t)K / 2, KS = (int64_t)K / 32;
    const int nst = (int)(KB / kRowBytes);

    // code DMA sources: instruction i (0..3) of this wave covers rows 16*(4*wave+i) + lane/4;
    // the lane fetches logical chunk (lane%4) ^ ((row/4)%4) into physical slot lane%4
    const uint8_t* wsrc[4];
    const uint8_t* xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * (4 * wave + i) + (lane >> 2);
        const int chunk = (lane & 3) ^ ((row >> 2) & 3);
        wsrc[i] = qw + (int64_t)min(n0 + row, N - 1) * KB + 16 * chunk;
        xsrc[i] = qa + (int64_t)min(m0 + row, M - 1) * KB + 16 * chunk;
    }
    // scale DMA sources: row 64*wave + lane, one dword (4 blocks) per stage
    const uint8_t* wssrc = sw + (int64_t)min(n0 + 64 * wave + lane, N - 1) * KS;
    const uint8_t* xssrc = sa + (int64_t)min(m0 + 64 * wave + lane, M - 1) * KS;

    auto issue = [&](int s) {
        uint8_t* st = lds + (s % kStages) * kStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g2lds16(wsrc[i] + (int64_t)s * kRowBytes, st + (4 * wave + i) * 1024);
            g2lds16(xsrc[i] + (int64_t)s * kRowBytes, st + kOpBytes + (4 * wave + i) * 1024);
        }
        g2lds4(wssrc + 4 * s, st + kScaleOff + wave * 256);
        g2lds4(xssrc + 4 * s, st + kScaleOff + kRows * 4 + wave * 256);
    };

    v16f acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < nst) issue(s);

    // per-lane LDS offsets inside a stage
    int woff[4][2], xoff[4][2], wsoff[4], xsoff[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int wr = 128 * wn + 32 * f + l32, xr = 128 * wm + 32 * f + l32;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            woff[f][t] = wr * kRowBytes + 16 * ((2 * h + t) ^ ((wr >> 2) & 3));
            xoff[f][t] = kOpBytes + xr * kRowBytes + 16 * ((2 * h + t) ^ ((xr >> 2) & 3));
        }
        wsoff[f] = kScaleOff + wr * 4;
        xsoff[f] = kScaleOff + kRows * 4 + xr * 4;
    }
    const uint32_t base = lds_addr(lds);
    const int shift = 16 * h;

    for (int s = 0; s < nst; ++s) {
        const int ahead = min(kStages - 2, nst - 1 - s);
        __builtin_amdgcn_sched_barrier(0);
        if (ahead >= 2) wait_vmcnt<2 * kLoadsPerStage>();
        else if (ahead == 1) wait_vmcnt<kLoadsPerStage>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (s + kStages - 1 < nst) issue(s + kStages - 1);
        const uint32_t sb = base + (s % kStages) * kStage;
        uint32_t wsc[4], xsc[4];
        v4u wv[2][4], xv[2][4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            wsc[f] = lds_read4(sb + wsoff[f]);
            xsc[f] = lds_read4(sb + xsoff[f]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                wv[t][f] = lds_read16(sb + woff[f][t]);
                xv[t][f] = lds_read16(sb + xoff[f][t]);
            }
        // LDS results return in issue order: lgkmcnt(8) covers the scales and the t = 0 operands
        lds_wait_first(wv[0], xv[0], wsc, xsc);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                acc[f][g] = mfma32<kFmtFP4, 0>(fp4_operand(wv[0][f]), fp4_operand(xv[0][g]), acc[f][g],
                                               (int)(wsc[f] >> shift), (int)(xsc[g] >> shift));
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_rest(wv[1], xv[1]);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                acc[f][g] = mfma32<kFmtFP4, 1>(fp4_operand(wv[1][f]), fp4_operand(xv[1][g]), acc[f][g],
                                               (int)(wsc[f] >> shift), (int)(xsc[g] >> shift));
    }
    __builtin_amdgcn_sched_barrier(0);

    // epilogue (same layout as gemm_tile_kernel): Y[m][n .. n+3] per register quad
    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int m = m0 + 128 * wm + 32 * g + l32;
        if (m >= M) continue;
        uint16_t* yrow = y + (int64_t)m * N;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + 128 * wn + 32 * f + 8 * j + 4 * h;
                if (vec_ok && n + 3 < N) {
                    uint2 pk;
                    pk.x = bf16_rne(acc[f][g][4 * j]) | (bf16_rne(acc[f][g][4 * j + 1]) << 16);
                    pk.y = bf16_rne(acc[f][g][4 * j + 2]) | (bf16_rne(acc[f][g][4 * j + 3]) << 16);
                    *reinterpret_cast<uint2*>(yrow + n) = pk;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) yrow[n + e] = (uint16_t)bf16_rne(acc[f][g][4 * j + e]);
                }
            }
    }
}

// ============================================================================
// Tile path, FP4, K % 512 == 0: full-cache-line staging.
// A CU's vector memory path moves about one 64-byte half line per clock, and a
// request for part of a 128-byte line costs as much as the whole line, so
// every global -> LDS copy here moves whole lines: a superstage is K = 256
// (128 code bytes per row) of both TM-row operands, 8 rows per wave
// instruction, into a ring of S slots (S = 2; S = 4 for 128-row tiles when
// there is at most one tile per CU, whose small superstages would otherwise
// wait on copy latency).  Scales are fetched in bulk, 32 bytes per row (K = 1024, four
// superstages), into a ring of NB buffers, a quarter of a block with every
// superstage's copies.
// Output tile TM x TM (256, or 128 for shapes with too few 256-tiles to fill
// the CUs), 4 waves (2 x 2, each TM/2 x TM/2 from 32 x 32 x 64 MFMAs), four
// k-steps per superstage.  One barrier per superstage, placed once every wave
// has read all of superstage u (and its own copies of u + 1 have landed):
// after it, each wave reads the scales and the first two k-steps of u + 1 and
// issues the copies of u + S into the slot just released, both spread between
// the MFMAs of k-steps 2 and 3 of u; the operands of k-steps 2 and 3 are read
// between the MFMAs of k-steps 0 and 1.  Every such placement is fixed with
// scheduling barriers, so LDS reads and copies go out while the matrix core
// is busy, and a wave never has more than 15 LDS reads in flight.
// K-permutation inside a superstage: lane group h multiplies the row's 16-byte
// chunks 4h .. 4h+3 in k-steps t = 0..3, so the scale dword at byte 8q + 4h of
// the row's bulk scale segment (q = superstage within the block) serves all
// four k-steps with op_sel t.  LDS chunks are XOR-swizzled by (row / 2) % 8,
// which spreads the 16 lanes of every ds_read_b128 phase over all banks.
// ============================================================================
namespace tile_fp4 {
template <int TM, int S>
struct Cfg {
    static constexpr int kRows = TM;                          // rows of each operand
    static constexpr int kFW = TM / 64;                       // 32 x 32 fragments per wave and dimension
    static constexpr int kRowBytes = 128;                     // code bytes per row per superstage
    static constexpr int kOpBytes = kRows * kRowBytes;
    static constexpr int kSlot = 2 * kOpBytes;                // W rows, then A rows
    static constexpr int kHalfCopies = kRows / 32;            // code copies per wave per operand and superstage
    static constexpr int kCodeCopies = 2 * kHalfCopies;
    static constexpr int kScaleRow = 32;                      // bulk scale bytes per row (K = 1024)
    static constexpr int kScaleBuf = 2 * kRows * kScaleRow;   // W rows, then A rows
    static constexpr int kScLane = TM == 256 ? 16 : 4;        // scale bytes per lane and copy
    static constexpr int kScLanesPerRow = kScaleRow / kScLane;
    static constexpr int kScRowsPerCopy = 64 / kScLanesPerRow;
    static constexpr int kScaleCopies = kScaleBuf / (64 * kScLane);  // copies per block
    static constexpr int kScPerWave = kScaleCopies / 16;             // per wave and superstage
    static constexpr int kOutPitch = 2 * TM + 16;             // epilogue staging pitch (bytes), odd in 16 bytes
    // Code slots and scale buffers of the ring.  The codes of superstage v are copied S superstages
    // ahead, after the barrier of superstage v - S; part j of scale block b travels with the codes of
    // superstage 4b - 3 + j.  Block b lands in buffer b mod NB, which block b - NB (read last for
    // superstage 4b - 4 NB + 3) frees in time when S <= 4 NB - 6.  S = 4 (152 KB of LDS at 128-row
    // tiles) hides L2 / HBM latency when there is one workgroup per CU; S = 2 (80 KB) lets two
    // workgroups share a CU instead.
    static constexpr int kS = S;
    static constexpr int kNB = S == 2 ? 2 : 3;
    static_assert(kS <= 4 * kNB - 6, "scale ring too shallow for the code ring");
    static constexpr int kRing = kS * kSlot + kNB * kScaleBuf;
    static constexpr int kLds = kRing > TM * kOutPitch ? kRing : TM * kOutPitch;
    static_assert(kScPerWave >= 1 && kScaleCopies == 16 * kScPerWave && kFW >= 1, "tile shape");
    static_assert((kS - 1) * (kCodeCopies + kScPerWave) < 64, "vmcnt range");
    static_assert(kLds <= 160 * 1024, "LDS");
};
}  // namespace tile_fp4

// VEC: N % 8 == 0 and y 16-byte aligned (whole 16-byte output stores allowed).  S: code slots of
// the ring.  The library runs S = 2 (two 128-row workgroups per CU, or 256-row tiles); the 4-slot
// ring for at most one 128-row tile per CU runs as gemm_tile128_pc_fp4 (copy waves beside the MFMA
// waves), which measured 20% faster than this kernel with S = 4.
template <bool VEC, int TM, int S = 2>
__global__ __launch_bounds__(256, 1) void gemm_tile_fp4(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                        const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                        uint16_t* __restrict__ y, int M, int N, int K, int tiles_m,
                                                        int tiles_n) {
    using C = tile_fp4::Cfg<TM, S>;
    constexpr int FW = C::kFW;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * TM, n0 = tn * TM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = (int64_t)K / 2, KS = (int64_t)K / 32;
    const int nsup = K / 256;

    // code copy i (0 .. kCodeCopies-1): W rows for i < kHalfCopies, then A rows; copy i' = i mod
    // kHalfCopies moves rows 8 (kHalfCopies * wave + i') + lane / 8, the lane filling physical chunk
    // lane % 8 with logical chunk (lane % 8) ^ ((row / 2) % 8)
    const uint8_t* wrow[C::kHalfCopies];
    const uint8_t* xrow[C::kHalfCopies];
#pragma unroll
    for (int i = 0; i < C::kHalfCopies; ++i) {
        const int row = 8 * (C::kHalfCopies * wave + i) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        wrow[i] = qw + (int64_t)min(n0 + row, N - 1) * KB + 16 * chunk;
        xrow[i] = qa + (int64_t)min(m0 + row, M - 1) * KB + 16 * chunk;
    }
    auto issue_code = [&](int u, int i) {  // copy i of superstage min(u, nsup - 1) into the slot of u
        uint8_t* slot = lds + (u % C::kS) * C::kSlot;
        const int64_t koff = (int64_t)min(u, nsup - 1) * C::kRowBytes;
        if (i < C::kHalfCopies) g2lds16(wrow[i] + koff, slot + (C::kHalfCopies * wave + i) * 1024);
        else g2lds16(xrow[i - C::kHalfCopies] + koff, slot + C::kOpBytes + (C::kHalfCopies * wave + i - C::kHalfCopies) * 1024);
    };
    // scale copy q (0 .. kScaleCopies-1) of block b moves the 32-byte segments of rows
    // kScRowsPerCopy (q mod kScaleCopies/2) + lane / kScLanesPerRow (W rows, then A rows), each lane
    // kScLane bytes of one; it lands at byte 64 kScLane q of the buffer, so row r of W sits at 32 r
    // and row r of A at 32 (TM + r).  Part j (0..3) of a block is copies 4 kScPerWave j + kScPerWave
    // wave + c (c < kScPerWave): every wave carries the same number, so no wave branches.  Part j
    // travels with the codes of superstage 4b - 3 + j: after every wave has finished with block
    // b - 2 in the same buffer (last read for superstage 4b - 5) and in time for 4b.
    auto issue_scale_copy = [&](int q, int b) {
        constexpr int half = C::kScaleCopies / 2;
        const int row = C::kScRowsPerCopy * (q % half) + lane / C::kScLanesPerRow;
        int64_t off = 32 * (int64_t)b + C::kScLane * (lane % C::kScLanesPerRow);
        if (off >= KS) off = 0;  // past the last block: any in-row address, never read
        const uint8_t* src = q < half ? sw + (int64_t)min(n0 + row, N - 1) * KS + off
                                      : sa + (int64_t)min(m0 + row, M - 1) * KS + off;
        uint8_t* dst = lds + C::kS * C::kSlot + (b % C::kNB) * C::kScaleBuf + q * 64 * C::kScLane;
        if constexpr (C::kScLane == 16) g2lds16(src, dst);
        else g2lds4(src, dst);
    };
    auto issue_scale = [&](int u) {  // the scale part travelling with superstage u
#pragma unroll
        for (int c = 0; c < C::kScPerWave; ++c)
            issue_scale_copy(4 * C::kScPerWave * ((u + 3) & 3) + C::kScPerWave * wave + c, (u + 3) >> 2);
    };

    // per-lane LDS offsets
    int woff[FW], xoff[FW], wsoff[FW], xsoff[FW];
#pragma unroll
    for (int f = 0; f < FW; ++f) {
        const int wr = (TM / 2) * wn + 32 * f + l32, xr = (TM / 2) * wm + 32 * f + l32;
        woff[f] = wr * C::kRowBytes + ((wr >> 1) & 7);  // low bits: the swizzle key, split off below
        xoff[f] = C::kOpBytes + xr * C::kRowBytes + ((xr >> 1) & 7);
        wsoff[f] = wr * C::kScaleRow + 4 * h;
        xsoff[f] = (C::kRows + xr) * C::kScaleRow + 4 * h;
    }
    const uint32_t base = lds_addr(lds);
    auto rd_step = [&](v4u (&rw)[FW], v4u (&rx)[FW], int u, int t) {
        const uint32_t sb = base + (u % C::kS) * C::kSlot;
#pragma unroll
        for (int f = 0; f < FW; ++f) {
            rw[f] = lds_read16(sb + (woff[f] & ~7) + 16 * ((4 * h + t) ^ (woff[f] & 7)));
            rx[f] = lds_read16(sb + (xoff[f] & ~7) + 16 * ((4 * h + t) ^ (xoff[f] & 7)));
        }
    };
    // one operand of k-step t of superstage u: read i (0 .. 2 FW - 1) is fragment i / 2 of W (even i)
    // or of A (odd i), the order rd_step uses
    auto rd_one = [&](v4u (&rw)[FW], v4u (&rx)[FW], int u, int t, int i) {
        const uint32_t sb = base + (u % C::kS) * C::kSlot;
        const int f = i >> 1;
        if (i & 1) rx[f] = lds_read16(sb + (xoff[f] & ~7) + 16 * ((4 * h + t) ^ (xoff[f] & 7)));
        else rw[f] = lds_read16(sb + (woff[f] & ~7) + 16 * ((4 * h + t) ^ (woff[f] & 7)));
    };
    auto rd_scales = [&](uint32_t (&ws)[FW], uint32_t (&xs)[FW], int u) {
        const uint32_t scb = base + C::kS * C::kSlot + ((u >> 2) % C::kNB) * C::kScaleBuf + 8 * (u & 3);
#pragma unroll
        for (int f = 0; f < FW; ++f) {
            ws[f] = lds_read4(scb + wsoff[f]);
            xs[f] = lds_read4(scb + xsoff[f]);
        }
    };

    v16f acc[FW][FW];
#pragma unroll
    for (int f = 0; f < FW; ++f)
#pragma unroll
        for (int g = 0; g < FW; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;

    // prologue: scale block 0, the codes of superstage 0, then the batch of superstage 1
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < C::kScPerWave; ++c) issue_scale_copy(4 * C::kScPerWave * j + C::kScPerWave * wave + c, 0);
#pragma unroll
    for (int i = 0; i < C::kCodeCopies; ++i) issue_code(0, i);
#pragma unroll
    for (int v = 1; v < C::kS; ++v) {
        issue_scale(v);
#pragma unroll
        for (int i = 0; i < C::kCodeCopies; ++i) issue_code(v, i);
    }
    wait_vmcnt<(C::kS - 1) * (C::kCodeCopies + C::kScPerWave)>();  // superstage 0 and scale block 0 are in
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    uint32_t wsc[FW], xsc[FW];
    v4u r0w[FW], r0x[FW], r1w[FW], r1x[FW], r2w[FW], r2x[FW], r3w[FW], r3x[FW];
    rd_scales(wsc, xsc, 0);
    rd_step(r0w, r0x, 0, 0);
    rd_step(r1w, r1x, 0, 1);

    // The FW^2 MFMAs of k-step T, with the 2 FW operand reads of k-step TN issued between them (one
    // after every FW / 2 MFMAs), in this order: the reads go out while the matrix core is busy.
#define MX_STEP_RD(RW, RX, T, NW, NX, TN)                                                                          \
    _Pragma("unroll") for (int f = 0; f < FW; ++f) _Pragma("unroll") for (int g = 0; g < FW; ++g) {               \
        acc[f][g] = mfma32<kFmtFP4, T>(fp4_operand(RW[f]), fp4_operand(RX[g]), acc[f][g], (int)wsc[f], (int)xsc[g]); \
        if (((f * FW + g) % (FW / 2)) == FW / 2 - 1) rd_one(NW, NX, u, TN, (f * FW + g) / (FW / 2));             \
        __builtin_amdgcn_sched_barrier(0);                                                                         \
    }

    // superstage u; WAIT: the copies that may still be in flight once those of u + 1 have landed,
    // REFILL: issue the copies of u + S.  The last S superstages refill nothing, so neither their
    // barriers nor the epilogue wait for copies past the end (128-row tiles).  With fewer
    // superstages than slots (K = 512 at S = 4) the prologue's extra batches stay in flight, the
    // missing steps are skipped, and the waits kept count at most those batches too many (they
    // only wait longer).
    auto step = [&](int u, auto WAIT, auto REFILL) __attribute__((always_inline)) {
        // in flight: scales + k-steps 0, 1 of u (LDS reads); the copies of u + 1
        lds_wait_first_n<FW>(r0w, r0x, wsc, xsc);  // scales and k-step 0
        __builtin_amdgcn_sched_barrier(0);
        MX_STEP_RD(r0w, r0x, 0, r2w, r2x, 2)
        lds_wait_n_of<2 * FW, FW>(r1w, r1x);
        __builtin_amdgcn_sched_barrier(0);
        MX_STEP_RD(r1w, r1x, 1, r3w, r3x, 3)
        lds_wait_n_of<0, FW>(r2w, r2x);
        lds_wait_n_of<0, FW>(r3w, r3x);
        // this wave's copies of u + 1 (and of the scale part) have landed; those of u + 2 .. u + S - 1
        // may still be in flight
        wait_vmcnt<decltype(WAIT)::value>();
        __builtin_amdgcn_s_barrier();  // every wave: done reading u, copies of u + 1 complete
        __builtin_amdgcn_sched_barrier(0);
        uint32_t wsk[FW], xsk[FW];  // the scales of u, still needed for k-steps 2 and 3
#pragma unroll
        for (int f = 0; f < FW; ++f) {
            wsk[f] = wsc[f];
            xsk[f] = xsc[f];
        }
        rd_scales(wsc, xsc, u + 1);  // past the end these read stale data: unused
        if constexpr (decltype(REFILL)::value) issue_scale(u + C::kS);
        // k-steps 2 and 3 of u (2 FW^2 MFMAs), in this order, with the kCodeCopies copies of u + S and
        // the 4 FW operand reads of k-steps 0 and 1 of u + 1 spread between them (a wave keeps at most
        // 15 LDS reads in flight, so a burst of them would stall it)
        constexpr int kMf = 2 * FW * FW;
        constexpr int kEvery = kMf / C::kCodeCopies > 0 ? kMf / C::kCodeCopies : 1;
        constexpr int kRdEvery = kMf / (4 * FW);
#pragma unroll
        for (int t = 2; t < 4; ++t)
#pragma unroll
            for (int f = 0; f < FW; ++f)
#pragma unroll
                for (int g = 0; g < FW; ++g) {
                    const int i = (t - 2) * FW * FW + f * FW + g;
                    if (t == 2)
                        acc[f][g] = mfma32<kFmtFP4, 2>(fp4_operand(r2w[f]), fp4_operand(r2x[g]), acc[f][g], (int)wsk[f],
                                                       (int)xsk[g]);
                    else
                        acc[f][g] = mfma32<kFmtFP4, 3>(fp4_operand(r3w[f]), fp4_operand(r3x[g]), acc[f][g], (int)wsk[f],
                                                       (int)xsk[g]);
                    if constexpr (decltype(REFILL)::value)
                        if ((i % kEvery) == kEvery - 1 && i / kEvery < C::kCodeCopies) issue_code(u + C::kS, i / kEvery);
                    if ((i % kRdEvery) == kRdEvery - 1) {
                        const int ri = i / kRdEvery;
                        if (ri < 2 * FW) rd_one(r0w, r0x, u + 1, 0, ri);
                        else rd_one(r1w, r1x, u + 1, 1, ri - 2 * FW);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
    };
    constexpr int kBatch = C::kCodeCopies + C::kScPerWave;
    if constexpr (TM == 256) {
        // one call site: the peeled copies of the 256-row body no longer fit the registers (spills),
        // so every superstage refills (past the end: copies of the last superstage, never read)
        for (int u = 0; u < nsup; ++u) step(u, std::integral_constant<int, (C::kS - 2) * kBatch>{}, std::true_type{});
    } else {
        for (int u = 0; u < nsup - C::kS; ++u)
            step(u, std::integral_constant<int, (C::kS - 2) * kBatch>{}, std::true_type{});
        static_for<C::kS>([&](auto t) {
            constexpr int T = decltype(t)::value;
            const int u = nsup - C::kS + T;
            if (u >= 0)
                step(u, std::integral_constant<int, (C::kS - 2 - T > 0 ? C::kS - 2 - T : 0) * kBatch>{}, std::false_type{});
        });
    }
#undef MX_STEP_RD
    wait_vmcnt<0>();
    lds_wait_n_of<0, FW>(r0w, r0x);
    lds_wait_n_of<0, FW>(r1w, r1x);
    lds_tie(wsc);  // the last superstage's (unused) scale reads have landed before their registers are reused
    lds_tie(xsc);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // Epilogue through LDS: each wave writes its BF16 sub-tile row-major (padded pitch), then the
    // workgroup stores whole tile rows (2 TM bytes each).
#pragma unroll
    for (int g = 0; g < FW; ++g) {
        const int ml = (TM / 2) * wm + 32 * g + l32;
#pragma unroll
        for (int f = 0; f < FW; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int nl = (TM / 2) * wn + 32 * f + 8 * j + 4 * h;
                uint2 pk;
                pk.x = bf16x2_rne(acc[f][g][4 * j], acc[f][g][4 * j + 1]);
                pk.y = bf16x2_rne(acc[f][g][4 * j + 2], acc[f][g][4 * j + 3]);
                *reinterpret_cast<uint2*>(lds + ml * C::kOutPitch + 2 * nl) = pk;
            }
    }
    __syncthreads();
    constexpr int kLanesPerRow = TM / 8;          // 16-byte pieces per tile row
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    const int lr = lane / kLanesPerRow, lc = lane % kLanesPerRow;
#pragma unroll 4
    for (int r = 0; r < TM / 4 / kRowsPerStore; ++r) {
        const int ml = (TM / 4) * wave + kRowsPerStore * r + lr;
        const int m = m0 + ml;
        const int n = n0 + 8 * lc;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + ml * C::kOutPitch + 16 * lc);
        if (m >= M) continue;
        uint16_t* dst = y + (int64_t)m * N + n;
        if (VEC && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// ============================================================================
// Tile path, FP4, 128 x 128 tiles when they fit one round (at most 256 tiles): the staging, ring and
// MFMA schedule of gemm_tile_fp4<VEC, 128, 4>, split over 8 waves.  Waves 4..7 (producers) issue the
// global -> LDS copies of codes and scales that wave w - 4 of the 4-wave kernel issues, and wait for
// them; waves 0..3 (consumers) only read LDS and run the MFMAs of their 64 x 64 quarter.  Both meet at
// the same barriers (one per superstage: every consumer done reading superstage u, every copy of u + 1
// landed; then the producers refill u's slot with u + 4).  With one wave per SIMD the 4-wave kernel
// serialised the copy issue and waits, the LDS reads and the MFMAs (their costs added up); here each
// SIMD holds a consumer and a producer (159 registers per wave, so two fit), and the copies leave the
// MFMA waves' instruction stream.  Measured at N = 7168, K = 8192 (graph-replayed, 4 rotated weight
// copies, bit-identical outputs): M = 300 / 384 / 512: 20.4 / 20.9–21.2 / 22.9–24.9 us against 26.6 /
// 26.9–27.2 / 28.1–30.2 us.
// KP > 1: K split into KP parts of K / KP (a multiple of 1024) over KP workgroups per tile, whose FP32
// partials the consumers sum through the split-K tail of gemm_splitk.hpp (sk::tail_sum, a consumer's
// 2 x 2 fragments as MF = 4, compact slots) in ws (zero-filled before first use and left zero;
// sk::workspace_bytes_compact(tiles, KP, 4) bytes), so every workgroup of the grid must be resident at
// once.  Workgroup b belongs to XCD b % 8's run of tiles x TX .. x TX + TX - 1 (x = b % 8, TX =
// ceil(tiles / 8), tile t = tm + tiles_m tn, so an XCD's tiles share weight panels), as part (b / 8) % KP
// of tile x TX + (b / 8) / KP: the parts of a tile sit on one XCD.  KP == 1 follows tile_coords.
// ============================================================================
template <bool VEC, int KP = 1>
__global__ __launch_bounds__(512, 1) void gemm_tile128_pc_fp4(const uint8_t* __restrict__ qa,
                                                              const uint8_t* __restrict__ sa,
                                                              const uint8_t* __restrict__ qw,
                                                              const uint8_t* __restrict__ sw, uint16_t* __restrict__ y,
                                                              int M, int N, int K, int tiles_m, int tiles_n,
                                                              uint8_t* __restrict__ ws) {
    constexpr int TM = 128;
    using C = tile_fp4::Cfg<TM, 4>;
    constexpr int FW = C::kFW;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];

    int tm, tn, kq = 0, tile = 0;  // kq: this workgroup's K part
    if constexpr (KP == 1) {
        tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    } else {
        const int T = tiles_m * tiles_n, TX = (T + 7) >> 3, r = (int)blockIdx.x >> 3;
        kq = r % KP;
        tile = ((int)blockIdx.x & 7) * TX + r / KP;
        if (tile >= T) return;  // padding of the last XCD's run: no part of any tile
        tm = tile % tiles_m;
        tn = tile / tiles_m;
    }
    const int m0 = tm * TM, n0 = tn * TM;
    const int lane = threadIdx.x & 63;
    const int wave8 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform role
    const int wave = wave8 & 3;  // the 4-wave kernel's wave whose copies (producer) or quarter (consumer) this is
    const int64_t KB = (int64_t)K / 2, KS = (int64_t)K / 32;
    const int nsup = K / KP / 256;                     // superstages of this workgroup's K part
    const int64_t kbase = kq * (KB / KP), sbase = kq * (KS / KP);  // code / scale bytes of a row before it
    constexpr int kBatch = C::kCodeCopies + C::kScPerWave;          // copies per producer and superstage

    if (wave8 >= 4) {
        // Producer.  Code copy i (0 .. kCodeCopies-1): W rows for i < kHalfCopies, then A rows; copy
        // i' = i mod kHalfCopies moves rows 8 (kHalfCopies * wave + i') + lane / 8, the lane filling
        // physical chunk lane % 8 with logical chunk (lane % 8) ^ sk::key(row): any 8 consecutive rows get 8
        // distinct keys, so the consumers' reads of 8 rows hit distinct banks (the (row / 2) % 8 key of
        // gemm_tile_fp4 conflicts two ways; this key measured 1-2.5% faster here at M = 256 .. 512).
        const uint8_t* wrow[C::kHalfCopies];
        const uint8_t* xrow[C::kHalfCopies];
#pragma unroll
        for (int i = 0; i < C::kHalfCopies; ++i) {
            const int row = 8 * (C::kHalfCopies * wave + i) + (lane >> 3);
            const int chunk = (lane & 7) ^ sk::key(row);
            wrow[i] = qw + (int64_t)min(n0 + row, N - 1) * KB + 16 * chunk;
            xrow[i] = qa + (int64_t)min(m0 + row, M - 1) * KB + 16 * chunk;
        }
        auto issue_code = [&](int u, int i) {  // copy i of superstage min(u, nsup - 1) into the slot of u
            uint8_t* slot = lds + (u % C::kS) * C::kSlot;
            const int64_t koff = kbase + (int64_t)min(u, nsup - 1) * C::kRowBytes;
            if (i < C::kHalfCopies) g2lds16(wrow[i] + koff, slot + (C::kHalfCopies * wave + i) * 1024);
            else
                g2lds16(xrow[i - C::kHalfCopies] + koff,
                        slot + C::kOpBytes + (C::kHalfCopies * wave + i - C::kHalfCopies) * 1024);
        };
        // scale copy q of block b: as in gemm_tile_fp4 (4 bytes per lane; part j of a block travels with
        // the codes of superstage 4b - 3 + j), within this workgroup's K part
        auto issue_scale_copy = [&](int q, int b) {
            constexpr int half = C::kScaleCopies / 2;
            const int row = C::kScRowsPerCopy * (q % half) + lane / C::kScLanesPerRow;
            int64_t off = 32 * (int64_t)b + C::kScLane * (lane % C::kScLanesPerRow);
            if (off >= KS / KP) off = 0;  // past the part's scale bytes: any in-row address, never read
            off += sbase;
            const uint8_t* src = q < half ? sw + (int64_t)min(n0 + row, N - 1) * KS + off
                                          : sa + (int64_t)min(m0 + row, M - 1) * KS + off;
            g2lds4(src, lds + C::kS * C::kSlot + (b % C::kNB) * C::kScaleBuf + q * 64 * C::kScLane);
        };
        auto issue_scale = [&](int u) {  // the scale part travelling with superstage u
#pragma unroll
            for (int c = 0; c < C::kScPerWave; ++c)
                issue_scale_copy(4 * C::kScPerWave * ((u + 3) & 3) + C::kScPerWave * wave + c, (u + 3) >> 2);
        };
        auto batch = [&](int u) {
            issue_scale(u);
#pragma unroll
            for (int i = 0; i < C::kCodeCopies; ++i) issue_code(u, i);
        };
        // prologue: scale block 0, the codes of superstage 0, then the batches of superstages 1 .. S - 1
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < C::kScPerWave; ++c) issue_scale_copy(4 * C::kScPerWave * j + C::kScPerWave * wave + c, 0);
#pragma unroll
        for (int i = 0; i < C::kCodeCopies; ++i) issue_code(0, i);
#pragma unroll
        for (int v = 1; v < C::kS; ++v) batch(v);
        wait_vmcnt<(C::kS - 1) * kBatch>();  // superstage 0 and scale block 0 are in
        __builtin_amdgcn_s_barrier();
        // barrier of superstage u: this wave's copies of u + 1 have landed (those of u + 2 .. u + S - 1
        // may be in flight); then the slot of u takes u + S.  The last S barriers refill nothing, and their
        // waits count down to the batches still in flight (with fewer superstages than slots the prologue's
        // extra batches only make them wait longer).
        for (int u = 0; u < nsup - C::kS; ++u) {
            wait_vmcnt<(C::kS - 2) * kBatch>();
            __builtin_amdgcn_s_barrier();
            batch(u + C::kS);
        }
        static_for<C::kS>([&](auto t) {
            constexpr int T = decltype(t)::value;
            if (nsup - C::kS + T >= 0) {
                wait_vmcnt<(C::kS - 2 - T > 0 ? C::kS - 2 - T : 0) * kBatch>();
                __builtin_amdgcn_s_barrier();
            }
        });
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // the consumers' barrier before the epilogue: no copy lands after it
    } else {
        // Consumer: the LDS reads and MFMAs of the 4-wave kernel's wave, 2 x 2 fragments of 32 x 32.
        const int wn = wave & 1, wm = wave >> 1;
        const int l32 = lane & 31, h = lane >> 5;
        int woff[FW], xoff[FW], wsoff[FW], xsoff[FW];
#pragma unroll
        for (int f = 0; f < FW; ++f) {
            const int wr = (TM / 2) * wn + 32 * f + l32, xr = (TM / 2) * wm + 32 * f + l32;
            woff[f] = wr * C::kRowBytes + sk::key(wr);  // low bits: the swizzle key, split off below
            xoff[f] = C::kOpBytes + xr * C::kRowBytes + sk::key(xr);
            wsoff[f] = wr * C::kScaleRow + 4 * h;
            xsoff[f] = (C::kRows + xr) * C::kScaleRow + 4 * h;
        }
        const uint32_t base = lds_addr(lds);
        auto rd_step = [&](v4u (&rw)[FW], v4u (&rx)[FW], int u, int t) {
            const uint32_t sb = base + (u % C::kS) * C::kSlot;
#pragma unroll
            for (int f = 0; f < FW; ++f) {
                rw[f] = lds_read16(sb + (woff[f] & ~7) + 16 * ((4 * h + t) ^ (woff[f] & 7)));
                rx[f] = lds_read16(sb + (xoff[f] & ~7) + 16 * ((4 * h + t) ^ (xoff[f] & 7)));
            }
        };
        // read i (0 .. 2 FW - 1) of k-step t of superstage u: fragment i / 2 of W (even i) or of A (odd i)
        auto rd_one = [&](v4u (&rw)[FW], v4u (&rx)[FW], int u, int t, int i) {
            const uint32_t sb = base + (u % C::kS) * C::kSlot;
            const int f = i >> 1;
            if (i & 1) rx[f] = lds_read16(sb + (xoff[f] & ~7) + 16 * ((4 * h + t) ^ (xoff[f] & 7)));
            else rw[f] = lds_read16(sb + (woff[f] & ~7) + 16 * ((4 * h + t) ^ (woff[f] & 7)));
        };
        auto rd_scales = [&](uint32_t (&ws4)[FW], uint32_t (&xs4)[FW], int u) {
            const uint32_t scb = base + C::kS * C::kSlot + ((u >> 2) % C::kNB) * C::kScaleBuf + 8 * (u & 3);
#pragma unroll
            for (int f = 0; f < FW; ++f) {
                ws4[f] = lds_read4(scb + wsoff[f]);
                xs4[f] = lds_read4(scb + xsoff[f]);
            }
        };
        v16f acc[FW][FW];
#pragma unroll
        for (int f = 0; f < FW; ++f)
#pragma unroll
            for (int g = 0; g < FW; ++g)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;
        __builtin_amdgcn_s_barrier();  // superstage 0 and scale block 0 are in
        __builtin_amdgcn_sched_barrier(0);
        uint32_t wsc[FW], xsc[FW];
        v4u r0w[FW], r0x[FW], r1w[FW], r1x[FW], r2w[FW], r2x[FW], r3w[FW], r3x[FW];
        rd_scales(wsc, xsc, 0);
        rd_step(r0w, r0x, 0, 0);
        rd_step(r1w, r1x, 0, 1);
        // the FW^2 MFMAs of k-step T with the 2 FW operand reads of k-step TN between them
#define MX_STEP_RD(RW, RX, T, NW, NX, TN)                                                                          \
    _Pragma("unroll") for (int f = 0; f < FW; ++f) _Pragma("unroll") for (int g = 0; g < FW; ++g) {               \
        acc[f][g] = mfma32<kFmtFP4, T>(fp4_operand(RW[f]), fp4_operand(RX[g]), acc[f][g], (int)wsc[f], (int)xsc[g]); \
        if (((f * FW + g) % (FW / 2)) == FW / 2 - 1) rd_one(NW, NX, u, TN, (f * FW + g) / (FW / 2));             \
        __builtin_amdgcn_sched_barrier(0);                                                                         \
    }
        // superstage u: k-steps 0 and 1, the barrier, then k-steps 2 and 3 with the scale reads and the
        // k-step 0 and 1 reads of u + 1 between the MFMAs (past the end these read stale data, never used)
        auto step = [&](int u) __attribute__((always_inline)) {
            lds_wait_first_n<FW>(r0w, r0x, wsc, xsc);  // scales and k-step 0
            __builtin_amdgcn_sched_barrier(0);
            MX_STEP_RD(r0w, r0x, 0, r2w, r2x, 2)
            lds_wait_n_of<2 * FW, FW>(r1w, r1x);
            __builtin_amdgcn_sched_barrier(0);
            MX_STEP_RD(r1w, r1x, 1, r3w, r3x, 3)
            lds_wait_n_of<0, FW>(r2w, r2x);
            lds_wait_n_of<0, FW>(r3w, r3x);
            __builtin_amdgcn_s_barrier();  // every consumer done reading u; every copy of u + 1 landed
            __builtin_amdgcn_sched_barrier(0);
            uint32_t wsk[FW], xsk[FW];  // the scales of u, still needed for k-steps 2 and 3
#pragma unroll
            for (int f = 0; f < FW; ++f) {
                wsk[f] = wsc[f];
                xsk[f] = xsc[f];
            }
            rd_scales(wsc, xsc, u + 1);
            constexpr int kRdEvery = (2 * FW * FW) / (4 * FW);
#pragma unroll
            for (int t = 2; t < 4; ++t)
#pragma unroll
                for (int f = 0; f < FW; ++f)
#pragma unroll
                    for (int g = 0; g < FW; ++g) {
                        const int i = (t - 2) * FW * FW + f * FW + g;
                        if (t == 2)
                            acc[f][g] = mfma32<kFmtFP4, 2>(fp4_operand(r2w[f]), fp4_operand(r2x[g]), acc[f][g],
                                                           (int)wsk[f], (int)xsk[g]);
                        else
                            acc[f][g] = mfma32<kFmtFP4, 3>(fp4_operand(r3w[f]), fp4_operand(r3x[g]), acc[f][g],
                                                           (int)wsk[f], (int)xsk[g]);
                        if ((i % kRdEvery) == kRdEvery - 1) {
                            const int ri = i / kRdEvery;
                            if (ri < 2 * FW) rd_one(r0w, r0x, u + 1, 0, ri);
                            else rd_one(r1w, r1x, u + 1, 1, ri - 2 * FW);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
        };
        for (int u = 0; u < nsup; ++u) step(u);
#undef MX_STEP_RD
        lds_wait_n_of<0, FW>(r0w, r0x);
        lds_wait_n_of<0, FW>(r1w, r1x);
        lds_tie(wsc);  // the last superstage's (unused) scale reads have landed before their registers are reused
        lds_tie(xsc);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (KP > 1) {
            // the K parts' sum: fragment (f, g) is tail fragment FW f + g, its registers 4 j .. 4 j + 3
            // the 4 consecutive n of one m
            v4f mine[FW * FW][4];
#pragma unroll
            for (int f = 0; f < FW; ++f)
#pragma unroll
                for (int g = 0; g < FW; ++g)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        mine[FW * f + g][j] = v4f{acc[f][g][4 * j], acc[f][g][4 * j + 1], acc[f][g][4 * j + 2],
                                                  acc[f][g][4 * j + 3]};
            auto store_one = [&](int fr, int j, const v4f& v) {
                const int f = fr / FW, g = fr % FW;
                const int m = m0 + (TM / 2) * wm + 32 * g + l32, n = n0 + (TM / 2) * wn + 32 * f + 8 * j + 4 * h;
                if (m >= M) return;
                uint16_t* dst = y + (int64_t)m * N + n;
                const uint32_t w2[2] = {bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3])};
                if (VEC && n + 3 < N) {
                    *reinterpret_cast<uint2*>(dst) = make_uint2(w2[0], w2[1]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) dst[e] = (uint16_t)(w2[e >> 1] >> (16 * (e & 1)));
                }
            };
            sk::tail_sum<FW * FW, KP>(mine, ws, (int)sk::workspace_bytes_compact(tiles_m * tiles_n, KP, FW * FW), tile,
                                      kq, wave, lane, store_one, std::true_type{});
        } else {
            // BF16 sub-tile into LDS (padded pitch) for whole-row stores below
#pragma unroll
            for (int g = 0; g < FW; ++g) {
                const int ml = (TM / 2) * wm + 32 * g + l32;
#pragma unroll
                for (int f = 0; f < FW; ++f)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int nl = (TM / 2) * wn + 32 * f + 8 * j + 4 * h;
                        uint2 pk;
                        pk.x = bf16x2_rne(acc[f][g][4 * j], acc[f][g][4 * j + 1]);
                        pk.y = bf16x2_rne(acc[f][g][4 * j + 2], acc[f][g][4 * j + 3]);
                        *reinterpret_cast<uint2*>(lds + ml * C::kOutPitch + 2 * nl) = pk;
                    }
            }
        }
    }
    if constexpr (KP > 1) return;
    __syncthreads();
    // all 8 waves store whole tile rows (2 TM bytes each): wave w rows 16 w .. 16 w + 15
    constexpr int kLanesPerRow = TM / 8;  // 16-byte pieces per tile row
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    const int lr = lane / kLanesPerRow, lc = lane % kLanesPerRow;
#pragma unroll
    for (int r = 0; r < TM / 8 / kRowsPerStore; ++r) {
        const int ml = (TM / 8) * wave8 + kRowsPerStore * r + lr;
        const int m = m0 + ml;
        const int n = n0 + 8 * lc;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + ml * C::kOutPitch + 16 * lc);
        if (m >= M) continue;
        uint16_t* dst = y + (int64_t)m * N + n;
        if (VEC && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// ============================================================================
// Tile path, FP4, K % 512 == 0: 256 x 224 output tiles from 16 x 16 x 128
// scaled MFMAs.  N = 7168 is 32 tiles of 224, so M = 8192 gives 32 x 32 =
// 1024 tiles, four full rounds on 256 CUs; 256 x 256 tiles give 896 = 3.5
// rounds and leave half the CUs idle in the last one.  Staging as in
// gemm_tile_fp4: superstages of K = 256 (128 code bytes per row, whole cache
// lines) of the 224 weight and 256 activation rows, 8 rows per wave copy,
// into two 60 KB slots; scales in bulk, 32 bytes per row (K = 1024), into two
// 16 KB buffers, a quarter block travelling with each superstage (15 copies
// of 32 rows per block and one dummy, so each wave carries one per
// superstage).  4 waves in 2 x 2, each 128 (m) x 112 (n): 8 activation and 7
// weight fragments of 16 rows, 56 accumulators of 4 values.
// A superstage is two k-steps.  Lane group g (lanes 16g .. 16g+15) multiplies
// the row's 16-byte chunks 2g (k-step 0) and 2g + 1 (k-step 1), so one 16-bit
// read at byte 8q + 2g of the row's bulk scale segment (q = superstage within
// the block) serves both k-steps with op_sel 0 and 1.  Chunks are XOR-swizzled
// in LDS by (row / 2) % 8 as in gemm_tile_fp4.
// Per superstage u: the MFMAs of k-step 0 with the reads of k-step 1
// between them; a barrier once every wave has read all of u and its own
// copies of u + 1 have landed; then the MFMAs of k-step 1 with the scale
// reads and k-step-0 reads of u + 1 and the copies of u + 2 (into the slot
// just released) between them.  Scheduling barriers fix every placement.
// ============================================================================
namespace tile224 {
constexpr int kTM = 256, kTN = 224;            // activation rows (m), weight rows (n) per tile
constexpr int kFA = 8, kFW = 7;                // 16-row fragments per wave: activation, weight
constexpr int kRowBytes = 128;                 // code bytes per row per superstage
constexpr int kWBytes = kTN * kRowBytes;       // weight rows first in a slot, then activation rows
constexpr int kSlot = kWBytes + kTM * kRowBytes;
constexpr int kWCopies = kTN / 32, kACopies = kTM / 32;  // code copies per wave and superstage
constexpr int kCodeCopies = kWCopies + kACopies;
constexpr int kScaleRow = 32;                  // bulk scale bytes per row (K = 1024)
constexpr int kScaleBuf = 16 * 1024;           // 15 copies of 32 rows x 32 bytes, one dummy
constexpr int kOutPitch = 2 * kTN + 16;        // epilogue staging pitch (bytes)
constexpr int kRing = 2 * kSlot + 2 * kScaleBuf;
constexpr int kLds = kRing > kTM * kOutPitch ? kRing : kTM * kOutPitch;
constexpr int kMf = kFW * kFA;                 // MFMAs per wave and k-step
static_assert(kLds <= 160 * 1024, "LDS");
static_assert((kTN + kTM) / 32 == 15, "15 scale copies of 32 rows per block");
}  // namespace tile224

// VEC: N % 8 == 0 and y 16-byte aligned (whole 16-byte output stores allowed).
template <bool VEC>
__global__ __launch_bounds__(256, 1) void gemm_tile224_fp4(const uint8_t* __restrict__ qa,
                                                           const uint8_t* __restrict__ sa,
                                                           const uint8_t* __restrict__ qw,
                                                           const uint8_t* __restrict__ sw, uint16_t* __restrict__ y,
                                                           int M, int N, int K, int tiles_m, int tiles_n) {
    using namespace tile224;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kTM, n0 = tn * kTN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar registers
    const int wn = wave & 1, wm = wave >> 1;
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t KB = (int64_t)K / 2, KS = (int64_t)K / 32;
    const int nsup = K / 256;

    // code copy i: weight rows 8 (kWCopies wave + i) + lane / 8 for i < kWCopies, else activation
    // rows 8 (kACopies wave + i - kWCopies) + lane / 8; the lane fills physical chunk lane % 8 with
    // logical chunk (lane % 8) ^ ((row / 2) % 8).  The copies are buffer loads: a 32-bit offset per
    // lane, the superstage in the scalar offset, and the operand's size as the descriptor's range, so
    // rows past M or N read as zeros (their outputs are never stored).  The host keeps rows * K / 2
    // below 2^31.
    constexpr int kRawBufferWord3 = 0x00020000;
    const __amdgpu_buffer_rsrc_t wrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)qw, (short)0, (int)(N * KB), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t arsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)qa, (short)0, (int)(M * KB), kRawBufferWord3);
    uint32_t coff[kCodeCopies];
    int cdst[kCodeCopies];
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i) {
        const bool isw = i < kWCopies;
        const int row = isw ? 8 * (kWCopies * wave + i) + (lane >> 3) : 8 * (kACopies * wave + i - kWCopies) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        coff[i] = (uint32_t)(((isw ? n0 : m0) + row) * KB + 16 * chunk);
        cdst[i] = isw ? (kWCopies * wave + i) * 1024 : kWBytes + (kACopies * wave + i - kWCopies) * 1024;
    }
    auto issue_code = [&](int u, int i) {  // copy i of superstage min(u, nsup - 1) into the slot of u
        const int koff = min(u, nsup - 1) * kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(i < kWCopies ? wrsrc : arsrc,
                                                 (__attribute__((address_space(3))) void*)(lds + (u & 1) * kSlot + cdst[i]),
                                                 16, coff[i], koff, 0, 0);
    };
    // scale copy q (0..15) of block b: q < 7 moves weight rows 32 q + lane / 2, 7 <= q < 15
    // activation rows 32 (q - 7) + lane / 2, each lane 16 bytes of the row's 32-byte segment; copy q
    // lands at 1024 q, so weight row r sits at 32 r and activation row r at 32 (kTN + r).  Copy 15
    // is a dummy (an in-bounds activation row into the unused last KB).  Part j (0..3) of block b is
    // copy 4j + wave and travels with the codes of superstage 4b - 3 + j: after every wave has read
    // block b - 2 in the same buffer (last for superstage 4b - 5) and in time for superstage 4b.
    auto issue_scale = [&](int u) {
        const int b = (u + 3) >> 2, q = 4 * ((u + 3) & 3) + wave;
        const bool isw = q < 7;
        const int r = isw ? min(n0 + 32 * q + (lane >> 1), N - 1) : min(m0 + 32 * (q - 7) + (lane >> 1), M - 1);
        int64_t off = 32 * (int64_t)b + 16 * (lane & 1);
        off = off >= KS ? 0 : off;  // past the last block: any in-row address, never read
        const uint8_t* src = (isw ? sw : sa) + (int64_t)r * KS + off;
        g2lds16(src, lds + 2 * kSlot + (b & 1) * kScaleBuf + q * 1024);
    };

    // LDS addressing: fragment f of a wave's weight rows starts 16 f rows (2048 f bytes) after its
    // first, so every read is a per-lane base plus an immediate.  The swizzle key of row r,
    // (r / 2) % 8, is (l16 / 2) for every fragment (fragments start at multiples of 16 rows), so
    // the chunk offset of k-step t, 16 ((2g + t) ^ key), is one value per lane and k-step.
    const int key = l16 >> 1;
    const uint32_t base = lds_addr(lds);
    const uint32_t wrow0 = ((kTN / 2) * wn + l16) * kRowBytes, xrow0 = kWBytes + ((kTM / 2) * wm + l16) * kRowBytes;
    const uint32_t ck0 = 16 * ((2 * g) ^ key), ck1 = 16 * ((2 * g + 1) ^ key);
    const uint32_t wsrow0 = ((kTN / 2) * wn + l16) * kScaleRow + 2 * g;
    const uint32_t xsrow0 = (kTN + (kTM / 2) * wm + l16) * kScaleRow + 2 * g;
    // read i (0 .. kFW + kFA - 1) of k-step T of superstage u: weight fragment i, then activation
    // fragment i - kFW
    auto rd_one = [&](v4u (&rw)[kFW], v4u (&rx)[kFA], uint32_t wb, uint32_t xb, auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < kFW) rw[i] = lds_read16_at<i * 16 * kRowBytes>(wb);
        else rx[i - kFW] = lds_read16_at<(i - kFW) * 16 * kRowBytes>(xb);
    };
    auto rd_scale = [&](uint32_t (&ws)[kFW], uint32_t (&xs)[kFA], uint32_t wb, uint32_t xb, auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < kFW) ws[i] = lds_read2_at<i * 16 * kScaleRow>(wb);
        else xs[i - kFW] = lds_read2_at<(i - kFW) * 16 * kScaleRow>(xb);
    };
    auto slot_of = [&](int u) { return base + (u & 1) * kSlot; };
    auto sc_of = [&](int u) { return base + 2 * kSlot + ((u >> 2) & 1) * kScaleBuf + 8 * (u & 3); };

    v4f acc[kFW][kFA];
#pragma unroll
    for (int f = 0; f < kFW; ++f)
#pragma unroll
        for (int j = 0; j < kFA; ++j) {
            acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+a"(acc[f][j]));  // zeros in place in the AGPRs before the wait below
        }
    wait_states8<2>();  // VALU writes of the accumulators -> first MFMA

    // prologue: scale block 0, the codes of superstage 0, then the batch of superstage 1
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_scale(j - 3);
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i) issue_code(0, i);
    issue_scale(1);
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i) issue_code(1, i);
    wait_vmcnt<kCodeCopies + 1>();  // superstage 0 and scale block 0 are in
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    constexpr int kRd = kFW + kFA;  // operand reads per k-step (and scale reads per superstage)
    uint32_t wsc[kFW], xsc[kFA];
    v4u r0w[kFW], r0x[kFA], r1w[kFW], r1x[kFA];
    static_for<kRd>([&](auto ic) { rd_scale(wsc, xsc, sc_of(0) + wsrow0, sc_of(0) + xsrow0, ic); });
    static_for<kRd>([&](auto ic) { rd_one(r0w, r0x, slot_of(0) + wrow0 + ck0, slot_of(0) + xrow0 + ck0, ic); });

    // superstage u; REFILL: issue the copies of u + 2 (the last two superstages have none to issue,
    // so neither their barriers nor the epilogue wait for copies past the end)
    auto step = [&](int u, auto REFILL) __attribute__((always_inline)) {
        // in flight: the scales and k-step 0 of u (LDS reads); the copies of u + 1
        lds_wait<0>();
        lds_tie(r0w);
        lds_tie(r0x);
        lds_tie(wsc);
        lds_tie(xsc);
        __builtin_amdgcn_sched_barrier(0);
        // k-step 0 (weight-fragment-major), with the reads of k-step 1 between the MFMAs: activation
        // fragment j after MFMA 2j; weight fragment f once row f of the MFMAs has read r0w[f] (two
        // MFMAs later, so it can take those registers), f = 6 early
        {
            const uint32_t wb = slot_of(u) + wrow0 + ck1, xb = slot_of(u) + xrow0 + ck1;
            static_for<kMf>([&](auto ic) {
                constexpr int i = decltype(ic)::value, f = i / kFA, j = i % kFA;
                mfma16_fp4_agpr<0>(acc[f][j], r0w[f], r0x[j], wsc[f], xsc[j]);
                static_for<kRd>([&](auto rc) {
                    constexpr int ri = decltype(rc)::value;  // < kFW: weight fragment ri, else activation ri - kFW
                    constexpr int at = ri >= kFW ? 2 * (ri - kFW) : ri == kFW - 1 ? 3 : kFA * ri + kFA + 2;
                    if constexpr (at == i) rd_one(r1w, r1x, wb, xb, rc);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        lds_wait<0>();
        lds_tie(r1w);
        lds_tie(r1x);
        wait_vmcnt<0>();  // this wave's copies of u + 1 (and of the scale part) have landed
        __builtin_amdgcn_s_barrier();  // every wave: done reading u, copies of u + 1 complete
        __builtin_amdgcn_sched_barrier(0);
        uint32_t wsk[kFW], xsk[kFA];  // the scales of u, still needed for k-step 1
#pragma unroll
        for (int f = 0; f < kFW; ++f) wsk[f] = wsc[f];
#pragma unroll
        for (int j = 0; j < kFA; ++j) xsk[j] = xsc[j];
        lds_tie(wsk);  // the copies (VALU) are done here ...
        lds_tie(xsk);
        if constexpr (decltype(REFILL)::value) issue_scale(u + 2);
        wait_states8<1>();  // ... and some wait states before an MFMA reads them
        __builtin_amdgcn_sched_barrier(0);
        // k-step 1, with the kCodeCopies copies of u + 2 and the 2 kRd reads (scales, then k-step 0)
        // of u + 1 spread between the MFMAs; past the end these read stale slot data, never used
        // k-step 1 (activation-fragment-major), with the copies of u + 2 and the reads of u + 1 between
        // the MFMAs: the 15 scales first, the weight fragments (fresh registers), then activation
        // fragment j once column j has read r1x[j] (two MFMAs later), j = 7 early
        {
            const uint32_t wb = slot_of(u + 1) + wrow0 + ck0, xb = slot_of(u + 1) + xrow0 + ck0;
            const uint32_t wsb = sc_of(u + 1) + wsrow0, xsb = sc_of(u + 1) + xsrow0;
            static_for<kMf>([&](auto ic) {
                constexpr int i = decltype(ic)::value, j = i / kFW, f = i % kFW;
                mfma16_fp4_agpr<1>(acc[f][j], r1w[f], r1x[j], wsk[f], xsk[j]);
                static_for<kCodeCopies>([&](auto cc) {
                    if constexpr (decltype(REFILL)::value && (decltype(cc)::value * kMf) / kCodeCopies == i)
                        issue_code(u + 2, decltype(cc)::value);
                });
                static_for<kRd>([&](auto rc) {
                    if constexpr (decltype(rc)::value == i) rd_scale(wsc, xsc, wsb, xsb, rc);
                });
                static_for<kRd>([&](auto rc) {
                    constexpr int ri = decltype(rc)::value;
                    constexpr int at = ri < kFW ? kRd + 2 * ri : ri == kRd - 1 ? kRd + 2 * kFW : kFW * (ri - kFW) + kFW + 2;
                    if constexpr (at == i) rd_one(r0w, r0x, wb, xb, rc);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    };
    for (int u = 0; u < nsup - 2; ++u) step(u, std::true_type{});
    if (nsup >= 2) step(nsup - 2, std::false_type{});
    step(nsup - 1, std::false_type{});
    wait_vmcnt<0>();
    lds_wait<0>();
    lds_tie(r0w);
    lds_tie(r0x);
    lds_tie(wsc);
    lds_tie(xsc);
    wait_states8<3>();  // last MFMA -> reads of the accumulators (tied here, so none moves above)
#pragma unroll
    for (int f = 0; f < kFW; ++f)
#pragma unroll
        for (int j = 0; j < kFA; ++j) asm volatile("" : "+a"(acc[f][j]));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // Epilogue through LDS: each lane holds 4 consecutive n of one m per fragment pair; the
    // workgroup then stores whole 448-byte tile rows.
#pragma unroll
    for (int f = 0; f < kFW; ++f) {
        const int nl = (kTN / 2) * wn + 16 * f + 4 * g;
#pragma unroll
        for (int j = 0; j < kFA; ++j) {
            const int ml = (kTM / 2) * wm + 16 * j + l16;
            uint2 pk;
            pk.x = bf16x2_rne(acc[f][j][0], acc[f][j][1]);
            pk.y = bf16x2_rne(acc[f][j][2], acc[f][j][3]);
            *reinterpret_cast<uint2*>(lds + ml * kOutPitch + 2 * nl) = pk;
        }
    }
    __syncthreads();
    constexpr int kPieces = kTN / 8;  // 16-byte pieces per tile row
#pragma unroll 4
    for (int it = 0; it < kPieces; ++it) {  // wave w stores tile rows 64 w .. 64 w + 63
        const int p = 64 * it + lane;
        const int row = p / kPieces, col = p - kPieces * row;
        const int ml = 64 * wave + row;
        const int m = m0 + ml, n = n0 + 8 * col;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + ml * kOutPitch + 16 * col);
        if (m >= M) continue;
        uint16_t* dst = y + (int64_t)m * N + n;
        if (VEC && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// ============================================================================
// Tile path, FP8 (E4M3 widened exactly to FP16), any K % 128 == 0.
// The structure of gemm_tile_fp4: 256 x 256 output tile, 4 waves (2 x 2,
// 128 x 128 each, 4 x 4 fragments of 32 x 32 in AGPRs), superstages of 128
// code bytes per row (K = 128 here) copied whole-line global -> LDS into two
// 64 KB slots, one barrier per superstage.  Every E4M3 value is an FP16 value,
// so a 16-byte LDS read widens exactly into two 8-value FP16 operands of the
// 32 x 32 x 16 FP16 MFMA (the FP8 MFMA rounds small products away next to
// large ones; FP16 does not).  Lane group h multiplies the row's chunks
// 4h .. 4h+3: read group j (chunk 4h + j) feeds two k-steps.  After the
// barrier of superstage u each wave reads the first two groups of u + 1 and
// issues the copies of u + 2, spread over the MFMAs of the last two groups of
// u.  The per-row FP32 scales are applied in the epilogue, (acc * sA) * sW,
// before the BF16 rounding.
// ============================================================================
namespace tile_fp8 {
constexpr int kRows = 256;
constexpr int kRowBytes = 128;                   // code bytes (K values) per row per superstage
constexpr int kOpBytes = kRows * kRowBytes;      // 32 KB
constexpr int kSlot = 2 * kOpBytes;              // W rows, then A rows
constexpr int kOutPitch = 2 * kTileN + 16;       // epilogue staging pitch (bytes)
constexpr int kLds = (2 * kSlot > kTileM * kOutPitch) ? 2 * kSlot : kTileM * kOutPitch;
static_assert(kLds <= 160 * 1024, "LDS");
}  // namespace tile_fp8

// VEC: N % 8 == 0 and y 16-byte aligned (whole 16-byte output stores allowed).
template <bool VEC>
__global__ __launch_bounds__(256, 1) void gemm_tile_fp8(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                        const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                        uint16_t* __restrict__ y, int M, int N, int K, int tiles_m,
                                                        int tiles_n) {
    using namespace tile_fp8;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kTileM, n0 = tn * kTileN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = (int64_t)K;
    const int nst = K / 128;

    // code copy i (0..15): W rows for i < 8, A rows for i >= 8; rows 64 * wave + 8 * (i % 8) + lane / 8,
    // the lane fills physical chunk lane % 8 with logical chunk (lane % 8) ^ ((row / 2) % 8)
    const uint8_t* wrow[8];
    const uint8_t* xrow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 64 * wave + 8 * i + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        wrow[i] = qw + (int64_t)min(n0 + row, N - 1) * KB + 16 * chunk;
        xrow[i] = qa + (int64_t)min(m0 + row, M - 1) * KB + 16 * chunk;
    }
    auto issue_code = [&](int u, int i) {  // copy i of superstage min(u, nst - 1) into the slot of u
        uint8_t* slot = lds + (u & 1) * kSlot;
        const int64_t koff = (int64_t)min(u, nst - 1) * kRowBytes;
        if (i < 8) g2lds16(wrow[i] + koff, slot + (8 * wave + i) * 1024);
        else g2lds16(xrow[i - 8] + koff, slot + kOpBytes + (8 * wave + i - 8) * 1024);
    };

    int woff[4], xoff[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int wr = 128 * wn + 32 * f + l32, xr = 128 * wm + 32 * f + l32;
        woff[f] = wr * kRowBytes + ((wr >> 1) & 7);  // low bits: the swizzle key, split off below
        xoff[f] = kOpBytes + xr * kRowBytes + ((xr >> 1) & 7);
    }
    const uint32_t base = lds_addr(lds);
    auto rd_group = [&](v4u (&rw)[4], v4u (&rx)[4], int u, int j) {
        const uint32_t sb = base + (u & 1) * kSlot;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            rw[f] = lds_read16(sb + (woff[f] & ~7) + 16 * ((4 * h + j) ^ (woff[f] & 7)));
            rx[f] = lds_read16(sb + (xoff[f] & ~7) + 16 * ((4 * h + j) ^ (xoff[f] & 7)));
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;

    // one read group: widen half 0 to FP16, run its 16 MFMAs with the widening of half 1 spread
    // between them (one 8-value operand per two MFMAs, so the VALU work hides behind the MFMA
    // pipe), then the 16 MFMAs of half 1; CP copies interleaved, one after every fourth MFMA
    auto group = [&](const v4u (&rw)[4], const v4u (&rx)[4], int cu, int c0, int CP) {
        v8h wa0[4], xv0[4], wa1[4], xv1[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            wa0[f] = e4m3x8_to_f16x8(rw[f][0], rw[f][1]);
            xv0[f] = e4m3x8_to_f16x8(rx[f][0], rx[f][1]);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int i = f * 4 + g;
                acc[f][g] = mfma32_f16(wa0[f], xv0[g], acc[f][g]);
                if (i & 1) {
                    const int k = i >> 1;  // 0..7: W operands 0..3, then A operands 0..3
                    if (k < 4) wa1[k] = e4m3x8_to_f16x8(rw[k][2], rw[k][3]);
                    else xv1[k - 4] = e4m3x8_to_f16x8(rx[k - 4][2], rx[k - 4][3]);
                }
                if (CP && (i & 3) == 3) issue_code(cu, c0 + (i >> 2));
            }
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int i = f * 4 + g;
                acc[f][g] = mfma32_f16(wa1[f], xv1[g], acc[f][g]);
                if (CP && (i & 3) == 3) issue_code(cu, c0 + 4 + (i >> 2));
            }
    };

    // prologue: superstages 0 and 1
#pragma unroll
    for (int i = 0; i < 16; ++i) issue_code(0, i);
#pragma unroll
    for (int i = 0; i < 16; ++i) issue_code(1, i);
    wait_vmcnt<16>();  // this wave's copies of superstage 0 have landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    v4u g0w[4], g0x[4], g1w[4], g1x[4], g2w[4], g2x[4], g3w[4], g3x[4];
    rd_group(g0w, g0x, 0, 0);
    rd_group(g1w, g1x, 0, 1);

    for (int u = 0; u < nst; ++u) {
        // in flight: LDS reads of groups 0, 1 of u; the copies of u + 1
        lds_wait_n<8>(g0w, g0x);
        group(g0w, g0x, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        rd_group(g2w, g2x, u, 2);
        lds_wait_n<8>(g1w, g1x);
        group(g1w, g1x, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        rd_group(g3w, g3x, u, 3);
        lds_wait_n<8>(g2w, g2x);
        lds_wait_n<0>(g3w, g3x);
        wait_vmcnt<0>();               // this wave's copies of u + 1 have landed
        __builtin_amdgcn_s_barrier();  // every wave: done reading u, copies of u + 1 complete
        __builtin_amdgcn_sched_barrier(0);
        rd_group(g0w, g0x, u + 1, 0);  // past the end these read the repeated last superstage: unused
        rd_group(g1w, g1x, u + 1, 1);
        // refill the slot just released with superstage u + 2 (past the end: the last one again,
        // into a slot that is not read any more), one copy after every fourth MFMA
        group(g2w, g2x, u + 2, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        group(g3w, g3x, u + 2, 8, 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();
    lds_wait_n<0>(g0w, g0x);
    lds_wait_n<0>(g1w, g1x);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // Epilogue through LDS: scaled BF16 sub-tiles row-major (padded pitch), then whole 512-byte rows.
    float swv[4][4][4];  // sW of this lane's columns: [f][j][e]
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) swv[f][j][e] = sw[min(n0 + 128 * wn + 32 * f + 8 * j + 4 * h + e, N - 1)];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int ml = 128 * wm + 32 * g + l32;
        const float sxm = sa[min(m0 + ml, M - 1)];
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int nl = 128 * wn + 32 * f + 8 * j + 4 * h;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = ptpc_scaled(acc[f][g][4 * j + e], sxm, swv[f][j][e]);
                uint2 pk;
                pk.x = bf16x2_rne(v[0], v[1]);
                pk.y = bf16x2_rne(v[2], v[3]);
                *reinterpret_cast<uint2*>(lds + ml * kOutPitch + 2 * nl) = pk;
            }
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
        const int ml = 64 * wave + 2 * r + h;
        const int m = m0 + ml;
        const int n = n0 + 8 * l32;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + ml * kOutPitch + 16 * l32);
        if (m >= M) continue;
        uint16_t* dst = y + (int64_t)m * N + n;
        if (VEC && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// ============================================================================
// Tile path, FP8 (E4M3 widened exactly to FP16), 128 x 128 tiles when they fit one round: the copy-wave /
// MFMA-wave split of gemm_tile128_pc_fp4 on E4M3 codes.  A superstage is K = 128 (128 code bytes per row, as
// the FP4 kernels' K = 256) of the 128 weight and 128 activation rows, in a 4-slot ring of 32 KB slots; no
// scales travel (the per-row FP32 scales are applied at the end, (acc * sA) * sW, before the BF16
// rounding).  Waves 4..7 copy (8 copies of 8 rows each per superstage and wave); waves 0..3 each own 2 x 2
// fragments of 32 x 32 and read the row's chunk 4h + j for read group j, which widens into two 8 x FP16
// operands (two k-steps of v_mfma_f32_32x32x16_f16; the other half of each chunk is widened between the
// first half's MFMAs).  KP > 1 splits K into KP parts of K / KP (a multiple of 128) over KP workgroups per
// tile, the accumulators summed by sk::tail_sum (compact slots, sk::workspace_bytes_compact(tiles, KP, 4)
// bytes of zero-filled workspace) before the scales; the workgroup-to-tile mapping is gemm_tile128_pc_fp4's.
// ============================================================================
namespace tile128_fp8 {
constexpr int kRows = 128;
constexpr int kRowBytes = 128;                 // code bytes (K values) per row per superstage
constexpr int kOpBytes = kRows * kRowBytes;    // 16 KB
constexpr int kSlot = 2 * kOpBytes;            // W rows, then A rows
constexpr int kS = 4;                          // ring slots
constexpr int kCopies = 2 * kRows / 32;        // code copies per producer wave and superstage (W, then A)
constexpr int kOutPitch = 2 * kRows + 16;      // epilogue staging pitch (bytes)
constexpr int kLds = kS * kSlot > kRows * kOutPitch ? kS * kSlot : kRows * kOutPitch;
static_assert(kLds <= 160 * 1024, "LDS");
}  // namespace tile128_fp8

template <bool VEC, int KP = 1>
__global__ __launch_bounds__(512, 1) void gemm_tile128_pc_fp8(const uint8_t* __restrict__ qa,
                                                              const float* __restrict__ sa,
                                                              const uint8_t* __restrict__ qw,
                                                              const float* __restrict__ sw, uint16_t* __restrict__ y,
                                                              int M, int N, int K, int tiles_m, int tiles_n,
                                                              uint8_t* __restrict__ ws) {
    using namespace tile128_fp8;
    constexpr int TM = kRows, FW = 2;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];

    int tm, tn, kq = 0, tile = 0;  // kq: this workgroup's K part
    if constexpr (KP == 1) {
        tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    } else {
        const int T = tiles_m * tiles_n, TX = (T + 7) >> 3, r = (int)blockIdx.x >> 3;
        kq = r % KP;
        tile = ((int)blockIdx.x & 7) * TX + r / KP;
        if (tile >= T) return;  // padding of the last XCD's run: no part of any tile
        tm = tile % tiles_m;
        tn = tile / tiles_m;
    }
    const int m0 = tm * TM, n0 = tn * TM;
    const int lane = threadIdx.x & 63;
    const int wave8 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform role
    const int wave = wave8 & 3;
    const int64_t KB = (int64_t)K;
    const int nsup = K / KP / 128;               // superstages of this workgroup's K part
    const int64_t kbase = kq * (KB / KP);        // code bytes of a row before the part

    if (wave8 >= 4) {
        // Producer: copy i moves W rows (i < 4) or A rows 8 (4 wave + i % 4) + lane / 8, the lane filling
        // physical chunk lane % 8 with logical chunk (lane % 8) ^ sk::key(row), conflict-free for the consumers'
        // reads of 8 rows (1.5-2% faster here than the (row / 2) % 8 key).
        const uint8_t* src[kCopies];
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int row = 8 * (4 * wave + (i & 3)) + (lane >> 3);
            const int chunk = (lane & 7) ^ sk::key(row);
            src[i] = i < 4 ? qw + (int64_t)min(n0 + row, N - 1) * KB + 16 * chunk
                           : qa + (int64_t)min(m0 + row, M - 1) * KB + 16 * chunk;
        }
        auto batch = [&](int u) {  // the copies of superstage min(u, nsup - 1) into the slot of u
            uint8_t* slot = lds + (u % kS) * kSlot;
            const int64_t koff = kbase + (int64_t)min(u, nsup - 1) * kRowBytes;
#pragma unroll
            for (int i = 0; i < kCopies; ++i)
                g2lds16(src[i] + koff, slot + (i < 4 ? 0 : kOpBytes) + (4 * wave + (i & 3)) * 1024);
        };
#pragma unroll
        for (int v = 0; v < kS; ++v) batch(v);
        wait_vmcnt<(kS - 1) * kCopies>();  // superstage 0 is in
        __builtin_amdgcn_s_barrier();
        for (int u = 0; u < nsup - kS; ++u) {
            wait_vmcnt<(kS - 2) * kCopies>();  // this wave's copies of u + 1 have landed
            __builtin_amdgcn_s_barrier();
            batch(u + kS);
        }
        static_for<kS>([&](auto t) {
            constexpr int T = decltype(t)::value;
            if (nsup - kS + T >= 0) {
                wait_vmcnt<(kS - 2 - T > 0 ? kS - 2 - T : 0) * kCopies>();
                __builtin_amdgcn_s_barrier();
            }
        });
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // the consumers' barrier before the epilogue: no copy lands after it
    } else {
        // Consumer: 2 x 2 fragments of 32 x 32 (f: weight rows 64 wn + 32 f, g: activation rows 64 wm + 32 g).
        const int wn = wave & 1, wm = wave >> 1;
        const int l32 = lane & 31, h = lane >> 5;
        int woff[FW], xoff[FW];
#pragma unroll
        for (int f = 0; f < FW; ++f) {
            const int wr = 64 * wn + 32 * f + l32, xr = 64 * wm + 32 * f + l32;
            woff[f] = wr * kRowBytes + sk::key(wr);  // low bits: the swizzle key, split off below
            xoff[f] = kOpBytes + xr * kRowBytes + sk::key(xr);
        }
        const uint32_t base = lds_addr(lds);
        // read i (0 .. 2 FW - 1) of group j of superstage u: fragment i / 2 of W (even i) or of A (odd i)
        auto rd_one = [&](v4u (&rw)[FW], v4u (&rx)[FW], int u, int j, int i) {
            const uint32_t sb = base + (u % kS) * kSlot;
            const int f = i >> 1;
            if (i & 1) rx[f] = lds_read16(sb + (xoff[f] & ~7) + 16 * ((4 * h + j) ^ (xoff[f] & 7)));
            else rw[f] = lds_read16(sb + (woff[f] & ~7) + 16 * ((4 * h + j) ^ (woff[f] & 7)));
        };
        v16f acc[FW][FW];
#pragma unroll
        for (int f = 0; f < FW; ++f)
#pragma unroll
            for (int g = 0; g < FW; ++g)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.f;
        // read group (RW, RX): half 0 widened, its FW^2 MFMAs with half 1's widening between them, then half
        // 1's MFMAs; the 2 FW reads of the next group (NW, NX of superstage NU, group NJ) spread over the 2 FW^2
        // MFMAs, one after every FW of them
        auto group = [&](const v4u (&RW)[FW], const v4u (&RX)[FW], v4u (&NW)[FW], v4u (&NX)[FW], int nu, int nj) {
            v8h wa0[FW], xv0[FW], wa1[FW], xv1[FW];
#pragma unroll
            for (int f = 0; f < FW; ++f) {
                wa0[f] = e4m3x8_to_f16x8(RW[f][0], RW[f][1]);
                xv0[f] = e4m3x8_to_f16x8(RX[f][0], RX[f][1]);
            }
#pragma unroll
            for (int f = 0; f < FW; ++f)
#pragma unroll
                for (int g = 0; g < FW; ++g) {
                    const int i = f * FW + g;
                    acc[f][g] = mfma32_f16(wa0[f], xv0[g], acc[f][g]);
                    if (i < FW) wa1[i] = e4m3x8_to_f16x8(RW[i][2], RW[i][3]);  // FW^2 == 2 FW operands
                    else xv1[i - FW] = e4m3x8_to_f16x8(RX[i - FW][2], RX[i - FW][3]);
                    if ((i % FW) == FW - 1) rd_one(NW, NX, nu, nj, i / FW);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
            for (int f = 0; f < FW; ++f)
#pragma unroll
                for (int g = 0; g < FW; ++g) {
                    const int i = f * FW + g;
                    acc[f][g] = mfma32_f16(wa1[f], xv1[g], acc[f][g]);
                    if ((i % FW) == FW - 1) rd_one(NW, NX, nu, nj, FW + i / FW);
                    __builtin_amdgcn_sched_barrier(0);
                }
        };
        __builtin_amdgcn_s_barrier();  // superstage 0 is in
        __builtin_amdgcn_sched_barrier(0);
        v4u g0w[FW], g0x[FW], g1w[FW], g1x[FW], g2w[FW], g2x[FW], g3w[FW], g3x[FW];
#pragma unroll
        for (int i = 0; i < 2 * FW; ++i) rd_one(g0w, g0x, 0, 0, i);
#pragma unroll
        for (int i = 0; i < 2 * FW; ++i) rd_one(g1w, g1x, 0, 1, i);
        // superstage u: groups 0 and 1 (reading groups 2 and 3 meanwhile), the barrier, then groups 2 and 3
        // (reading groups 0 and 1 of u + 1; past the end these read stale slot data, never used)
        for (int u = 0; u < nsup; ++u) {
            lds_wait_n_of<2 * FW, FW>(g0w, g0x);
            __builtin_amdgcn_sched_barrier(0);
            group(g0w, g0x, g2w, g2x, u, 2);
            lds_wait_n_of<2 * FW, FW>(g1w, g1x);
            __builtin_amdgcn_sched_barrier(0);
            group(g1w, g1x, g3w, g3x, u, 3);
            lds_wait_n_of<0, FW>(g2w, g2x);
            lds_wait_n_of<0, FW>(g3w, g3x);
            __builtin_amdgcn_s_barrier();  // every consumer done reading u; every copy of u + 1 landed
            __builtin_amdgcn_sched_barrier(0);
            group(g2w, g2x, g0w, g0x, u + 1, 0);
            group(g3w, g3x, g1w, g1x, u + 1, 1);
        }
        lds_wait_n_of<0, FW>(g0w, g0x);
        lds_wait_n_of<0, FW>(g1w, g1x);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (KP > 1) {
            // the K parts' sum: fragment (f, g) is tail fragment FW f + g, its registers 4 j .. 4 j + 3 the 4
            // consecutive n of one m; scaled and rounded as in the one-part epilogue
            v4f mine[FW * FW][4];
#pragma unroll
            for (int f = 0; f < FW; ++f)
#pragma unroll
                for (int g = 0; g < FW; ++g)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        mine[FW * f + g][j] = v4f{acc[f][g][4 * j], acc[f][g][4 * j + 1], acc[f][g][4 * j + 2],
                                                  acc[f][g][4 * j + 3]};
            auto store_one = [&](int fr, int j, const v4f& v) {
                const int f = fr / FW, g = fr % FW;
                const int m = m0 + 64 * wm + 32 * g + l32, n = n0 + 64 * wn + 32 * f + 8 * j + 4 * h;
                if (m >= M) return;
                const float sxm = sa[m];
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = ptpc_scaled(v[e], sxm, sw[min(n + e, N - 1)]);
                uint16_t* dst = y + (int64_t)m * N + n;
                const uint32_t w2[2] = {bf16x2_rne(o[0], o[1]), bf16x2_rne(o[2], o[3])};
                if (VEC && n + 3 < N) {
                    *reinterpret_cast<uint2*>(dst) = make_uint2(w2[0], w2[1]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) dst[e] = (uint16_t)(w2[e >> 1] >> (16 * (e & 1)));
                }
            };
            sk::tail_sum<FW * FW, KP>(mine, ws, (int)sk::workspace_bytes_compact(tiles_m * tiles_n, KP, FW * FW), tile,
                                      kq, wave, lane, store_one, std::true_type{});
        } else {
            // scaled BF16 sub-tile into LDS (padded pitch) for whole-row stores below
#pragma unroll
            for (int g = 0; g < FW; ++g) {
                const int ml = 64 * wm + 32 * g + l32;
                const float sxm = sa[min(m0 + ml, M - 1)];
#pragma unroll
                for (int f = 0; f < FW; ++f)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int nl = 64 * wn + 32 * f + 8 * j + 4 * h;
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = ptpc_scaled(acc[f][g][4 * j + e], sxm, sw[min(n0 + nl + e, N - 1)]);
                        uint2 pk;
                        pk.x = bf16x2_rne(v[0], v[1]);
                        pk.y = bf16x2_rne(v[2], v[3]);
                        *reinterpret_cast<uint2*>(lds + ml * kOutPitch + 2 * nl) = pk;
                    }
            }
        }
    }
    if constexpr (KP > 1) return;
    __syncthreads();
    // all 8 waves store whole tile rows (2 TM bytes each): wave w rows 16 w .. 16 w + 15
    constexpr int kLanesPerRow = TM / 8;  // 16-byte pieces per tile row
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    const int lr = lane / kLanesPerRow, lc = lane % kLanesPerRow;
#pragma unroll
    for (int r = 0; r < TM / 8 / kRowsPerStore; ++r) {
        const int ml = (TM / 8) * wave8 + kRowsPerStore * r + lr;
        const int m = m0 + ml;
        const int n = n0 + 8 * lc;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + ml * kOutPitch + 16 * lc);
        if (m >= M) continue;
        uint16_t* dst = y + (int64_t)m * N + n;
        if (VEC && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// ============================================================================
// Tile path, FP8 (E4M3 widened exactly to FP16), K % 128 == 0: 256 x 224
// output tiles from 16 x 16 x 32 FP16 MFMAs, four full rounds at N = 7168
// and M = 8192 (as gemm_tile224_fp4).  Same staging: a superstage is K = 128
// (128 code bytes per row) of the 224 weight and 256 activation rows, copied
// with whole-line buffer loads into two 60 KB slots; rows past M or N read as
// zeros.  4 waves in 2 x 2, each 128 (m) x 112 (n), 56 accumulators of 4.
// A superstage is two read steps of four MFMA k-steps: lane group g reads the
// row's chunks 2g (read step 0) and 2g + 1 (read step 1); bytes 0..7 of a
// chunk widen to the 8 FP16 operand values of one k-step, bytes 8..15 to the
// next.  Every E4M3 value is an FP16 normal, and the FP16 MFMA is exact up to
// the FP32 accumulation (the FP8 MFMA drops small products next to large
// ones within groups of 8).  The MFMAs run weight-fragment-major: the 8
// activation operands of a k-step are widened during the k-step before, the
// weight operand of row f + 1 during row f, each tied a row or more before
// its MFMA (the MFMA is inline asm, so these distances are the VALU -> MFMA
// wait states).  Per superstage u: read step 0 with the LDS reads of read
// step 1 between its MFMAs; a barrier once every wave has read all of u and
// its own copies of u + 1 have landed; read step 1 with the copies of u + 2
// and the reads of read step 0 of u + 1 between its MFMAs.  The per-row FP32
// scales are applied in the epilogue, (acc * sA) * sW, before rounding.
// ============================================================================
namespace tile224_fp8 {
constexpr int kTM = 256, kTN = 224;            // activation rows (m), weight rows (n) per tile
constexpr int kFA = 8, kFW = 7;                // 16-row fragments per wave: activation, weight
constexpr int kRowBytes = 128;                 // code bytes (K values) per row per superstage
constexpr int kWBytes = kTN * kRowBytes;       // weight rows first in a slot, then activation rows
constexpr int kSlot = kWBytes + kTM * kRowBytes;
constexpr int kWCopies = kTN / 32, kACopies = kTM / 32;  // code copies per wave and superstage
constexpr int kCodeCopies = kWCopies + kACopies;
constexpr int kOutPitch = 2 * kTN + 16;        // epilogue staging pitch (bytes)
constexpr int kLds = 2 * kSlot > kTM * kOutPitch ? 2 * kSlot : kTM * kOutPitch;
constexpr int kMf = kFW * kFA;                 // MFMAs per wave and k-step
constexpr int kRd = kFW + kFA;                 // LDS reads per wave and read step
static_assert(kLds <= 160 * 1024, "LDS");
}  // namespace tile224_fp8

// VEC: N % 8 == 0 and y 16-byte aligned (whole 16-byte output stores allowed).
// KP > 1: K split into KP parts of K / KP (a multiple of 128) over KP workgroups per tile.  Their FP32
// accumulators (before the scales) are summed in K-part order by sk::tail_sum_chunked in ws (zero-filled
// before first use and left zero; sk::workspace_bytes_chunked(tiles, KP, 56) bytes), and the sum is scaled
// and rounded as the KP == 1 epilogue does; every workgroup of the grid must be resident at once.
// Workgroup b belongs to XCD b % 8's run of tiles x TX .. x TX + TX - 1 (x = b % 8, TX = ceil(tiles / 8),
// tile t = tm + tiles_m tn), as part (b / 8) % KP of tile x TX + (b / 8) / KP: the parts of a tile sit on one
// XCD.  KP == 1 follows tile_coords.
template <bool VEC, int KP = 1>
__global__ __launch_bounds__(256, 1) void gemm_tile224_fp8(const uint8_t* __restrict__ qa,
                                                           const float* __restrict__ sa,
                                                           const uint8_t* __restrict__ qw,
                                                           const float* __restrict__ sw, uint16_t* __restrict__ y,
                                                           int M, int N, int K, int tiles_m, int tiles_n,
                                                           uint8_t* __restrict__ ws) {
    using namespace tile224_fp8;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];

    int tm, tn, kq = 0, tile = 0;  // kq: this workgroup's K part
    if constexpr (KP == 1) {
        tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    } else {
        const int T = tiles_m * tiles_n, TX = (T + 7) >> 3, r = (int)blockIdx.x >> 3;
        kq = r % KP;
        tile = ((int)blockIdx.x & 7) * TX + r / KP;
        if (tile >= T) return;  // padding of the last XCD's run: no part of any tile
        tm = tile % tiles_m;
        tn = tile / tiles_m;
    }
    const int m0 = tm * kTM, n0 = tn * kTN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar registers
    const int wn = wave & 1, wm = wave >> 1;
    const int l16 = lane & 15, g = lane >> 4;
    const int KB = K;  // code bytes per row
    const int nsup = K / KP / 128;  // superstages of this workgroup's K part
    const int kbase = kq * (K / KP);  // code bytes of a row before the part

    // code copies as in gemm_tile224_fp4: buffer loads with the operand's size as the range (the
    // host keeps rows * K below 2^31), rows 8 (copies per wave * wave + i) + lane / 8, physical chunk
    // lane % 8 holding logical chunk (lane % 8) ^ ((row / 2) % 8)
    constexpr int kRawBufferWord3 = 0x00020000;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)qw, (short)0, N * KB, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)qa, (short)0, M * KB, kRawBufferWord3);
    uint32_t coff[kCodeCopies];
    int cdst[kCodeCopies];
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i) {
        const bool isw = i < kWCopies;
        const int row = isw ? 8 * (kWCopies * wave + i) + (lane >> 3) : 8 * (kACopies * wave + i - kWCopies) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        coff[i] = (uint32_t)(((isw ? n0 : m0) + row) * KB + 16 * chunk);
        cdst[i] = isw ? (kWCopies * wave + i) * 1024 : kWBytes + (kACopies * wave + i - kWCopies) * 1024;
    }
    auto issue_code = [&](int u, int i) {  // copy i of superstage min(u, nsup - 1) into the slot of u
        const int koff = kbase + min(u, nsup - 1) * kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(i < kWCopies ? wrsrc : arsrc,
                                                 (__attribute__((address_space(3))) void*)(lds + (u & 1) * kSlot + cdst[i]),
                                                 16, coff[i], koff, 0, 0);
    };

    // LDS addressing: per-lane bases plus immediates (the swizzle key is l16 / 2 for every fragment)
    const int key = l16 >> 1;
    const uint32_t base = lds_addr(lds);
    const uint32_t wrow0 = ((kTN / 2) * wn + l16) * kRowBytes, xrow0 = kWBytes + ((kTM / 2) * wm + l16) * kRowBytes;
    const uint32_t ck0 = 16 * ((2 * g) ^ key), ck1 = 16 * ((2 * g + 1) ^ key);
    auto slot_of = [&](int u) { return base + (u & 1) * kSlot; };
    // read i (0 .. kRd - 1) of a read step: weight fragment i, then activation fragment i - kFW
    auto rd_one = [&](v4u (&rw)[kFW], v4u (&rx)[kFA], uint32_t wb, uint32_t xb, auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < kFW) rw[i] = lds_read16_at<i * 16 * kRowBytes>(wb);
        else rx[i - kFW] = lds_read16_at<(i - kFW) * 16 * kRowBytes>(xb);
    };
    // half HF of a raw 16-byte chunk widened to one 8 x FP16 operand
    auto widen = [](const v4u& r, auto hc) -> v8h {
        constexpr int hf = decltype(hc)::value;
        return hf == 0 ? e4m3x8_to_f16x8(r[0], r[1]) : e4m3x8_to_f16x8(r[2], r[3]);
    };

    v4f acc[kFW][kFA];
#pragma unroll
    for (int f = 0; f < kFW; ++f)
#pragma unroll
        for (int j = 0; j < kFA; ++j) {
            acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+a"(acc[f][j]));
        }
    wait_states8<2>();  // VALU writes of the accumulators -> first MFMA

    // prologue: superstages 0 and 1
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i) issue_code(0, i);
#pragma unroll
    for (int i = 0; i < kCodeCopies; ++i) issue_code(1, i);
    wait_vmcnt<kCodeCopies>();  // superstage 0 is in
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    v4u r0w[kFW], r0x[kFA], r1w[kFW], r1x[kFA];  // raw chunks of read steps 0 and 1
    v8h xa[kFA], xb_[kFA], wa[2];                 // widened activation operands (this / next k-step), weight
    static_for<kRd>([&](auto ic) { rd_one(r0w, r0x, slot_of(0) + wrow0 + ck0, slot_of(0) + xrow0 + ck0, ic); });
    lds_wait<0>();
    lds_tie(r0w);
    lds_tie(r0x);
    static_for<kFA>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        xa[j] = widen(r0x[j], std::integral_constant<int, 0>{});
        vgpr_tie(xa[j]);
    });
    wa[0] = widen(r0w[0], std::integral_constant<int, 0>{});
    vgpr_tie(wa[0]);
    wait_states8<1>();
    __builtin_amdgcn_sched_barrier(0);

    // One MFMA k-step (half HF of the raw sets RW / RX), weight-fragment-major.  Row f uses the
    // weight operand wa[(f + P) % 2] and every activation operand XC.  Between the MFMAs it widens the
    // weight operand of row f + 1 (after MFMA 1 of row f; for the last row, row 0 of the next k-step
    // from NW, half NHF, into wa[P ^ 1], the register that k-step's row 0 uses with parity P ^ 1) and
    // activation operand f of the next k-step into XN (after MFMA 4 of row f; operand 7 after MFMA 6
    // of row 6), from NX half NHF.  Each widened operand is tied at least 7 MFMAs before its first
    // use.  EXTRA(i) adds the k-step's other work after MFMA i.
    auto kstep = [&](const v8h (&XC)[kFA], v8h (&XN)[kFA], const v4u (&RW)[kFW], const v4u (&NW)[kFW],
                     const v4u (&NX)[kFA], auto hc, auto nhc, auto pc, auto&& extra) {
        constexpr int nhf = decltype(nhc)::value, P = decltype(pc)::value;
        static_for<kMf>([&](auto ic) {
            constexpr int i = decltype(ic)::value, f = i / kFA, j = i % kFA;
            mfma16_f16_agpr(acc[f][j], wa[(f + P) & 1], XC[j]);
            if constexpr (j == 1) {
                constexpr int r = (f + 1 + P) & 1;
                if constexpr (f + 1 < kFW) wa[r] = widen(RW[f + 1], hc);
                else wa[r] = widen(NW[0], nhc);
                vgpr_tie(wa[r]);
            }
            if constexpr (j == 4 || (f == kFW - 1 && j == 6)) {
                constexpr int x = j == 4 ? f : kFA - 1;
                XN[x] = widen(NX[x], std::integral_constant<int, nhf>{});
                vgpr_tie(XN[x]);
            }
            extra(ic);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    static_assert(kFW % 2 == 1 && kFA == kFW + 1, "the operand schedule assumes 7 x 8 fragments");
    auto none = [](auto) {};

    // superstage u; REFILL: issue the copies of u + 2 (the last two superstages have none to issue,
    // so neither their barriers nor the epilogue wait for copies past the end)
    auto step = [&](int u, auto REFILL) __attribute__((always_inline)) {
        // read step 0 (chunk 2g): k-step (0, 0) from xa, widening (0, 1) into xb_; k-step (0, 1) from
        // xb_, widening (1, 0) into xa once the reads of read step 1 are in.  The reads of read step 1
        // go out during k-step (0, 0).
        {
            const uint32_t wb = slot_of(u) + wrow0 + ck1, xb = slot_of(u) + xrow0 + ck1;
            kstep(xa, xb_, r0w, r0w, r0x, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{},
                  std::integral_constant<int, 0>{},
                  [&](auto ic) {
                      constexpr int i = decltype(ic)::value;
                      static_for<kRd>([&](auto rc) {
                          if constexpr ((decltype(rc)::value * kMf) / kRd == i) rd_one(r1w, r1x, wb, xb, rc);
                      });
                  });
        }
        lds_wait<0>();
        lds_tie(r1w);
        lds_tie(r1x);
        __builtin_amdgcn_sched_barrier(0);
        // widening for k-step (1, 0) reads xa's registers; the MFMAs of (0, 1) read xb_ (not xa)
        kstep(xb_, xa, r0w, r1w, r1x, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{},
              std::integral_constant<int, 1>{}, none);
        wait_vmcnt<0>();  // this wave's copies of u + 1 have landed
        __builtin_amdgcn_s_barrier();  // every wave: done reading u, copies of u + 1 complete
        __builtin_amdgcn_sched_barrier(0);
        // read step 1 (chunk 2g + 1): k-step (1, 0) from xa, widening (1, 1) into xb_, with the copies
        // of u + 2 and the reads of read step 0 of u + 1; k-step (1, 1) from xb_, widening (0, 0) of
        // u + 1 into xa (past the end these read stale slot data, never used)
        {
            const uint32_t wb = slot_of(u + 1) + wrow0 + ck0, xb = slot_of(u + 1) + xrow0 + ck0;
            kstep(xa, xb_, r1w, r1w, r1x, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{},
                  std::integral_constant<int, 0>{},
                  [&](auto ic) {
                      constexpr int i = decltype(ic)::value;
                      static_for<kCodeCopies>([&](auto cc) {
                          if constexpr (decltype(REFILL)::value && (decltype(cc)::value * kMf) / kCodeCopies == i)
                              issue_code(u + 2, decltype(cc)::value);
                      });
                      static_for<kRd>([&](auto rc) {
                          if constexpr ((decltype(rc)::value * kMf) / kRd == i) rd_one(r0w, r0x, wb, xb, rc);
                      });
                  });
        }
        lds_wait<0>();
        lds_tie(r0w);
        lds_tie(r0x);
        __builtin_amdgcn_sched_barrier(0);
        kstep(xb_, xa, r1w, r0w, r0x, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{},
              std::integral_constant<int, 1>{}, none);
    };
    for (int u = 0; u < nsup - 2; ++u) step(u, std::true_type{});
    if (nsup >= 2) step(nsup - 2, std::false_type{});  // K = 128: one superstage
    step(nsup - 1, std::false_type{});
    wait_vmcnt<0>();
    wait_states8<3>();  // last MFMA -> reads of the accumulators (tied here, so none moves above)
#pragma unroll
    for (int f = 0; f < kFW; ++f)
#pragma unroll
        for (int j = 0; j < kFA; ++j) asm volatile("" : "+a"(acc[f][j]));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (KP > 1) {
        // the K parts' sum: accumulator u = f kFA + j of a lane is the 4 consecutive n of one m stored below,
        // scaled and rounded as in the epilogue that follows
        auto mine = [&](auto uc) -> v4f {
            constexpr int u = decltype(uc)::value;
            return acc[u / kFA][u % kFA];
        };
        auto store_one = [&](int u, const v4f& v) {
            const int f = u / kFA, j = u % kFA;
            const int m = m0 + (kTM / 2) * wm + 16 * j + l16, n = n0 + (kTN / 2) * wn + 16 * f + 4 * g;
            if (m >= M) return;
            const float sxm = sa[m];
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = ptpc_scaled(v[e], sxm, sw[min(n + e, N - 1)]);
            uint16_t* dst = y + (int64_t)m * N + n;
            const uint32_t w2[2] = {bf16x2_rne(o[0], o[1]), bf16x2_rne(o[2], o[3])};
            if (VEC && n + 3 < N) {
                *reinterpret_cast<uint2*>(dst) = make_uint2(w2[0], w2[1]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) dst[e] = (uint16_t)(w2[e >> 1] >> (16 * (e & 1)));
            }
        };
        const int ws_range = (int)sk::workspace_bytes_chunked(tiles_m * tiles_n, KP, kMf);
        sk::tail_sum_chunked<kMf, KP, 7>(mine, ws, ws_range, tile, kq, wave, lane, store_one);
        return;
    }

    // Epilogue through LDS: acc * sA[m] * sW[n] (in FP64) rounded to BF16, each lane 4 consecutive n of one
    // m per fragment pair; then whole 448-byte tile rows.
    float sxm[kFA];
#pragma unroll
    for (int j = 0; j < kFA; ++j) sxm[j] = sa[min(m0 + (kTM / 2) * wm + 16 * j + l16, M - 1)];
#pragma unroll
    for (int f = 0; f < kFW; ++f) {
        const int nl = (kTN / 2) * wn + 16 * f + 4 * g;
        float swn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) swn[e] = sw[min(n0 + nl + e, N - 1)];
#pragma unroll
        for (int j = 0; j < kFA; ++j) {
            const int ml = (kTM / 2) * wm + 16 * j + l16;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = ptpc_scaled(acc[f][j][e], sxm[j], swn[e]);
            uint2 pk;
            pk.x = bf16x2_rne(v[0], v[1]);
            pk.y = bf16x2_rne(v[2], v[3]);
            *reinterpret_cast<uint2*>(lds + ml * kOutPitch + 2 * nl) = pk;
        }
    }
    __syncthreads();
    constexpr int kPieces = kTN / 8;  // 16-byte pieces per tile row
#pragma unroll 4
    for (int it = 0; it < kPieces; ++it) {  // wave w stores tile rows 64 w .. 64 w + 63
        const int p = 64 * it + lane;
        const int row = p / kPieces, col = p - kPieces * row;
        const int ml = 64 * wave + row;
        const int m = m0 + ml, n = n0 + 8 * col;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + ml * kOutPitch + 16 * col);
        if (m >= M) continue;
        uint16_t* dst = y + (int64_t)m * N + n;
        if (VEC && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
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
    const bool scales16 = ((reinterpret_cast<uintptr_t>(sa) | reinterpret_cast<uintptr_t>(sw)) & 15) == 0;
    if (!FP8 && M <= 64 && K % 2048 == 0 && K <= 1024 * dec4::kMaxMine && scales16) {
        const dim3 grid((unsigned)((N + dec4::kNT - 1) / dec4::kNT));
        const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
        const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
        // M <= 32: a 2-slot ring measured faster than 3 or 4 slots (M = 1, 16, 32 at K = 8192:
        // 8.5 -> 8.0, 8.9 -> 8.3, 9.5 -> 9.0 us)
        if (M <= 32 && K <= 8192)
            hipLaunchKernelGGL((gemm_decode_fp4<1, 2, 256>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
        else if (M <= 32)
            hipLaunchKernelGGL((gemm_decode_fp4<1, 4, 512>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
        else if (K <= 8192)
            hipLaunchKernelGGL((gemm_decode_fp4<2, 2, 256>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
        else
            hipLaunchKernelGGL((gemm_decode_fp4<2, 2, 512>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
    } else if (!FP8 && M <= 128 && K % 2048 == 0 && K <= 8192 && scales16) {
        // two row halves of 64 rows: the per-wave slabs of the M = 64 kernel, and every CU reads the
        // activations once (128 scale rows + 32: a 40 KB scale block beside the 96 KB ring)
        hipLaunchKernelGGL((gemm_decode_fp4<2, 2, 256, false, 2>), dim3((unsigned)((N + dec4::kNT - 1) / dec4::kNT)),
                           dim3(256), 0, st, a, reinterpret_cast<const uint8_t*>(sa), w,
                           reinterpret_cast<const uint8_t*>(sw), out, m, n, k, nullptr);
    } else if (!FP8 && M <= 128 && K % 512 == 0) {
        const dim3 grid((unsigned)((N + 31) / 32));
        const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
        const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
        if (M <= 16)
            hipLaunchKernelGGL((gemm_decode_lds_fp4<1>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
        else if (M <= 32)
            hipLaunchKernelGGL((gemm_decode_lds_fp4<2>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
        else if (M <= 64)
            hipLaunchKernelGGL((gemm_decode_lds_fp4<4>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
        else
            hipLaunchKernelGGL((gemm_decode_lds_fp4<8>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                               nullptr);
    } else if (FP8 && M <= 64 && K % 512 == 0) {
        const dim3 grid((unsigned)((N + dec8::kNT - 1) / dec8::kNT));
        const float* sa32 = reinterpret_cast<const float*>(sa);
        const float* sw32 = reinterpret_cast<const float*>(sw);
        if (M <= 32)
            hipLaunchKernelGGL((gemm_decode_fp8<1, 5>), grid, dim3(256), 0, st, a, sa32, w, sw32, out, m, n, k);
        else
            hipLaunchKernelGGL((gemm_decode_fp8<2, 3>), grid, dim3(256), 0, st, a, sa32, w, sw32, out, m, n, k);
    } else if (FP8 && M <= 128 && K % 512 == 0) {
        // two row halves of 64 rows (the per-wave slabs of the M = 64 kernel)
        hipLaunchKernelGGL((gemm_decode_fp8<2, 3, 2>), dim3((unsigned)((N + dec8::kNT - 1) / dec8::kNT)), dim3(256),
                           0, st, a, reinterpret_cast<const float*>(sa), w, reinterpret_cast<const float*>(sw), out, m,
                           n, k);
    } else if (M <= 128) {
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
        const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
        const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
        const bool vec16 = N % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
        // FP8: 256 x 224 tiles when they take fewer rounds on 256 CUs (see the FP4 branch)
        const int tn224 = (int)((N + tile224_fp8::kTN - 1) / tile224_fp8::kTN);
        const int64_t t256 = (int64_t)tiles_m * tiles_n, t224 = (int64_t)tiles_m * tn224;
        const bool fp8_224 = FP8 && 7 * ((t224 + 255) / 256) < 8 * ((t256 + 255) / 256) &&
                             (M > N ? M : N) * K < ((int64_t)1 << 31);
        if (fp8_224 && vec16)
            hipLaunchKernelGGL((gemm_tile224_fp8<true, 1>), dim3((unsigned)t224), dim3(256), 0, st, a,
                               reinterpret_cast<const float*>(sa), w, reinterpret_cast<const float*>(sw), out, m, n, k,
                               tiles_m, tn224, nullptr);
        else if (fp8_224)
            hipLaunchKernelGGL((gemm_tile224_fp8<false, 1>), dim3((unsigned)t224), dim3(256), 0, st, a,
                               reinterpret_cast<const float*>(sa), w, reinterpret_cast<const float*>(sw), out, m, n, k,
                               tiles_m, tn224, nullptr);
        else if (FP8 && vec16)
            hipLaunchKernelGGL(gemm_tile_fp8<true>, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, a,
                               reinterpret_cast<const float*>(sa), w, reinterpret_cast<const float*>(sw), out, m, n, k,
                               tiles_m, tiles_n);
        else if (FP8)
            hipLaunchKernelGGL(gemm_tile_fp8<false>, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, a,
                               reinterpret_cast<const float*>(sa), w, reinterpret_cast<const float*>(sw), out, m, n, k,
                               tiles_m, tiles_n);
        else if (!FP8 && K % 512 == 0 && scales16) {
            // 128-row tiles when 256-row tiles would leave many CUs idle: up to about 160 256-tiles
            // (on 256 CUs) four times as many 128-tiles finish sooner.  Otherwise 256 x 224 tiles when
            // they fill the CUs in fewer rounds (a round of them costs 7/8 of a round of 256 x 256
            // tiles; N = 7168 is 32 tiles of 224), else 256 x 256.
            constexpr int64_t kCUs = 256;
            const int64_t t256 = (int64_t)tiles_m * tiles_n;
            const bool small = t256 <= 160;
            const int tm128 = (int)((M + 127) / 128), tn128 = (int)((N + 127) / 128);
            const int tn224 = (int)((N + tile224::kTN - 1) / tile224::kTN);
            const int64_t t224 = (int64_t)tiles_m * tn224;
            const bool use224 = 7 * ((t224 + kCUs - 1) / kCUs) < 8 * ((t256 + kCUs - 1) / kCUs) &&
                                (M > N ? M : N) * (K / 2) < ((int64_t)1 << 31);
            const dim3 g256((unsigned)t256), g128((unsigned)(tm128 * tn128)), g224((unsigned)t224);
            // at most one 128-tile per CU: the deeper ring (152 KB of LDS) with copy and MFMA waves; more: two
            // 4-wave workgroups per CU
            const bool deep = (int64_t)tm128 * tn128 <= kCUs;
            if (small && deep && vec16)
                hipLaunchKernelGGL((gemm_tile128_pc_fp4<true, 1>), g128, dim3(512), 0, st, a, sa8, w, sw8, out, m, n,
                                   k, tm128, tn128, nullptr);
            else if (small && deep)
                hipLaunchKernelGGL((gemm_tile128_pc_fp4<false, 1>), g128, dim3(512), 0, st, a, sa8, w, sw8, out, m, n,
                                   k, tm128, tn128, nullptr);
            else if (small && vec16)
                hipLaunchKernelGGL((gemm_tile_fp4<true, 128>), g128, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                                   tm128, tn128);
            else if (small)
                hipLaunchKernelGGL((gemm_tile_fp4<false, 128>), g128, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                                   tm128, tn128);
            else if (use224 && vec16)
                hipLaunchKernelGGL(gemm_tile224_fp4<true>, g224, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                                   tiles_m, tn224);
            else if (use224)
                hipLaunchKernelGGL(gemm_tile224_fp4<false>, g224, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                                   tiles_m, tn224);
            else if (vec16)
                hipLaunchKernelGGL((gemm_tile_fp4<true, 256>), g256, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                                   tiles_m, tiles_n);
            else
                hipLaunchKernelGGL((gemm_tile_fp4<false, 256>), g256, dim3(256), 0, st, a, sa8, w, sw8, out, m, n, k,
                                   tiles_m, tiles_n);
        }
        else if (!FP8 && K % 256 == 0)
            hipLaunchKernelGGL(gemm_tile_dma_fp4<4>, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, a,
                               reinterpret_cast<const uint8_t*>(sa), w, reinterpret_cast<const uint8_t*>(sw), out, m, n,
                               k, tiles_m, tiles_n);
        else if constexpr (!FP8) {  // the FP8 branches above take every K
            if (N % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0)
                hipLaunchKernelGGL(gemm_tile_kernel<true>, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, a,
                                   sa8, w, sw8, out, m, n, k, tiles_m, tiles_n);
            else
                hipLaunchKernelGGL(gemm_tile_kernel<false>, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, st, a,
                                   sa8, w, sw8, out, m, n, k, tiles_m, tiles_n);
        }
    }
    return hipGetLastError();
}

// Grouped A4W4 decode GEMM (MoE experts): grid (N / 32, G); max_rows (the largest group, or a bound on it)
// picks 32- or 64-row chunks - every row of every group is written either way.  K % 512 == 0, K <= 16384,
// all code and scale pointers 16-byte aligned (checked by the caller, which takes gemm_grouped_fp4 of
// gemm_splitk.hpp instead where that measured faster): K % 2048 == 0 with max_rows <= 32 takes the decode
// ring in 32-row chunks, everything else the LDS-staged decode kernel.
inline hipError_t launch_gemm_a4w4_grouped(const void* qa, const void* sa, const void* qw, const void* sw, void* y,
                                           const int32_t* offsets, int64_t G, int64_t max_rows, int64_t N, int64_t K,
                                           hipStream_t st) {
    const uint8_t* a = reinterpret_cast<const uint8_t*>(qa);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(qw);
    const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* sw8 = reinterpret_cast<const uint8_t*>(sw);
    uint16_t* out = reinterpret_cast<uint16_t*>(y);
    const int n = (int)N, k = (int)K;
    const dim3 grid((unsigned)((N + dec4::kNT - 1) / dec4::kNT), (unsigned)G);
    if (K % 2048 != 0 || max_rows > 32) {  // (the caller sends max_rows > 32 with K % 1024 == 0 to the tiles)
        if (max_rows <= 32)
            hipLaunchKernelGGL((gemm_decode_lds_fp4<2, true>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, 0, n, k,
                               offsets);
        else
            hipLaunchKernelGGL((gemm_decode_lds_fp4<4, true>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, 0, n, k,
                               offsets);
        return hipGetLastError();
    }
    if (K <= 8192)
        hipLaunchKernelGGL((gemm_decode_fp4<1, 2, 256, true>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, 0, n, k,
                           offsets);
    else
        hipLaunchKernelGGL((gemm_decode_fp4<1, 4, 512, true>), grid, dim3(256), 0, st, a, sa8, w, sw8, out, 0, n, k,
                           offsets);
    return hipGetLastError();
}

}  // namespace mx
