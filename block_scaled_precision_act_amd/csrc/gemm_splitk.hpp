// gemm_splitk.hpp - decode-size GEMMs with K split across workgroups (gfx950):
//   gemm_splitk_fp4     A4W4, M <= 64 (and the one-launch layer, FUSED)
//   gemm_splitk_fp4_rh  A4W4, 64 < M <= 128, in two 64-row halves
//   gemm_splitk_fp8     PTPC A8W8, 33 <= M <= 64
// all sharing one tail (sk::tail_sum), and gemm_grouped_fp4 (MoE experts, K % 1024 == 0), the first's
// tile body walking K in parts within the workgroup.  The tail also sums the K parts of the tile kernels
// of gemm_kernels.hpp that split K (the 128-row tiles with copy and MFMA waves, in compact slots; the FP8
// 256 x 224 tile through sk::tail_sum_chunked).  The design, described for the first:
//
// The layer ("Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact quantization
// coverage": weight (7168, 8192) MXFP4 with (7168, 256) E8M0 scales, dynamic
// MXFP4 activations) is bound by the weight stream at decode sizes (M <= 64):
// the weight is 96% of the bytes.  When one workgroup owns a few output
// columns over all of K, every CU also reads the whole activation matrix
// (256 KB at M = 64, K = 8192) beside its 128 KB share of the weight.  Here a
// workgroup owns a 128-column tile and one of KP contiguous K parts:
//
//   * its K part of the activation codes (32 MF rows x K/KP/2 bytes, at most
//     64 KB) is copied into LDS once, with the activation and weight scales of
//     the part; so a CU reads 1/KP of the activations;
//   * its 4 waves own 32 columns each and stream their weight rows through a
//     private LDS ring of S slabs (K = 256, 128 bytes per row, whole cache
//     lines per copy), waiting only for their own copies: no barrier in the
//     main loop.  The order of a workgroup's slabs is rotated by its tile, so
//     the workgroups streaming at one moment spread over the HBM channels;
//   * the KP partial tiles of a column group (tile, wave: 32 MF x 32 FP32) are
//     summed across workgroups slice by slice: part p < min(KP, 4 MF) owns one
//     slice, every wave stores the slices it does not own into their owners'
//     workspace slots without waiting, and each owner polls its slots until
//     every word has arrived, adds the KP slices in K-part order (0, 1, ...,
//     KP - 1: deterministic, whatever the arrival order), writes BF16 and
//     clears the slots.  So the tail costs one L2 round trip after the last
//     partial lands, not a store-acknowledge, a counter and a read in turn.
//
// An owner waits for other workgroups, so every workgroup of the grid must be
// resident at once: the host launches this kernel only when the grid (at most
// 256 workgroups, one per CU, as the LDS block rules out two) fits the
// device's CUs.  The KP workgroups of a tile are blockIdx t % 8 + 8 (KP (t / 8)
// + q): equal modulo 8, which places them on one XCD (workgroups are dealt
// round-robin to the XCDs), so the partials meet in that XCD's L2 without
// cache maintenance; polls read with device-scope coherence (never from the
// CU's L1).  The workspace must be zero-filled before its first use; every
// launch leaves it all zero, so one workspace serves launches of any shapes in
// turn.  Launches that share a workspace must not overlap.
#pragma once

#include "mx_device.hpp"

namespace mx {

namespace sk {
constexpr int kTN = 128;    // output columns per tile (4 waves x 32)
constexpr int kSlab = 128;  // code bytes per row per slab (K = 256)
// XOR key of a 128-byte line's 16-byte chunks: any 8 consecutive rows get 8 distinct keys, so the
// MFMA-layout ds_read_b128s of 8 rows (one LDS cycle) hit distinct banks
__device__ __forceinline__ int key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// MF: 32-row activation fragments (M <= 32 MF); S: weight ring slots per wave; NSL: slabs per K part
template <int MF, int S, int NSL>
struct Cfg {
    static constexpr int kArows = 32 * MF;
    static constexpr int kAct = kArows * NSL * kSlab;        // activation codes of the K part
    static constexpr int kP = NSL / 2;                       // 16-byte scale pieces per row
    static constexpr int kScRows = kArows + kTN;             // activation rows, then weight rows
    static constexpr int kSc = kScRows * 8 * NSL;            // scale bytes of the K part
    static constexpr int kRingWave = S * 32 * kSlab;         // 4 KB per slot
    static constexpr int kLds = kAct + kSc + 4 * kRingWave;
    static constexpr int kActCopies = kAct / 1024;
    static constexpr int kScCopies = kScRows * kP / 64;
    static_assert(NSL % 2 == 0 && NSL >= S, "slabs per part");
    static_assert((kScRows * kP) % 64 == 0, "scale copies");
    static_assert(kActCopies % 4 == 0, "activation copies per wave");
    static_assert(S * 4 <= 63, "vmcnt");
    static_assert(kLds <= 160 * 1024, "LDS");
};

// Workspace: the partial slots of every column group (tile, wave), KP x MF x 4 KB per group.  A launch has
// at most kMaxGrid workgroups (all resident at once, one per CU), so at most 8 MiB; every A4W4 plan (the
// compact slots of the two-part 128-row tile included) stays within it.  The FP8 256 x 224 tile's chunked
// slots (workspace_bytes_chunked, two K parts) take up to 28 MiB of the A8W8 caller's workspace.
constexpr int kMaxGrid = 256;
__host__ __device__ inline size_t workspace_bytes(int tiles, int KP, int MF) {
    return (size_t)tiles * KP * 4 * MF * 4096;
}
constexpr size_t kMaxWorkspaceBytes = (size_t)kMaxGrid * 4 * 2 * 4096;
// The compact layout (tail_sum<..., true>) keeps only the slots that are written: KP - 1 per slice.
__host__ __device__ inline size_t workspace_bytes_compact(int tiles, int KP, int MF) {
    return (size_t)tiles * (KP - 1) * 4 * MF * 4096;
}
// tail_sum_chunked's slots: KP - 1 slots of NF / KP float4s per lane for each slice of each (tile, wave).
__host__ __device__ inline size_t workspace_bytes_chunked(int tiles, int KP, int NF) {
    return (size_t)tiles * 4 * (KP - 1) * NF * 1024;
}
}  // namespace sk

// FUSED prologue: quantize rows 0 .. M-1 of BF16 X, K-values 256 s0 .. 256 (s0 + NSL) - 1, into the LDS
// activation block and scale rows of the split-K kernel, bit for bit as mx_quant_act_bf16 does.  A row's
// part is NSL / 2 pieces of 1 KB; one wave instruction loads a whole piece (whole cache lines), so a 32-value
// block (64 bytes) spans the four lanes of a quad: lane l holds values 8 (l % 4) .. +7 of block 16 k + l / 4
// of piece k.  The block's exponent maximum is reduced over the quad (DPP lane swaps), each lane converts
// its eight values and writes their 4 code bytes to the block's 16-byte chunk, and the quad writes the
// scale byte.  Wave w takes pieces w, w + 4, ... in chunks of kB, two chunks in flight (the next chunk's
// loads are issued before the current one is converted); a chunk's loads are unconditional (pieces past
// the wave's count reload its last piece, not converted), so the compiler's waits count exactly one chunk.
// Rows at or past M are not written (they only feed output rows that are never stored).
template <int MF, int S, int NSL, int kB>
__device__ __forceinline__ void quantize_chunks(const uint8_t* __restrict__ x, int K, int s0, int wave, int lane,
                                                int count, uint8_t* actb, uint8_t* scb) {
    using C = sk::Cfg<MF, S, NSL>;
    constexpr int kPieces = NSL / 2;  // 1 KB pieces per row
    const int pc = lane & 3;
    auto load = [&](uint4 (&v)[kB], int n0) {
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int i = wave + 4 * min(n0 + u, count - 1);
            const int r = i / kPieces, k = i % kPieces;
            v[u] = ldg16(x + ((int64_t)r * K + (int64_t)s0 * 256 + 512 * k) * 2 + 16 * lane);
        }
    };
    auto convert = [&](const uint4 (&v)[kB], int n0) {
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (n0 + u >= count) break;  // wave-uniform
            const int i = wave + 4 * (n0 + u);
            const int r = i / kPieces, k = i % kPieces;
            const uint32_t scale = mx_scale_of_emax(quad_max(bf16x8_emax(v[u])));
            const uint32_t codes = bf16x8_codes(v[u], scale);
            const int b = 16 * k + (lane >> 2);  // block within the part
            const int j = b >> 3, c = b & 7;     // slab and chunk within the slab's 128-byte line
            *reinterpret_cast<uint32_t*>(actb + (r * NSL + j) * sk::kSlab + 16 * (c ^ sk::key(r)) + 4 * pc) =
                scale == 0xffu ? 0u : codes;
            scb[r * 8 * NSL + 16 * ((b / 16 + r) % C::kP) + (b & 15)] = (uint8_t)scale;
        }
    };
    uint4 va[kB], vb[kB];
    load(va, 0);
    for (int n0 = 0; n0 < count; n0 += 2 * kB) {
        if (n0 + kB < count) {
            load(vb, n0 + kB);
            convert(va, n0);
            if (n0 + 2 * kB < count) {
                load(va, n0 + 2 * kB);
                convert(vb, n0 + kB);
            } else {
                convert(vb, n0 + kB);
            }
        } else {
            convert(va, n0);
        }
    }
}

template <int MF, int S, int NSL>
__device__ __forceinline__ void quantize_part(const uint8_t* __restrict__ x, int M, int K, int s0, int wave, int lane,
                                              uint8_t* actb, uint8_t* scb) {
    const int count = (M * (NSL / 2) - wave + 3) / 4;  // pieces of this wave
    if (count <= 0) return;
    if (count <= 4) quantize_chunks<MF, S, NSL, 2>(x, K, s0, wave, lane, count, actb, scb);
    else if (count <= 16) quantize_chunks<MF, S, NSL, 8>(x, K, s0, wave, lane, count, actb, scb);
    else quantize_chunks<MF, S, NSL, 16>(x, K, s0, wave, lane, count, actb, scb);
}

namespace sk {
// Partial sums cross workgroups as 32-bit words, complemented, with every NaN made the quiet NaN
// 0x7FC00000 first: a stored word is never 0, so a 0 word reads as "not written yet".  Both tails leave
// every word they wrote at 0 again before the launch ends, so the partial area is all 0 between launches.
__device__ __forceinline__ uint32_t partial_word(float v) { return ~(v != v ? 0x7FC00000u : __float_as_uint(v)); }
__device__ __forceinline__ float partial_value(uint32_t w) { return __uint_as_float(~w); }
__device__ __forceinline__ v4u partial_words(const v4f& v) {
    return v4u{partial_word(v[0]), partial_word(v[1]), partial_word(v[2]), partial_word(v[3])};
}
__device__ __forceinline__ v4f partial_values(const v4u& w) {
    return v4f{partial_value(w[0]), partial_value(w[1]), partial_value(w[2]), partial_value(w[3])};
}
constexpr int kBufferWord3 = 0x00020000;  // raw (unformatted) buffer descriptor
constexpr int kSpinLimit = 1 << 18;       // polls before a tail gives up (about 0.3 s)

// Tail: the KP workgroups of a tile are all resident at once (the host checks that the grid fits the
// device), and the first R = min(KP, 4 MF) parts each sum one slice of the column group's partial tile:
// part p < R owns the float4s u = U p .. U p + U - 1 (U = 4 MF / R) of every lane's 4 MF (float4 u is
// fragment u / 4, registers 4 (u % 4) .. +3).  Each wave stores the slices it does not own to their
// owners' slots, without waiting; an owner then polls its slot of every other part (coherent loads that
// skip the CU's L1) until no word reads 0, adds the KP slices in K-part order, stores BF16 and clears the
// slots it read.  Every store it waits for was issued by a resident wave, so the poll ends; a bounded
// count of polls keeps the kernel finite even if the co-residency the host checked were broken: the slice
// is then stored as NaN, and a partial arriving after the owner gave up leaves the workspace non-zero, so
// it must be zero-filled again before its next use.
template <int MF, int KP, typename Store, bool COMPACT = false>
__device__ __forceinline__ void tail_sum(const v4f (&mine)[MF][4], uint8_t* ws, int ws_range, int t, int q, int wave,
                                          int lane, Store&& store_one, std::bool_constant<COMPACT> = {}) {
    constexpr int R = KP < 4 * MF ? KP : 4 * MF;  // parts that own a slice
    constexpr int U = 4 * MF / R;                 // float4s per lane in a slice
    static_assert(U * R == 4 * MF, "slices of whole float4s");
    // slot (p, qq) of column group (t, wave): slice p of part qq, written by qq, read by p; float4 uu of lane
    // l at + 1024 uu + 16 l.  R KP slots of 1024 U bytes per group: the group's share of the workspace
    // (COMPACT: R (KP - 1), leaving out the slots (p, p), which are never written).
    auto slot = [&](int p, int qq) -> uint32_t {
        if constexpr (COMPACT)
            return (uint32_t)(((((size_t)t * 4 + wave) * R + p) * (KP - 1) + (qq < p ? qq : qq - 1)) * (1024 * U) +
                              16 * lane);
        else
            return (uint32_t)(((((size_t)t * 4 + wave) * R + p) * KP + qq) * (1024 * U) + 16 * lane);
    };
    static_for<R>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        if (p == q) return;
        v4u* const dst = reinterpret_cast<v4u*>(ws + slot(p, q));
        static_for<U>([&](auto uc) {
            constexpr int uu = decltype(uc)::value, u = U * p + uu;
            dst[64 * uu] = partial_words(mine[u / 4][u % 4]);
        });
    });
    if (q >= R) return;  // a part without a slice only contributes
    v4f own[U] = {};
    static_for<R>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        if (p != q) return;
        static_for<U>([&](auto uc) {
            constexpr int uu = decltype(uc)::value, u = U * p + uu;
            own[uu] = partial_values(partial_words(mine[u / 4][u % 4]));  // NaNs made canonical, as the others'
        });
    });
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(ws, (short)0, ws_range, kBufferWord3);
    v4u pv[KP - 1][U];
    bool complete = false;
    for (int it = 0; it < kSpinLimit && !complete; ++it) {
        uint32_t present = 1;
        static_for<KP - 1>([&](auto oc) {
            constexpr int o = decltype(oc)::value;
            uint32_t off = slot(q, o < q ? o : o + 1);
            asm volatile("" : "+v"(off));  // an opaque address: the loads are repeated, not hoisted out of the loop
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                // cache policy sc1: coherent at device scope, so every poll reads L2 again, never the L1
                pv[o][uu] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024 * uu, 0, 16));
                present &= (pv[o][uu][0] != 0u) & (pv[o][uu][1] != 0u) & (pv[o][uu][2] != 0u) & (pv[o][uu][3] != 0u);
            }
        });
        complete = __all(present);
        if (!complete) __builtin_amdgcn_s_sleep(1);
    }
    v4f sum[U];
    static_for<KP>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int below = p < KP - 1 ? p : KP - 2;
        constexpr int above = p > 0 ? p - 1 : 0;
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const v4f v = p == q ? own[uu] : partial_values(p < q ? pv[below][uu] : pv[above][uu]);
            if constexpr (p == 0) sum[uu] = v;
            else sum[uu] += v;
        }
    });
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
        const int u = U * q + uu;
        const float nan = __uint_as_float(0x7FC00000u);
        store_one(u / 4, u % 4, complete ? sum[uu] : v4f{nan, nan, nan, nan});  // a timed-out wait shows as NaN
    }
    static_for<KP - 1>([&](auto oc) {
        constexpr int o = decltype(oc)::value;
        v4u* const dst = reinterpret_cast<v4u*>(ws + slot(q, o < q ? o : o + 1));
#pragma unroll
        for (int uu = 0; uu < U; ++uu) dst[64 * uu] = v4u{0u, 0u, 0u, 0u};
    });
}

// The same protocol for a wave holding NF float4s per lane (a large output tile, its accumulators in AGPRs):
// every part p < KP owns the slice of float4s U p .. U p + U - 1 (U = NF / KP), the slots are compact (slot
// (p, qq) of a (tile, wave): slice p written by part qq != p; float4 uu of lane l at + 1024 uu + 16 l), and the
// owner polls, sums in K-part order, stores and clears its slice CH float4s at a time, so only CH float4s of
// each other part are in registers at once.  mine(ic) returns the wave's float4 ic (an integral_constant);
// store_one(u, v) stores the sum of float4 u.  The poll budget kSpinLimit is shared by the chunks: once it is
// spent, every chunk not yet complete is stored as NaN after one more poll.
template <int NF, int KP, int CH, typename Mine, typename Store>
__device__ __forceinline__ void tail_sum_chunked(Mine&& mine, uint8_t* ws, int ws_range, int t, int q, int wave,
                                                  int lane, Store&& store_one) {
    constexpr int U = NF / KP;
    static_assert(U * KP == NF && U % CH == 0, "slices of whole chunks");
    auto slot = [&](int p, int qq) -> uint32_t {
        return (uint32_t)(((((size_t)t * 4 + wave) * KP + p) * (KP - 1) + (qq < p ? qq : qq - 1)) * (1024 * U) +
                          16 * lane);
    };
    static_for<KP>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        if (p == q) return;
        v4u* const dst = reinterpret_cast<v4u*>(ws + slot(p, q));
        static_for<U>([&](auto uc) {
            constexpr int uu = decltype(uc)::value;
            dst[64 * uu] = partial_words(mine(std::integral_constant<int, U * p + uu>{}));
        });
    });
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(ws, (short)0, ws_range, kBufferWord3);
    int spins = 0;
    static_for<KP>([&](auto pc) {
        constexpr int p = decltype(pc)::value;  // this part's slice: p == q
        if (p != q) return;
        static_for<U / CH>([&](auto cc) {
            constexpr int c0 = decltype(cc)::value * CH;  // first float4 of the chunk within the slice
            v4u pv[KP - 1][CH];
            bool complete = false;
            do {
                uint32_t present = 1;
                static_for<KP - 1>([&](auto oc) {
                    constexpr int o = decltype(oc)::value;  // slot o holds part o < p ? o : o + 1
                    uint32_t off = slot(p, o < p ? o : o + 1);
                    asm volatile("" : "+v"(off));  // an opaque address: the loads are repeated each poll
#pragma unroll
                    for (int k = 0; k < CH; ++k) {
                        // cache policy sc1: coherent at device scope, so every poll reads L2 again
                        pv[o][k] = __builtin_bit_cast(
                            v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024 * (c0 + k), 0, 16));
                        present &= (pv[o][k][0] != 0u) & (pv[o][k][1] != 0u) & (pv[o][k][2] != 0u) &
                                   (pv[o][k][3] != 0u);
                    }
                });
                complete = __all(present);
                if (!complete) __builtin_amdgcn_s_sleep(1);
            } while (!complete && ++spins < kSpinLimit);
            static_for<CH>([&](auto kc) {
                constexpr int k = decltype(kc)::value, u = U * p + c0 + k;
                v4f sum;
                static_for<KP>([&](auto sc) {
                    constexpr int s = decltype(sc)::value;
                    v4f v;
                    if constexpr (s == p)  // NaNs made canonical, as the others'
                        v = partial_values(partial_words(mine(std::integral_constant<int, u>{})));
                    else
                        v = partial_values(pv[s < p ? s : s - 1][k]);
                    if constexpr (s == 0) sum = v;
                    else sum += v;
                });
                const float nan = __uint_as_float(0x7FC00000u);
                store_one(u, complete ? sum : v4f{nan, nan, nan, nan});  // a timed-out wait shows as NaN
            });
            static_for<KP - 1>([&](auto oc) {
                constexpr int o = decltype(oc)::value;
                v4u* const dst = reinterpret_cast<v4u*>(ws + slot(p, o < p ? o : o + 1));
#pragma unroll
                for (int k = 0; k < CH; ++k) dst[64 * (c0 + k)] = v4u{0u, 0u, 0u, 0u};
            });
        });
    });
}
}  // namespace sk

// KP: K parts (K = 256 NSL KP).  FUSED: the activations arrive as BF16 X [M, K] (in qa; sa unused) and
// each workgroup quantizes its K part into the LDS block itself (the one-launch decode layer).
// The main loop of one workgroup: tile t, K part q (slabs NSL q .. NSL q + NSL - 1; M rows of qa / sa), with
// the workgroup's LDS block, adding into acc.
template <int MF, int S, int NSL, bool FUSED>
__device__ __forceinline__ void splitk_fp4_part(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                int M, int N, int K, int t, int q, uint8_t* lds, v16f (&acc)[MF]) {
    using C = sk::Cfg<MF, S, NSL>;
    using sk::key;
    uint8_t* const actb = lds;                   // [kArows][NSL][128], chunks XOR-swizzled by key(row)
    uint8_t* const scb = lds + C::kAct;          // [kScRows][8 NSL]: 16-byte piece p of row r at (p + r) % kP
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = (int64_t)K / 2;
    const int KS = K / 32;
    const int n0 = t * sk::kTN;
    const int s0 = q * NSL;                      // first slab of the part (in K = 256 units)
    const int rot = (t + 3 * q) % NSL;           // local slab j reads slab s0 + (j + rot) % NSL
    uint8_t* const ring = lds + C::kAct + C::kSc + wave * C::kRingWave;

    // 1. the part's activation codes: line (r, j) = row r, slab s0 + j, at LDS (r NSL + j) * 128; copy c moves
    //    lines 8c .. 8c+7.  Copies whose rows all lie at or past M are skipped (those rows only feed output
    //    columns that are never stored); partly valid ones read row M - 1 for the rest.
#pragma unroll
    for (int e = 0; e < (FUSED ? 0 : C::kActCopies / 4); ++e) {
        const int c = wave * (C::kActCopies / 4) + e;
        if ((8 * c) / NSL >= M) break;           // wave-uniform
        const int line = 8 * c + (lane >> 3);
        const int r = line / NSL, j = line % NSL;
        const uint8_t* src = qa + (int64_t)min(r, M - 1) * KB + (int64_t)(s0 + j) * sk::kSlab + 16 * ((lane & 7) ^ key(r));
        g2lds16(src, actb + 1024 * c);
    }
    // 2. scales of the part: kP pieces of 16 bytes per row (8 bytes per slab); the activation rows' ones are
    //    the first kArows kP / 64 copies (FUSED computes those itself)
    for (int c = (FUSED ? C::kArows * C::kP / 64 : 0) + wave; c < C::kScCopies; c += 4) {
        const int u = 64 * c + lane;
        const int r = u / C::kP, pos = u % C::kP;
        const int p = (pos + C::kP - r % C::kP) % C::kP;   // the piece stored at position pos
        const uint8_t* src = r < C::kArows ? sa + (int64_t)min(r, M - 1) * KS
                                           : sw + (int64_t)min(n0 + r - C::kArows, N - 1) * KS;
        g2lds16(src + 8 * s0 + 16 * p, scb + 1024 * c);
    }
    // 3. this wave's weight rows n0 + 32 wave + (0 .. 31); copy i of a slab moves rows 8i .. 8i+7, whole lines
    const uint8_t* wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        wrow[i] = qw + (int64_t)min(n0 + 32 * wave + r, N - 1) * KB + 16 * ((lane & 7) ^ key(r));
    }
    auto issue = [&](int j) {  // local slab j into slot j % S (streamed once: non-temporal)
        const int64_t koff = (int64_t)(s0 + (j + rot) % NSL) * sk::kSlab;
#pragma unroll
        for (int i = 0; i < 4; ++i) g2lds16_nt(wrow[i] + koff, ring + (j % S) * 4096 + 1024 * i);
    };
#pragma unroll
    for (int j = 0; j < S; ++j) issue(j);
    if constexpr (FUSED) {
        quantize_part<MF, S, NSL>(qa, M, K, s0, wave, lane, actb, scb);
        __syncthreads();  // the quantized block, the scales and this wave's first slabs are in LDS
    } else {
        wait_vmcnt<S * 4>();           // activations and scales (issued before the ring) have landed
        __builtin_amdgcn_s_barrier();  // for every wave
    }

    // per-lane LDS addresses: weight row l32 of this wave, activation rows 32 g + l32
    const uint32_t rbase = lds_addr(ring), abase = lds_addr(actb), sbase = lds_addr(scb);
    const int wkey = key(l32);
    const int wsr = C::kArows + 32 * wave + l32;
    int xoff[MF], xkey[MF], xsr[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g) {
        const int r = 32 * g + l32;
        xoff[g] = r * NSL * sk::kSlab;
        xkey[g] = key(r);
        xsr[g] = r;
    }
    // scale dword of row r for slab jj (K-part local), lane group h: bytes 8 jj + 4h .. +3 of the row
    auto scale_at = [&](int r, int jj) -> uint32_t {
        const int pos = (jj / 2 + r) % C::kP;
        return lds_read4(sbase + r * 8 * NSL + 16 * pos + 8 * (jj & 1) + 4 * h);
    };

    static_for<NSL>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int kNewer = (S - 1 < NSL - 1 - j) ? S - 1 : NSL - 1 - j;  // later slabs already issued
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kNewer * 4>();
        __builtin_amdgcn_sched_barrier(0);
        const int jj = (j + rot) % NSL;
        const uint32_t sl = rbase + (j % S) * 4096;
        uint32_t ws_ = scale_at(wsr, jj);
        uint32_t xs[MF];
#pragma unroll
        for (int g = 0; g < MF; ++g) xs[g] = scale_at(xsr[g], jj);
        v4u wv[4], xv[4][MF];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            wv[tt] = lds_read16(sl + l32 * sk::kSlab + 16 * ((4 * h + tt) ^ wkey));
#pragma unroll
            for (int g = 0; g < MF; ++g)
                xv[tt][g] = lds_read16(abase + xoff[g] + jj * sk::kSlab + 16 * ((4 * h + tt) ^ xkey[g]));
        }
        lds_wait_dec<MF>(wv, xv, ws_, xs);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j + S < NSL) issue(j + S);  // the slot is read: refill it
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < MF; ++g) {
            acc[g] = mfma32<kFmtFP4, 0>(fp4_operand(wv[0]), fp4_operand(xv[0][g]), acc[g], (int)ws_, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 1>(fp4_operand(wv[1]), fp4_operand(xv[1][g]), acc[g], (int)ws_, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 2>(fp4_operand(wv[2]), fp4_operand(xv[2][g]), acc[g], (int)ws_, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 3>(fp4_operand(wv[3]), fp4_operand(xv[3][g]), acc[g], (int)ws_, (int)xs[g]);
            asm volatile("" : "+a"(acc[g]));  // the slab's MFMAs stay in this iteration (not sunk to the end)
        }
    });

}

// The workgroup's results: BF16 of acc into y (KP = 1), or the partials of K part q summed across the tile's
// workgroups in the workspace first.
template <int MF, int KP>
__device__ __forceinline__ void splitk_fp4_finish(const v16f (&acc)[MF], uint16_t* __restrict__ y, int M, int N,
                                                  int tiles, uint8_t* __restrict__ ws, int t, int q) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int n0 = t * sk::kTN;
    // 4. D[n][m] of fragment g: lane l holds column m = 32 g + l32 and rows n = 8 i + 4 h + e in register
    //    4 i + e.  With KP > 1 the partials of the column group (tile t, wave) meet in the workspace.
    const int nw = n0 + 32 * wave + 4 * h;
    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
    // BF16 of fragment g, registers 4 i .. 4 i + 3 (rows n .. n + 3 of column m)
    auto store_one = [&](int g, int i, const v4f& v) {
        const int m = 32 * g + l32;
        if (m >= M) return;
        const int n = nw + 8 * i;
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
    };
    v4f mine[MF][4];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[g][i] = v4f{acc[g][4 * i], acc[g][4 * i + 1], acc[g][4 * i + 2], acc[g][4 * i + 3]};
    if constexpr (KP == 1) {
#pragma unroll
        for (int g = 0; g < MF; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) store_one(g, i, mine[g][i]);
    } else {
        sk::tail_sum<MF, KP>(mine, ws, (int)sk::workspace_bytes(tiles, KP, MF), t, q, wave, lane, store_one);
    }
}

// One workgroup's work: tile t, K part q (M rows of qa / sa / y), with the workgroup's LDS block.
template <int MF, int S, int NSL, int KP, bool FUSED>
__device__ __forceinline__ void splitk_fp4_tile(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                uint16_t* __restrict__ y, int M, int N, int K, int tiles,
                                                uint8_t* __restrict__ ws, int t, int q, uint8_t* lds) {
    v16f acc[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
    splitk_fp4_part<MF, S, NSL, FUSED>(qa, sa, qw, sw, M, N, K, t, q, lds, acc);
    splitk_fp4_finish<MF, KP>(acc, y, M, N, tiles, ws, t, q);
}

template <int MF, int S, int NSL, int KP, bool FUSED = false>
__global__ __launch_bounds__(256, 1) void gemm_splitk_fp4(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                          const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                          uint16_t* __restrict__ y, int M, int N, int K, int tiles,
                                                          uint8_t* __restrict__ ws) {
    const int b = blockIdx.x;
    const int slot8 = b >> 3;
    const int q = slot8 % KP;                    // K part
    const int t = (slot8 / KP) * 8 + (b & 7);    // tile
    if (t >= tiles) return;                      // the whole workgroup, before any barrier
    __shared__ __attribute__((aligned(1024))) uint8_t lds[sk::Cfg<MF, S, NSL>::kLds];
    splitk_fp4_tile<MF, S, NSL, KP, FUSED>(qa, sa, qw, sw, y, M, N, K, tiles, ws, t, q, lds);
}

// Grouped A4W4 GEMM over MoE experts ("Kimi-K3-Quark-MXFP4-AttnFP8", section "Model Quantization": expert
// weights and activations in OCP MXFP4) in the same per-tile design without a K split across workgroups:
// workgroup (t, e) computes the 128 columns of tile t for the rows goff[e] .. goff[e+1] - 1 of expert e, in
// chunks of 32 MF rows, and walks K in parts of NSL slabs (K % (256 NSL) == 0), adding each part's products
// into the same accumulators; a barrier separates parts and row chunks, which reuse the LDS block.  Every
// row of every group is written, and the sums run in the K order of the split-K kernel's parts.
// The tiles of one expert are consecutive workgroups, dealt round-robin to the XCDs, so each XCD's tiles of
// an expert read its activation rows through one L2.  An empty group's workgroups return at once.  A
// configuration whose LDS block fits twice in a CU's 160 KB is compiled for two workgroups per CU.
template <int MF, int S, int NSL>
__global__ __launch_bounds__(256, (2 * sk::Cfg<MF, S, NSL>::kLds <= 160 * 1024 ? 2 : 1)) void gemm_grouped_fp4(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                           const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                           uint16_t* __restrict__ y, int N, int K, int tiles,
                                                           const int32_t* __restrict__ goff) {
    constexpr int kRows = 32 * MF;
    const int t = blockIdx.x, e = blockIdx.y;
    const int r0 = __builtin_amdgcn_readfirstlane(goff[e]);
    const int rows = __builtin_amdgcn_readfirstlane(goff[e + 1]) - r0;
    if (rows <= 0) return;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[sk::Cfg<MF, S, NSL>::kLds];
    const int64_t KB = (int64_t)K / 2, KS = K / 32;
    const uint8_t* const qwe = qw + (int64_t)e * N * KB;
    const uint8_t* const swe = sw + (int64_t)e * N * KS;
    const int parts = K / (256 * NSL);
#pragma nounroll
    for (int c = 0; c < rows; c += kRows) {
        const int64_t r = r0 + c;
        const int mc = min(rows - c, kRows);
        v16f acc[MF];
#pragma unroll
        for (int g = 0; g < MF; ++g)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
#pragma nounroll
        for (int q = 0; q < parts; ++q) {
            if (c > 0 || q > 0) {
                wait_vmcnt<0>();   // the earlier stores and copies are done before the next copies are counted
                __syncthreads();   // and every wave is done with its LDS
            }
            splitk_fp4_part<MF, S, NSL, false>(qa + r * KB, sa + r * KS, qwe, swe, mc, N, K, t, q, lds, acc);
        }
        splitk_fp4_finish<MF, 1>(acc, y + r * N, mc, N, tiles, nullptr, t, 0);
    }
}

// ---------------------------------------------------------------------------------------------------------
// The A8W8 (PTPC FP8) decode GEMM in the same decomposition ("Kimi-K3-DSpark-FP8-PTPC", section "Phase 1
// FP8 PTPC Quantization": E4M3 weights and per-token E4M3 activations, FP32 per-token and
// per-output-channel scales).  An E4M3 activation row is 1 byte per value, so a K part of 64 rows does not
// fit in LDS beside the weight rings; instead the activation slabs stream through a ring shared by the
// workgroup's waves, each wave copying its share of every slab beside its own weight rows.  A slab is
// K = 128 (128 bytes per row); its 32 MF activation rows are read by all 4 waves, so a barrier per slab
// separates the copies of slab j from its reads, and a slot is refilled only after the next barrier (when
// every wave has read it): S - 1 slabs stay in flight.  E4M3 widens exactly to FP16 and the products run
// on the 32 x 32 x 16 FP16 MFMA, as in the ring kernel.  The K parts' partial sums meet in the same tail;
// the scales are applied to the sum, acc sA sW in FP64, then BF16.
namespace sk8 {
constexpr int kSlab = 128;  // code bytes per row per slab (K = 128)
template <int MF, int S>
struct Cfg {
    static constexpr int kArows = 32 * MF;
    static constexpr int kActSlab = kArows * kSlab;      // shared activation slot
    static constexpr int kWSlab = 32 * kSlab;            // a wave's weight slot
    static constexpr int kSlot = kActSlab + 4 * kWSlab;
    static constexpr int kLds = S * kSlot;
    static constexpr int kCopies = MF + 4;              // per wave and slab: activation share, weight rows
    static_assert(S >= 3 && S * kCopies <= 63, "vmcnt");
    static_assert(kLds <= 160 * 1024, "LDS");
};
}  // namespace sk8

template <int MF, int S, int NSL, int KP>
__global__ __launch_bounds__(256, 1) void gemm_splitk_fp8(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                          const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                                          uint16_t* __restrict__ y, int M, int N, int K, int tiles,
                                                          uint8_t* __restrict__ ws) {
    using C = sk8::Cfg<MF, S>;
    using sk::key;
    const int b = blockIdx.x;
    const int slot8 = b >> 3;
    const int q = slot8 % KP;                    // K part
    const int t = (slot8 / KP) * 8 + (b & 7);    // tile
    if (t >= tiles) return;                      // the whole workgroup, before any barrier

    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int n0 = t * sk::kTN;
    const int s0 = q * NSL;                      // first slab of the part (in K = 128 units)
    const int rot = (t + 3 * q) % NSL;           // local slab j reads slab s0 + (j + rot) % NSL

    // Copies of local slab j into slot j % S: activation rows 8c .. 8c+7 for c = MF wave .. MF wave + MF - 1
    // (rows at or past M read row M - 1; a copy whose rows all lie past M reads one line for all its lanes:
    // those rows only feed outputs that are never stored), then this wave's weight rows n0 + 32 wave + 8i ..
    // +7.  The lane fills chunk lane % 8 of its row with logical chunk (lane % 8) ^ key(row).
    const uint8_t* arow[MF];
#pragma unroll
    for (int e = 0; e < MF; ++e) {
        const int c = wave * MF + e;
        const int r = 8 * c + (lane >> 3);
        arow[e] = 8 * c >= M ? qa + (int64_t)(M - 1) * K : qa + (int64_t)min(r, M - 1) * K + 16 * ((lane & 7) ^ key(r));
    }
    const uint8_t* wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        wrow[i] = qw + (int64_t)min(n0 + 32 * wave + r, N - 1) * K + 16 * ((lane & 7) ^ key(r));
    }
    auto issue = [&](int j) {
        uint8_t* const slot = lds + (j % S) * C::kSlot;
        const int64_t koff = (int64_t)(s0 + (j + rot) % NSL) * sk8::kSlab;
#pragma unroll
        for (int e = 0; e < MF; ++e) g2lds16(arow[e] + koff, slot + 1024 * (wave * MF + e));  // reused by 7 CUs
#pragma unroll
        for (int i = 0; i < 4; ++i) g2lds16_nt(wrow[i] + koff, slot + C::kActSlab + wave * C::kWSlab + 1024 * i);
    };
#pragma unroll
    for (int j = 0; j < S; ++j) issue(j);

    const uint32_t base = lds_addr(lds);
    const int wkey = key(l32);
    const uint32_t woff = C::kActSlab + wave * C::kWSlab + l32 * sk8::kSlab;
    uint32_t xoff[MF];
    int xkey[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g) {
        xoff[g] = (32 * g + l32) * sk8::kSlab;
        xkey[g] = key(32 * g + l32);
    }
    v16f acc[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;

    static_for<NSL>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        // issued so far: slabs 0 .. S - 1 by the prologue, then one per earlier slab from slab 1 on, i.e.
        // 0 .. j + S - 2 for j >= 1; those after slab j may still be in flight
        constexpr int kIssued = j == 0 ? S - 1 : (j + S - 2 < NSL - 1 ? j + S - 2 : NSL - 1);
        constexpr int kLater = kIssued - j;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kLater * C::kCopies>();  // this wave's copies of slab j have landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();       // every wave's: slab j is whole, and slab j - 1 is read
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j >= 1 && j - 1 + S < NSL) issue(j - 1 + S);  // into the slot of slab j - 1
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t sb = base + (j % S) * C::kSlot;
        v4u wv[4], xv[4][MF];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            wv[tt] = lds_read16(sb + woff + 16 * ((4 * h + tt) ^ wkey));
#pragma unroll
            for (int g = 0; g < MF; ++g) xv[tt][g] = lds_read16(sb + xoff[g] + 16 * ((4 * h + tt) ^ xkey[g]));
        }
        lds_wait_codes<MF>(wv, xv);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const v8h w0 = e4m3x8_to_f16x8(wv[tt][0], wv[tt][1]);
            const v8h w1 = e4m3x8_to_f16x8(wv[tt][2], wv[tt][3]);
#pragma unroll
            for (int g = 0; g < MF; ++g) {
                acc[g] = mfma32_f16(w0, e4m3x8_to_f16x8(xv[tt][g][0], xv[tt][g][1]), acc[g]);
                acc[g] = mfma32_f16(w1, e4m3x8_to_f16x8(xv[tt][g][2], xv[tt][g][3]), acc[g]);
            }
        }
    });

    // D[n][m] of fragment g: lane l holds column m = 32 g + l32 and rows n = 8 i + 4 h + e in register 4 i + e.
    const int nw = n0 + 32 * wave + 4 * h;
    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
    auto store_one = [&](int g, int i, const v4f& v) {  // acc sA sW, then BF16
        const int m = 32 * g + l32;
        if (m >= M) return;
        const int n = nw + 8 * i;
        const float sam = sa[m];
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = ptpc_scaled(v[e], sam, sw[min(n + e, N - 1)]);
        uint16_t* dst = y + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
            uint2 pk;
            pk.x = bf16x2_rne(o[0], o[1]);
            pk.y = bf16x2_rne(o[2], o[3]);
            *reinterpret_cast<uint2*>(dst) = pk;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = (uint16_t)(bf16x2_rne(o[e], 0.f) & 0xffffu);
        }
    };
    v4f mine[MF][4];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[g][i] = v4f{acc[g][4 * i], acc[g][4 * i + 1], acc[g][4 * i + 2], acc[g][4 * i + 3]};
    wait_vmcnt<0>();  // no copy past the last slab is issued; nothing is in flight here
    sk::tail_sum<MF, KP>(mine, ws, (int)sk::workspace_bytes(tiles, KP, MF), t, q, wave, lane, store_one);
}

// ---------------------------------------------------------------------------------------------------------
// 64 < M <= 128: the A4W4 split-K decomposition over two row halves.  A workgroup owns a 128-column tile,
// one of KP K parts and one 64-row half of the activations, so a tile takes 2 KP workgroups (224 at
// (128, 7168, 8192) with KP = 2) and each CU reads 1/KP of its half's activations beside 1/KP of the tile's
// weight rows; the two halves of a tile read the same weight rows through one XCD's L2.  A K part of 64
// rows is too wide for LDS here (4096 K-values: 128 KB), so the activation slabs stream through a ring
// shared by the waves, as in gemm_splitk_fp8: each wave copies its share of every slab (K = 256, 8 KB)
// beside its own weight rows, a barrier per slab separates the copies of slab j from its reads, and a slot
// is refilled after the next barrier.  The part's activation and weight scales are copied once.  The K
// parts of a (tile, half) meet in the slice-owner tail.
namespace skr {
template <int S, int NSL>
struct Cfg {
    static constexpr int kArows = 64;                        // rows per half
    static constexpr int kActSlab = kArows * sk::kSlab;      // shared activation slot
    static constexpr int kWSlab = 32 * sk::kSlab;            // a wave's weight slot
    static constexpr int kSlot = kActSlab + 4 * kWSlab;
    static constexpr int kP = NSL / 2;                       // 16-byte scale pieces per row
    static constexpr int kScRows = kArows + sk::kTN;         // activation rows, then weight rows
    static constexpr int kSc = kScRows * 8 * NSL;
    static constexpr int kScCopies = kScRows * kP / 64;
    static constexpr int kLds = S * kSlot + kSc;
    static constexpr int kCopies = 2 + 4;                    // per wave and slab: activation share, weight rows
    static_assert(S >= 3 && S * kCopies <= 63, "vmcnt");
    static_assert(NSL % 2 == 0 && NSL >= S, "slabs per part");
    static_assert((kScRows * kP) % 64 == 0, "scale copies");
    static_assert(kLds <= 160 * 1024, "LDS");
};
}  // namespace skr

template <int S, int NSL, int KP>
__global__ __launch_bounds__(256, 1) void gemm_splitk_fp4_rh(const uint8_t* __restrict__ qa,
                                                             const uint8_t* __restrict__ sa,
                                                             const uint8_t* __restrict__ qw,
                                                             const uint8_t* __restrict__ sw, uint16_t* __restrict__ y,
                                                             int M, int N, int K, int tiles, uint8_t* __restrict__ ws) {
    using C = skr::Cfg<S, NSL>;
    using sk::key;
    constexpr int MF = 2;
    const int b = blockIdx.x;
    const int slot8 = b >> 3;
    const int grp = slot8 % (2 * KP);
    const int q = grp % KP, rh = grp / KP;       // K part, row half
    const int t = (slot8 / (2 * KP)) * 8 + (b & 7);
    if (t >= tiles) return;                      // the whole workgroup, before any barrier

    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];
    uint8_t* const scb = lds + S * C::kSlot;     // [kScRows][8 NSL]: 16-byte piece p of row r at (p + r) % kP
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t KB = (int64_t)K / 2;
    const int KS = K / 32;
    const int n0 = t * sk::kTN;
    const int m0 = rh * C::kArows;               // first activation row of this half
    const int mh = min(M - m0, C::kArows);       // rows of this half (>= 1)
    const int s0 = q * NSL;                      // first slab of the part (K = 256 units)
    const int rot = (t + 3 * q) % NSL;           // local slab j reads slab s0 + (j + rot) % NSL
    const uint8_t* const qah = qa + (int64_t)m0 * KB;
    const uint8_t* const sah = sa + (int64_t)m0 * KS;

    // scales of the part (activation rows of this half first, then the tile's weight rows)
    for (int c = wave; c < C::kScCopies; c += 4) {
        const int u = 64 * c + lane;
        const int r = u / C::kP, pos = u % C::kP;
        const int p = (pos + C::kP - r % C::kP) % C::kP;
        const uint8_t* src = r < C::kArows ? sah + (int64_t)min(r, mh - 1) * KS
                                           : sw + (int64_t)min(n0 + r - C::kArows, N - 1) * KS;
        g2lds16(src + 8 * s0 + 16 * p, scb + 1024 * c);
    }
    // per slab: this wave's two activation copies (rows 8c .. 8c+7, c = 2 wave, 2 wave + 1; rows past the half
    // read its last row, a copy wholly past it one line) and four weight copies
    const uint8_t* arow[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = 2 * wave + e;
        const int r = 8 * c + (lane >> 3);
        arow[e] = 8 * c >= mh ? qah + (int64_t)(mh - 1) * KB : qah + (int64_t)min(r, mh - 1) * KB + 16 * ((lane & 7) ^ key(r));
    }
    const uint8_t* wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        wrow[i] = qw + (int64_t)min(n0 + 32 * wave + r, N - 1) * KB + 16 * ((lane & 7) ^ key(r));
    }
    auto issue = [&](int j) {
        uint8_t* const slot = lds + (j % S) * C::kSlot;
        const int64_t koff = (int64_t)(s0 + (j + rot) % NSL) * sk::kSlab;
#pragma unroll
        for (int e = 0; e < 2; ++e) g2lds16(arow[e] + koff, slot + 1024 * (2 * wave + e));
#pragma unroll
        for (int i = 0; i < 4; ++i) g2lds16_nt(wrow[i] + koff, slot + C::kActSlab + wave * C::kWSlab + 1024 * i);
    };
#pragma unroll
    for (int j = 0; j < S; ++j) issue(j);

    const uint32_t base = lds_addr(lds), sbase = lds_addr(scb);
    const int wkey = key(l32);
    const uint32_t woff = C::kActSlab + wave * C::kWSlab + l32 * sk::kSlab;
    const int wsr = C::kArows + 32 * wave + l32;
    uint32_t xoff[MF];
    int xkey[MF], xsr[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g) {
        xoff[g] = (32 * g + l32) * sk::kSlab;
        xkey[g] = key(32 * g + l32);
        xsr[g] = 32 * g + l32;
    }
    auto scale_at = [&](int r, int jj) -> uint32_t {
        const int pos = (jj / 2 + r) % C::kP;
        return lds_read4(sbase + r * 8 * NSL + 16 * pos + 8 * (jj & 1) + 4 * h);
    };
    v16f acc[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;

    static_for<NSL>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        // issued so far: slabs 0 .. S - 1 by the prologue, then one per earlier slab from slab 1 on
        constexpr int kIssued = j == 0 ? S - 1 : (j + S - 2 < NSL - 1 ? j + S - 2 : NSL - 1);
        constexpr int kLater = kIssued - j;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kLater * C::kCopies>();  // this wave's copies of slab j (and the scales) have landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();       // every wave's: slab j is whole, and slab j - 1 is read
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j >= 1 && j - 1 + S < NSL) issue(j - 1 + S);  // into the slot of slab j - 1
        __builtin_amdgcn_sched_barrier(0);
        const int jj = (j + rot) % NSL;
        const uint32_t sb = base + (j % S) * C::kSlot;
        uint32_t ws_ = scale_at(wsr, jj);
        uint32_t xs[MF];
#pragma unroll
        for (int g = 0; g < MF; ++g) xs[g] = scale_at(xsr[g], jj);
        v4u wv[4], xv[4][MF];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            wv[tt] = lds_read16(sb + woff + 16 * ((4 * h + tt) ^ wkey));
#pragma unroll
            for (int g = 0; g < MF; ++g) xv[tt][g] = lds_read16(sb + xoff[g] + 16 * ((4 * h + tt) ^ xkey[g]));
        }
        lds_wait_dec<MF>(wv, xv, ws_, xs);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < MF; ++g) {
            acc[g] = mfma32<kFmtFP4, 0>(fp4_operand(wv[0]), fp4_operand(xv[0][g]), acc[g], (int)ws_, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 1>(fp4_operand(wv[1]), fp4_operand(xv[1][g]), acc[g], (int)ws_, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 2>(fp4_operand(wv[2]), fp4_operand(xv[2][g]), acc[g], (int)ws_, (int)xs[g]);
            acc[g] = mfma32<kFmtFP4, 3>(fp4_operand(wv[3]), fp4_operand(xv[3][g]), acc[g], (int)ws_, (int)xs[g]);
        }
    });

    const int nw = n0 + 32 * wave + 4 * h;
    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
    auto store_one = [&](int g, int i, const v4f& v) {
        const int m = m0 + 32 * g + l32;
        if (m >= M) return;
        const int n = nw + 8 * i;
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
    };
    v4f mine[MF][4];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[g][i] = v4f{acc[g][4 * i], acc[g][4 * i + 1], acc[g][4 * i + 2], acc[g][4 * i + 3]};
    // the column groups of (tile, half) pairs: 2 tiles' worth of slots
    sk::tail_sum<MF, KP>(mine, ws, (int)sk::workspace_bytes(2 * tiles, KP, MF), 2 * t + rh, q, wave, lane, store_one);
}

}  // namespace mx
