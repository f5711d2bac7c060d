// gemm_splitk.hpp - decode-size A4W4 GEMM with K split across workgroups (gfx950).
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
//   * the KP partial tiles of a column group are summed across workgroups: each
//     wave stores its FP32 partial (64 x 32) to the workspace, waits until the
//     stores are complete, and increments the group's counter.  The wave that
//     sees the count reach KP - 1 reads the other KP - 1 partials, adds all KP
//     in K-part order (0, 1, ..., KP - 1: deterministic, whatever the arrival
//     order), writes BF16 and resets the counter to 0.  No wave ever waits for
//     another workgroup, so the design needs no co-residency.
//
// The KP workgroups of a tile are blockIdx t % 8 + 8 (KP (t / 8) + q): equal
// modulo 8, which places them on one XCD (workgroups are dealt round-robin to
// the XCDs), so partials and counters meet in that XCD's L2 without cache
// maintenance.  The workspace holds one counter per column group in a fixed
// 4 KB area at its start (at most 256 tiles x 4 groups), then the partials.
// It must be zero-filled before its first use; every launch leaves the
// counters at zero, and no launch's partials reach into the counter area, so
// one workspace serves launches of any shapes in turn.  Launches that share a
// workspace must not overlap.
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

// Workspace: the counter area (4 per tile, at most kMaxTiles tiles), then KP partials of
// 4 waves x MF fragments x 4 KB per tile.
constexpr int kMaxTiles = 256;
constexpr size_t kCounterBytes = kMaxTiles * 4 * sizeof(uint32_t);
inline size_t workspace_bytes(int tiles, int KP, int MF) {
    return kCounterBytes + (size_t)tiles * KP * 4 * MF * 4096;
}
}  // namespace sk

// FUSED prologue: quantize rows 0 .. M-1 of BF16 X, K-values 256 s0 .. 256 (s0 + NSL) - 1, into the LDS
// activation block and scale rows of the split-K kernel, bit for bit as mx_quant_act_bf16 does.  A row's
// part is NSL / 2 pieces of 1 KB; one wave instruction loads a whole piece (whole cache lines), so a 32-value
// block (64 bytes) spans four lanes: lane l holds values 8 (l % 4) .. +7 of block 16 k + l / 4 of piece k.
// The block's exponent maximum is reduced over its four lanes; each lane converts its eight values and
// writes them (4 bytes) to the block's 16-byte chunk, and the block's first lane writes the scale byte.
// Rows at or past M are not written (they only feed output columns that are never stored).
template <int MF, int S, int NSL>
__device__ __forceinline__ void quantize_part_impl(const uint8_t* __restrict__ x, int M, int K, int s0, int wave,
                                                   int lane, uint8_t* actb, uint8_t* scb) {
    using C = sk::Cfg<MF, S, NSL>;
    constexpr int kPieces = NSL / 2;  // 1 KB pieces per row
    constexpr int kB = 8;             // pieces in flight per lane
    const int items = M * kPieces;
    const int pc = lane & 3;
    for (int i0 = wave; i0 < items; i0 += 4 * kB) {
        uint4 v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int i = min(i0 + 4 * u, items - 1);  // past the end: reload the last piece (not written)
            const int r = i / kPieces, k = i % kPieces;
            v[u] = ldg16(x + ((int64_t)r * K + (int64_t)s0 * 256 + 512 * k) * 2 + 16 * lane);
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int i = i0 + 4 * u;
            if (i >= items) break;  // wave-uniform
            const int r = i / kPieces, k = i % kPieces;
            uint32_t emax = bf16x8_emax(v[u]);
            emax = max(emax, (uint32_t)__shfl_xor((int)emax, 1));
            emax = max(emax, (uint32_t)__shfl_xor((int)emax, 2));
            const uint32_t scale = mx_scale_of_emax(emax);
            const uint32_t codes = scale == 0xffu ? 0u : bf16x8_codes(v[u], scale);
            const int b = 16 * k + (lane >> 2);  // block within the part
            const int j = b >> 3, c = b & 7;     // slab and chunk within the slab's 128-byte line
            *reinterpret_cast<uint32_t*>(actb + (r * NSL + j) * sk::kSlab + 16 * (c ^ sk::key(r)) + 4 * pc) = codes;
            if (pc == 0) scb[r * 8 * NSL + 16 * ((b / 16 + r) % C::kP) + (b & 15)] = (uint8_t)scale;
        }
    }
}

// KP: K parts (K = 256 NSL KP).  FUSED: the activations arrive as BF16 X [M, K] (in qa; sa unused) and
// each workgroup quantizes its K part into the LDS block itself (the one-launch decode layer).
template <int MF, int S, int NSL, int KP, bool FUSED = false>
__global__ __launch_bounds__(256, 1) void gemm_splitk_fp4(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa,
                                                          const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw,
                                                          uint16_t* __restrict__ y, int M, int N, int K, int tiles,
                                                          uint8_t* __restrict__ ws) {
    using C = sk::Cfg<MF, S, NSL>;
    using sk::key;
    const int b = blockIdx.x;
    const int slot8 = b >> 3;
    const int q = slot8 % KP;                    // K part
    const int t = (slot8 / KP) * 8 + (b & 7);    // tile
    if (t >= tiles) return;                      // the whole workgroup, before any barrier

    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];
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
        quantize_part_impl<MF, S, NSL>(qa, M, K, s0, wave, lane, actb, scb);
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

    v16f acc[MF];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;

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
        }
    });

    // 4. D[n][m] of fragment g: lane l holds column m = 32 g + l32 and rows n = 8 i + 4 h + e in register
    //    4 i + e.  With KP > 1 the partials of the column group (tile t, wave) meet in the workspace.
    const int nw = n0 + 32 * wave + 4 * h;
    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
    auto store_bf16 = [&](const v4f (&v)[MF][4]) {
#pragma unroll
        for (int g = 0; g < MF; ++g) {
            const int m = 32 * g + l32;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = nw + 8 * i;
                uint16_t* dst = y + (int64_t)m * N + n;
                if (vec_ok && n + 3 < N) {
                    uint2 pk;
                    pk.x = bf16x2_rne(v[g][i][0], v[g][i][1]);
                    pk.y = bf16x2_rne(v[g][i][2], v[g][i][3]);
                    *reinterpret_cast<uint2*>(dst) = pk;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) dst[e] = (uint16_t)(bf16x2_rne(v[g][i][e], 0.f) & 0xffffu);
                }
            }
        }
    };
    v4f mine[MF][4];
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[g][i] = v4f{acc[g][4 * i], acc[g][4 * i + 1], acc[g][4 * i + 2], acc[g][4 * i + 3]};
    if constexpr (KP == 1) {
        store_bf16(mine);
        return;
    }
    // partial (t, q', wave, g): 4 KB, float4 i of lane l at + 1024 i + 16 l (whole 1 KB rows per store)
    const size_t group = (size_t)t * 4 + wave;
    auto partial = [&](int qq, int g) {
        return reinterpret_cast<v4f*>(ws + sk::kCounterBytes + ((((size_t)t * KP + qq) * 4 + wave) * MF + g) * 4096) +
               lane;
    };
    uint32_t* const ctr = reinterpret_cast<uint32_t*>(ws) + group;
#pragma unroll
    for (int g = 0; g < MF; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) partial(q, g)[64 * i] = mine[g][i];
    wait_vmcnt<0>();  // the partial is in L2 before the count says so
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(KP - 1)) return;  // another wave of the group arrives later and sums
    asm volatile("" ::: "memory");          // the partial loads stay after the count
    // last of the group: every partial is complete.  The KP - 1 other parts are loaded first, all
    // unconditionally (other part o is part o, or o + 1 from q on); this wave's own part comes from its
    // registers.  Then the sum in K-part order 0, 1, ..., KP - 1, picking each part by a uniform select.
    v4f pv[KP - 1][MF][4];
    static_for<KP - 1>([&](auto oc) {
        constexpr int o = decltype(oc)::value;
        const int part_o = o < q ? o : o + 1;
#pragma unroll
        for (int g = 0; g < MF; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[o][g][i] = partial(part_o, g)[64 * i];
    });
    v4f sum[MF][4];
    static_for<KP>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int below = p < KP - 1 ? p : KP - 2;  // other-part slot of part p when p < q
        constexpr int above = p > 0 ? p - 1 : 0;        // ... when p > q
#pragma unroll
        for (int g = 0; g < MF; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4f v = p == q ? mine[g][i] : (p < q ? pv[below][g][i] : pv[above][g][i]);
                if constexpr (p == 0) sum[g][i] = v;
                else sum[g][i] += v;
            }
    });
    store_bf16(sum);
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mx
