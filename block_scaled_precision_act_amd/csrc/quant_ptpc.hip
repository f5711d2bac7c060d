// quant_ptpc.hip - per-token (activations) / per-output-channel (weights) FP8 E4M3 quantization.
//
// Scheme: "Kimi-K3-DSpark-FP8-PTPC", section "Phase 1 FP8 PTPC Quantization":
// float8_e4m3fn values with one FP32 scale per row (per output channel for the
// weight, (out_features, 1); per token for activations, computed online).
//
// Per row: a = max|x| (exact integer max over the magnitude bit patterns),
// s = fl32(a / 448) (s = 1 if a == 0), code = E4M3fn(fl32(x / s)) with
// round-to-nearest-even and saturation at 448.  Both divisions are IEEE
// binary32 divisions (hipcc's default for '/' on float is correctly rounded);
// for BF16 rows the per-element one is computed by div_corrected, which gives
// the same codes.
// A row holding NaN or Inf gets s = NaN and every code 0x7F.
//
// One 512-thread workgroup per row (grid-stride over rows).  A row of up to
// 512 * 8 * kVec values stays in registers between the max pass and the encode
// pass, so X is read from HBM once; longer rows re-read it (from L2).  The row
// maximum is one integer max over the magnitude bit patterns (an infinity or a
// NaN makes it >= 0x7F800000), by DPP lane swaps and readlanes within a wave and
// through LDS across waves; two shfl_xor chains (LDS round trips, one for the
// max and one for a non-finite flag) measured slower: BF16 64 x 8192 3.55 ->
// 2.92 us, 8192 x 8192 44.5 -> 39.3 us.
// Encoding: gfx950's v_cvt_pk_fp8_f32 rounds binary32 to E4M3fn to nearest
// even, keeping the sign; an exhaustive comparison with the exact rule (the
// magnitude rounded onto the E4M3 grid - subnormal step 2^-9, 3 fraction bits
// above 2^-6 - ties to the even code) over every binary32 of magnitude <= 464,
// both signs, subnormals included, found no difference.  Quotients here never
// exceed 448 * (1 + 2^-23) < 464 (|x| <= a and s = fl32(a / 448)), so its
// behaviour past the largest finite code never matters.
#include "launch.hpp"
#include "mx_device.hpp"

namespace mx {
namespace {

constexpr int kThreads = 512;
constexpr int kVec = 2;  // 8-value vectors per thread kept in registers

// fl32(x / s) for BF16 rows: r = fl32(1 / s) once per row, then the quotient q0 = fl32(x r) is
// corrected twice with the remainder x - q s (exact, an FMA) scaled by r (Markstein's method); the
// sign of x is restored for zeros.  Used only when s >= 2^-90, so that every remainder that can
// decide a code is a normal number.  An exhaustive comparison with the IEEE division, over every
// finite positive BF16 row maximum a (s = fl32(a / 448) >= 2^-90) and every BF16 x with |x| <= a,
// found the same quotient wherever it is at least 2^-10 (below that every code is a signed zero)
// and the same E4M3 code everywhere.
__device__ __forceinline__ float div_corrected(float x, float s, float r) {
    const float q0 = x * r;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
    const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, s, x), r, q1);
    return __builtin_copysignf(q2, x);
}

// E4M3fn codes of four binary32 quotients (|r| < 464), round to nearest even, packed low to high.
__device__ __forceinline__ uint32_t e4m3fn_x4(float r0, float r1, float r2, float r3) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, lo, true);
}

template <bool F32>
struct Row8 {  // eight consecutive values of a row as binary32
    float v[8];
    __device__ __forceinline__ void load(const void* base, int64_t vec) {
        if constexpr (F32) {
            const uint4* p = reinterpret_cast<const uint4*>(base) + 2 * vec;
            const uint4 a = p[0], b = p[1];
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
        } else {
            const uint4 a = reinterpret_cast<const uint4*>(base)[vec];
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    }
    // largest magnitude bit pattern: the row maximum when it is below 0x7F800000, else the row holds
    // an infinity or a NaN
    __device__ __forceinline__ void fold(uint32_t& mag_max) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) mag_max = max(mag_max, __float_as_uint(v[i]) & 0x7fffffffu);
    }
    __device__ __forceinline__ uint2 encode(float s) const {
        return make_uint2(e4m3fn_x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s),
                          e4m3fn_x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s));
    }
    __device__ __forceinline__ uint2 encode_corrected(float s, float r) const {  // BF16 rows, s >= 2^-90
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = div_corrected(v[i], s, r);
        return make_uint2(e4m3fn_x4(q[0], q[1], q[2], q[3]), e4m3fn_x4(q[4], q[5], q[6], q[7]));
    }
};

// Maximum of v over the wave: DPP lane swaps within each row of 16 lanes (quad swaps, then the half-row
// and row mirrors), then the four row maxima by readlane.  No LDS round trip; every lane must be active.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

template <bool F32>
__global__ __launch_bounds__(kThreads) void quant_ptpc_kernel(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                               float* __restrict__ s, int64_t rows, int64_t K) {
    __shared__ uint32_t red[2][kThreads / 64];  // by row parity: a row's slots are rewritten two rows later
    const int64_t nvec = K / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int par = 0;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x, par ^= 1) {
        const void* xrow = F32 ? (const void*)((const float*)x + row * K) : (const void*)((const uint16_t*)x + row * K);
        uint2* qrow = reinterpret_cast<uint2*>(q + row * K);
        Row8<F32> reg[kVec];
        uint32_t mag_max = 0;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int64_t v = threadIdx.x + (int64_t)j * kThreads;
            if (v < nvec) {
                reg[j].load(xrow, v);
                reg[j].fold(mag_max);
            }
        }
        for (int64_t v = threadIdx.x + (int64_t)kVec * kThreads; v < nvec; v += kThreads) {
            Row8<F32> t;
            t.load(xrow, v);
            t.fold(mag_max);
        }
        // wave then workgroup maximum (exact: an integer max).  Every wave passes this row's barrier
        // after reading red[par] and before writing red[par ^ 1]; the next writes of red[par] come after
        // the next row's barrier, so one barrier per row suffices.
        mag_max = wave_max(mag_max);
        if (lane == 0) red[par][wave] = mag_max;
        __syncthreads();
        mag_max = red[par][0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) mag_max = max(mag_max, red[par][w]);
        const bool nonfinite = mag_max >= 0x7f800000u;
        const uint32_t amax_bits = mag_max;
        const float amax = __uint_as_float(amax_bits);  // used only when finite
        const float sc = nonfinite ? __uint_as_float(0x7fc00000u) : (amax_bits == 0 ? 1.0f : amax / 448.0f);
        if (threadIdx.x == 0) s[row] = sc;
        if (nonfinite) {
            for (int64_t v = threadIdx.x; v < nvec; v += kThreads) qrow[v] = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
            continue;
        }
        if (!F32 && sc >= 0x1p-90f) {  // row-uniform
            const float rc = 1.0f / sc;
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int64_t v = threadIdx.x + (int64_t)j * kThreads;
                if (v < nvec) qrow[v] = reg[j].encode_corrected(sc, rc);
            }
            for (int64_t v = threadIdx.x + (int64_t)kVec * kThreads; v < nvec; v += kThreads) {
                Row8<F32> t;
                t.load(xrow, v);
                qrow[v] = t.encode_corrected(sc, rc);
            }
            continue;
        }
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int64_t v = threadIdx.x + (int64_t)j * kThreads;
            if (v < nvec) qrow[v] = reg[j].encode(sc);
        }
        for (int64_t v = threadIdx.x + (int64_t)kVec * kThreads; v < nvec; v += kThreads) {
            Row8<F32> t;
            t.load(xrow, v);
            qrow[v] = t.encode(sc);
        }
    }
}

template <bool F32>
hipError_t launch(const void* x, int64_t rows, int64_t K, void* q, float* s, hipStream_t st) {
    int64_t blocks = rows < (1 << 20) ? rows : (1 << 20);
    hipLaunchKernelGGL(quant_ptpc_kernel<F32>, dim3((unsigned)blocks), dim3(kThreads), 0, st, x,
                       reinterpret_cast<uint8_t*>(q), s, rows, K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_ptpc_bf16(const void* x, int64_t rows, int64_t K, void* q, float* s, hipStream_t st) {
    return launch<false>(x, rows, K, q, s, st);
}

hipError_t launch_quant_ptpc_f32(const void* x, int64_t rows, int64_t K, void* q, float* s, hipStream_t st) {
    return launch<true>(x, rows, K, q, s, st);
}

}  // namespace mx
