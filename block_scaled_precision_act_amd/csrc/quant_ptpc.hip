// quant_ptpc.hip - per-token (activations) / per-output-channel (weights) FP8 E4M3 quantization.
//
// Scheme: "Kimi-K3-DSpark-FP8-PTPC", section "Phase 1 FP8 PTPC Quantization":
// float8_e4m3fn values with one FP32 scale per row (per output channel for the
// weight, (out_features, 1); per token for activations, computed online).
//
// Per row: a = max|x| (exact integer max over the magnitude bit patterns),
// s = fl32(a / 448) (s = 1 if a == 0), code = E4M3fn(fl32(x / s)) with
// round-to-nearest-even and saturation at 448.  Both divisions are IEEE
// binary32 divisions (hipcc's default for '/' on float is correctly rounded).
// A row holding NaN or Inf gets s = NaN and every code 0x7F.
//
// One 256-thread workgroup per row (grid-stride over rows).  A row of up to
// 256 * 8 * kVec values stays in registers between the max pass and the encode
// pass, so X is read from HBM once; longer rows re-read it (from L2).
#include "launch.hpp"
#include "mx_device.hpp"

namespace mx {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;  // 8-value vectors per thread kept in registers

// E4M3fn code of a finite binary32 r: round to nearest even, saturate at 448.
__device__ __forceinline__ uint32_t e4m3fn_rne_sat(float r) {
    const uint32_t sign = (__float_as_uint(r) >> 24) & 0x80u;
    const float a = fabsf(r);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7eu;
    } else if (a < 0.015625f) {  // below 2^-6: subnormal grid, step 2^-9; 8 steps == 2^-6 == code 0x08
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        const uint32_t e = __float_as_uint(a) >> 23;                  // biased binary32 exponent, 121..135
        const float scaled = a * __uint_as_float((257u - e) << 23);   // a / 2^(e-130): exact, in [8, 16)
        const uint32_t m = (uint32_t)rintf(scaled);                    // 8..16; 16 carries into the exponent
        code = ((e - 120u) << 3) + (m - 8u);                           // E4M3 biased exponent = e - 127 + 7
    }
    return sign | code;
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
    __device__ __forceinline__ void fold(uint32_t& amax_bits, uint32_t& nonfinite) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t m = __float_as_uint(v[i]) & 0x7fffffffu;
            nonfinite |= (uint32_t)(m >= 0x7f800000u);
            amax_bits = max(amax_bits, m < 0x7f800000u ? m : 0u);
        }
    }
    __device__ __forceinline__ uint2 encode(float s) const {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo |= e4m3fn_rne_sat(v[i] / s) << (8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) hi |= e4m3fn_rne_sat(v[4 + i] / s) << (8 * i);
        return make_uint2(lo, hi);
    }
};

template <bool F32>
__global__ __launch_bounds__(kThreads) void quant_ptpc_kernel(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                               float* __restrict__ s, int64_t rows, int64_t K) {
    __shared__ uint32_t red_max[kThreads / 64], red_nf[kThreads / 64];
    const int64_t nvec = K / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const void* xrow = F32 ? (const void*)((const float*)x + row * K) : (const void*)((const uint16_t*)x + row * K);
        uint2* qrow = reinterpret_cast<uint2*>(q + row * K);
        Row8<F32> reg[kVec];
        uint32_t amax_bits = 0, nonfinite = 0;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int64_t v = threadIdx.x + (int64_t)j * kThreads;
            if (v < nvec) {
                reg[j].load(xrow, v);
                reg[j].fold(amax_bits, nonfinite);
            }
        }
        for (int64_t v = threadIdx.x + (int64_t)kVec * kThreads; v < nvec; v += kThreads) {
            Row8<F32> t;
            t.load(xrow, v);
            t.fold(amax_bits, nonfinite);
        }
        // wave then workgroup reduction (exact: integer max / or)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off));
            nonfinite |= (uint32_t)__shfl_xor((int)nonfinite, off);
        }
        if (lane == 0) {
            red_max[wave] = amax_bits;
            red_nf[wave] = nonfinite;
        }
        __syncthreads();
        amax_bits = red_max[0];
        nonfinite = red_nf[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) {
            amax_bits = max(amax_bits, red_max[w]);
            nonfinite |= red_nf[w];
        }
        __syncthreads();  // red_* is rewritten by the next row
        const float amax = __uint_as_float(amax_bits);
        const float sc = nonfinite ? __uint_as_float(0x7fc00000u) : (amax_bits == 0 ? 1.0f : amax / 448.0f);
        if (threadIdx.x == 0) s[row] = sc;
        if (nonfinite) {
            for (int64_t v = threadIdx.x; v < nvec; v += kThreads) qrow[v] = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
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
