// quant_mx.hip - MXFP4 quantization (E2M1 codes + one E8M0 scale per 32 K-values).
//
// Format: "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact quantization
// coverage" (32 consecutive input-channel values share one E8M0 scale; dynamic
// MXFP4 activations); standard "OCP MXFP4" named by "Kimi-K3-Quark-MXFP4-
// AttnFP8", section "Model Quantization".
//
// BF16 input (activations): one lane owns one 32-value block (four 16-byte loads,
// one 16-byte code store, one scale byte), using gfx950's scaled FP4 conversion,
// which takes the decisions below (the GPU tests compare every finite BF16
// pattern with the oracle).  FP32 input (offline weights): four lanes own one
// block, eight values (two 16-byte loads) each:
//   * shared exponent: the largest biased exponent field E of the block (a
//     4-lane max); scale byte = max(E - 2, 0), which is floor(log2 amax) - 2
//     + 127 clamped at the bottom of the E8M0 range; E == 255 (NaN/Inf in the
//     block) gives scale 0xFF and codes 0.
//   * element: with significand sig (hidden bit included; P fraction bits) and
//     effective exponent Ee = max(E, 1), |x| / 2^(scale-127) times 4 equals
//     sig / 2^u with u = scale + P - 2 - Ee >= P - 4, so every round-to-nearest-
//     even decision on the E2M1 grid {0,.5,1,1.5,2,3,4,6} is an exact integer
//     compare of sig against (midpoint*4) << u; ties at 0.25, 1.25, 2.5 and 5
//     stay below (even code), ties at 0.75, 1.75 and 3.5 go up; above 6 the
//     code saturates at 7.
//   * one 32-bit store of 8 nibbles per lane (element 2j in the low nibble of
//     byte j), one scale byte per block.
// HBM-bound: 2 (or 4) bytes in, 0.5 + 1/32 bytes out per value.
#include "launch.hpp"
#include "mx_device.hpp"

namespace mx {
namespace {

// magnitude code 0..7 of sig / 2^(u+2) on the E2M1 grid (see file comment)
__device__ __forceinline__ uint32_t e2m1_magnitude(uint32_t sig, uint32_t u) {
    return (uint32_t)(sig > (1u << u)) + (uint32_t)(sig >= (3u << u)) + (uint32_t)(sig > (5u << u)) +
           (uint32_t)(sig >= (7u << u)) + (uint32_t)(sig > (10u << u)) + (uint32_t)(sig >= (14u << u)) +
           (uint32_t)(sig > (20u << u));
}

template <int P>  // fraction bits of the input format (7 for BF16, 23 for FP32)
__device__ __forceinline__ uint32_t encode8(const uint32_t (&mag)[8], uint32_t scale) {
    uint32_t codes = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t e = mag[i] >> P;
        uint32_t sig = (mag[i] & ((1u << P) - 1u)) | (e ? (1u << P) : 0u);
        uint32_t ee = e ? e : 1u;
        uint32_t u = scale + (uint32_t)P - 2u - ee;
        u = u < (uint32_t)(P + 1) ? u : (uint32_t)(P + 1);  // beyond P+1 every threshold exceeds sig
        codes |= e2m1_magnitude(sig, u) << (4 * i);
    }
    return codes;
}

// One "unit" = 8 consecutive values = one quarter of a block.  units % 4 == 0
// and every stride is a multiple of 4, so the four lanes of a block always
// iterate together (the 4-lane shuffles below stay inside active lanes).
// FP32: eight values (two 16-byte loads) per lane, four lanes per block
struct Unit {
    uint4 a, b;
};

__device__ __forceinline__ Unit load_unit(const void* __restrict__ xin, int64_t u) {
    const uint4* p = reinterpret_cast<const uint4*>(xin) + 2 * u;
    return Unit{p[0], p[1]};
}

__device__ __forceinline__ void convert_unit(const Unit& x, uint32_t* __restrict__ q, uint8_t* __restrict__ s,
                                             int64_t u) {
    constexpr int P = 23;
    uint32_t codes, scale;
    uint32_t mag[8];
    uint32_t sgn = 0, emax = 0;
    const uint32_t w[8] = {x.a.x, x.a.y, x.a.z, x.a.w, x.b.x, x.b.y, x.b.z, x.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sgn |= (w[i] >> 31) << (4 * i + 3);
        mag[i] = w[i] & 0x7fffffffu;
        emax = max(emax, mag[i] >> 23);
    }
    emax = max(emax, (uint32_t)__shfl_xor((int)emax, 1));
    emax = max(emax, (uint32_t)__shfl_xor((int)emax, 2));
    if (emax == 0xffu) {  // NaN or Inf in the block
        scale = 0xffu;
        codes = 0;
    } else {
        scale = emax > 2u ? emax - 2u : 0u;
        codes = encode8<P>(mag, scale) | sgn;
    }
    q[u] = codes;
    if ((u & 3) == 0) s[u >> 2] = (uint8_t)scale;
}

// Grids as large as the input (capped, then grid-stride): the dispatcher keeps every CU streaming as
// workgroups retire, which measured faster (M = 8192, K = 8192, BF16: 33.7 -> 30.6 us) than 2048
// workgroups each keeping four loads per thread in flight.  One lane per block for BF16 then
// measured faster again (31.2 -> 28.0 us): a wave writes 64 contiguous scale bytes and 1 KB of codes
// instead of 16 scale bytes and 256 bytes of codes.
constexpr int64_t kMaxBlocks = 1 << 20;

__global__ __launch_bounds__(256) void quant_mx_bf16_kernel(const uint4* __restrict__ x, uint4* __restrict__ q,
                                                             uint8_t* __restrict__ s, int64_t blocks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < blocks; b += stride) {
        const uint4 v[4] = {x[4 * b], x[4 * b + 1], x[4 * b + 2], x[4 * b + 3]};
        uint32_t scale;
        q[b] = mx_bf16x32_codes(v, scale);
        s[b] = (uint8_t)scale;
    }
}

__global__ __launch_bounds__(256) void quant_mx_f32_kernel(const void* __restrict__ xin, uint32_t* __restrict__ q,
                                                            uint8_t* __restrict__ s, int64_t units) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += stride)
        convert_unit(load_unit(xin, u), q, s, u);
}

int64_t grid_for(int64_t items, int64_t threads = 256) {
    const int64_t g = (items + threads - 1) / threads;
    return g < kMaxBlocks ? g : kMaxBlocks;
}

}  // namespace

hipError_t launch_quant_mx_bf16(const void* x, int64_t rows, int64_t K, void* q, void* s, hipStream_t st) {
    const int64_t blocks = rows * (K / 32);
    // small inputs (the decode layer: 64 x 8192 is 16384 blocks) in single-wave workgroups, so they
    // still spread over the CUs
    const int64_t threads = blocks < 256 * 256 ? 64 : 256;
    hipLaunchKernelGGL(quant_mx_bf16_kernel, dim3((unsigned)grid_for(blocks, threads)), dim3((unsigned)threads), 0, st,
                       reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(q), reinterpret_cast<uint8_t*>(s),
                       blocks);
    return hipGetLastError();
}

hipError_t launch_quant_mx_f32(const void* x, int64_t rows, int64_t K, void* q, void* s, hipStream_t st) {
    const int64_t units = rows * (K / 8);
    hipLaunchKernelGGL(quant_mx_f32_kernel, dim3((unsigned)grid_for(units)), dim3(256), 0, st, x,
                       reinterpret_cast<uint32_t*>(q), reinterpret_cast<uint8_t*>(s), units);
    return hipGetLastError();
}

}  // namespace mx
