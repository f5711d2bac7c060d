// quant_mx.hip - MXFP4 quantization (E2M1 codes + one E8M0 scale per 32 K-values).
//
// Format: "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact quantization
// coverage" (32 consecutive input-channel values share one E8M0 scale; dynamic
// MXFP4 activations); standard "OCP MXFP4" named by "Kimi-K3-Quark-MXFP4-
// AttnFP8", section "Model Quantization".
//
// Both inputs go through gfx950's scaled FP4 conversion, which divides by the power-of-two scale
// and rounds to the nearest E2M1 value {0, .5, 1, 1.5, 2, 3, 4, 6}: ties to the even code, magnitudes
// above 6 saturate at 6, the sign is kept.  The shared exponent is the block's largest biased exponent
// field E; scale byte = max(E - 2, 0), which is floor(log2 amax) - 2 + 127 clamped at the bottom of the
// E8M0 range; E == 255 (NaN/Inf in the block) gives scale 0xFF and codes 0.  The GPU tests compare
// every finite BF16 pattern, and every FP32 mantissa of each binade that can round to a non-zero code
// at several scale bytes (subnormal ones included), with the oracle.
//   * BF16 input (activations): one lane owns one 32-value block (four 16-byte loads, one 16-byte code
//     store, one scale byte).
//   * FP32 input (offline weights): four lanes own one block, eight values (two 16-byte loads) each;
//     the block's exponent maximum is a 4-lane DPP max; one 32-bit store of 8 nibbles per lane
//     (element 2j in the low nibble of byte j), one scale byte per block.  The conversion replaced an
//     exact integer-compare ladder (the same decisions, about 200 VALU operations per 8 values), which
//     left this kernel ALU-bound: 7168 x 8192 FP32 went from 64-68 us to 47.6 us (5.6 TB/s).
#include "launch.hpp"
#include "mx_device.hpp"

namespace mx {
namespace {

// One "unit" = 8 consecutive values = one quarter of a block.  units % 4 == 0
// and every stride is a multiple of 4, so the four lanes of a block always
// iterate together (the 4-lane DPP max below sees only active lanes).
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
    const uint32_t w[8] = {x.a.x, x.a.y, x.a.z, x.a.w, x.b.x, x.b.y, x.b.z, x.b.w};
    uint32_t mag = 0;  // largest magnitude bit pattern: its exponent field is the largest one
#pragma unroll
    for (int i = 0; i < 8; ++i) mag = max(mag, w[i] & 0x7fffffffu);
    const uint32_t scale = mx_scale_of_emax(quad_max(mag >> 23));
    uint32_t codes = 0;
    if (scale != 0xffu) {
        // 2^(scale - 127) as an FP32 bit pattern (subnormal for scale byte 0)
        const float sc = __uint_as_float(scale ? scale << 23 : 1u << 22);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __uint_as_float(w[0]), __uint_as_float(w[1]), sc, 0);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, __uint_as_float(w[2]), __uint_as_float(w[3]), sc, 1);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, __uint_as_float(w[4]), __uint_as_float(w[5]), sc, 2);
        codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, __uint_as_float(w[6]), __uint_as_float(w[7]), sc, 3);
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
