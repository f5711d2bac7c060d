// mx_device.hpp - device-side helpers shared by the gfx950 kernels of libmxgemm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Scaled-MFMA operand format (cbsz / blgp field value) of E2M1.
constexpr int kFmtFP4 = 4;

// An FP4 MFMA operand occupies the low 4 dwords of the 8-dword operand.
__device__ __forceinline__ v8i fp4_operand(uint4 x) {
    v8i r = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    return r;
}

// Two E4M3 codes (the low or high 16 bits of w) -> two FP16 values, exactly:
// every finite E4M3 value (max 448, smallest 2^-9) is an FP16 normal.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    const v2h h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, h);
}

// Eight E4M3 codes (two dwords) -> one 8 x FP16 MFMA operand.
__device__ __forceinline__ v8h e4m3x8_to_f16x8(uint32_t w0, uint32_t w1) {
    const uint4 u = make_uint4(e4m3x2_to_f16x2<false>(w0), e4m3x2_to_f16x2<true>(w0), e4m3x2_to_f16x2<false>(w1),
                               e4m3x2_to_f16x2<true>(w1));
    return __builtin_bit_cast(v8h, u);
}

// D += A(16x128) . B(128x16) with per-lane E8M0 scales; OPSEL picks the scale byte.
template <int FMT, int OPSEL>
__device__ __forceinline__ v4f mfma16(v8i a, v8i b, v4f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, OPSEL, sa, OPSEL, sb);
}

// D += A(32x64) . B(64x32) with per-lane E8M0 scales; OPSEL picks the scale byte.
template <int FMT, int OPSEL>
__device__ __forceinline__ v16f mfma32(v8i a, v8i b, v16f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, OPSEL, sa, OPSEL, sb);
}

// D += A(16x32) . B(32x16), FP16 operands, FP32 accumulation.
__device__ __forceinline__ v4f mfma16_f16(v8h a, v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D += A(32x16) . B(16x32), FP16 operands, FP32 accumulation.
__device__ __forceinline__ v16f mfma32_f16(v8h a, v8h b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// binary32 -> bfloat16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ int ldg4(const uint8_t* p) { return *reinterpret_cast<const int*>(p); }

}  // namespace mx
