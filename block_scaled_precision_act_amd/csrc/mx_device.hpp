// mx_device.hpp - device-side helpers shared by the gfx950 kernels of libmxgemm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace mx {

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled at compile time, so
// indices can select registers, immediates and template arguments.
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

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
__device__ __forceinline__ v8i fp4_operand(unsigned __attribute__((ext_vector_type(4))) x) {
    v8i r = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
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

// Two binary32 -> two bfloat16 (low half = a), round to nearest even, NaN stays NaN
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// PTPC epilogue value acc * sa * sw: the FP32 sum and the two FP32 scales are multiplied in FP64,
// where the scale product is exact and nothing over- or underflows, then rounded to FP32 once (the
// caller rounds that to BF16).  In FP32 the product of the three could overflow or underflow part
// way although the result is an ordinary number (a 2^118 row scale against a 2^-60 column scale).
__device__ __forceinline__ float ptpc_scaled(float acc, float sa, float sw) {
    return (float)((double)acc * ((double)sa * (double)sw));
}

// 16 bytes per lane from global memory straight into LDS: lane i of the wave writes
// lds_base + 16 * i (lds_base must be the same for the whole wave).
__device__ __forceinline__ void g2lds16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Same, non-temporal (streamed data: allocate in the caches with evict-first priority).
__device__ __forceinline__ void g2lds16_nt(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 2);
}

// s_waitcnt vmcnt(N) (other counters untouched), N < 64.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS reads issued as inline asm: the compiler does not see them as LDS accesses, so it
// does not drain outstanding global->LDS loads before them.  The caller orders them after
// its own explicit vmcnt wait + barrier, and must call lds_wait_* on the results before use.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4u lds_read16(uint32_t addr) {
    v4u v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ uint32_t lds_read4(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
// ds_read_b128 at addr + OFF (OFF an immediate, < 65536).
template <int OFF>
__device__ __forceinline__ v4u lds_read16_at(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
    v4u v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}
// 16-bit LDS read at addr + OFF, zero-extended (2-byte aligned).
template <int OFF>
__device__ __forceinline__ uint32_t lds_read2_at(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
    uint32_t v;
    asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}
// D += A(16x128) . B(128x16), E2M1 operands with per-lane E8M0 scales (byte OPSEL of sa and sb),
// written as inline asm with the accumulator tied to AGPRs: the register allocator then keeps
// every accumulator in place (with 56 accumulators of 4 registers, the builtin's results were
// shuffled between register files on every loop iteration).  The compiler does not know this is
// an MFMA, so the caller owns its hazards: wait states between a VALU write of an operand or of
// the accumulator and the MFMA, and between the last MFMA and a read of the accumulator.
template <int OPSEL>
__device__ __forceinline__ void mfma16_fp4_agpr(v4f& c, v4u a, v4u b, uint32_t sa, uint32_t sb) {
    static_assert(OPSEL == 0 || OPSEL == 1, "scale byte 0 or 1");
    if constexpr (OPSEL == 0)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+a"(c)
                     : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,1,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+a"(c)
                     : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// D += A(16x32) . B(32x16), FP16 operands, FP32 accumulation, as inline asm with the accumulator
// tied to AGPRs (see mfma16_fp4_agpr: the caller owns the wait states around it).
__device__ __forceinline__ void mfma16_f16_agpr(v4f& c, v8h a, v8h b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Marks a VALU result as produced here (volatile asm statements keep their order), so it cannot
// be computed any later: a caller places this a few instructions before an inline-asm MFMA that
// reads the value.
__device__ __forceinline__ void vgpr_tie(v8h& x) { asm volatile("" : "+v"(x)); }
// s_nop 7, N times (8 N wait states).
template <int N>
__device__ __forceinline__ void wait_states8() {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("s_nop 7");
}
// s_waitcnt lgkmcnt(N) (N < 16); the caller ties the results it waited for with lds_tie.
template <int N>
__device__ __forceinline__ void lds_wait() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// After an lds_wait: marks LDS-read results as produced here, so no use of them moves above the wait.
template <int L>
__device__ __forceinline__ void lds_tie(v4u (&a)[L]) {
#pragma unroll
    for (int i = 0; i < L; ++i) asm volatile("" : "+v"(a[i]));
}
template <int L>
__device__ __forceinline__ void lds_tie(uint32_t (&a)[L]) {
#pragma unroll
    for (int i = 0; i < L; ++i) asm volatile("" : "+v"(a[i]));
}
// 4-byte global -> LDS (lane i writes lds_base + 4 * i).
__device__ __forceinline__ void g2lds4(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// lgkmcnt(8): all but the last eight LDS reads done; ties four 16-byte and four 4-byte
// results of each of two groups to the wait.
__device__ __forceinline__ void lds_wait_first(v4u (&a)[4], v4u (&b)[4], uint32_t (&c)[4], uint32_t (&d)[4]) {
    asm volatile("s_waitcnt lgkmcnt(8)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]),
                   "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
}
// lgkmcnt(0) tied to four 16-byte results of each of two groups.
__device__ __forceinline__ void lds_wait_rest(v4u (&a)[4], v4u (&b)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}

// lgkmcnt(N) tied to four 16-byte results of each of two groups.
template <int N>
__device__ __forceinline__ void lds_wait_n(v4u (&a)[4], v4u (&b)[4]) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
                 : "n"(N));
}

// lgkmcnt(0) tied to the decode kernel's per-slab operands and scales.
template <int MF>
__device__ __forceinline__ void lds_wait_dec(v4u (&w)[4], v4u (&x)[4][MF], uint32_t& ws, uint32_t (&xs)[MF]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(ws));
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int g = 0; g < MF; ++g) asm volatile("" : "+v"(x[t][g]));
#pragma unroll
    for (int g = 0; g < MF; ++g) asm volatile("" : "+v"(xs[g]));
}

// lgkmcnt(0) tied to the FP8 decode kernel's per-slab operands.
template <int MF>
__device__ __forceinline__ void lds_wait_codes(v4u (&w)[4], v4u (&x)[4][MF]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int g = 0; g < MF; ++g) asm volatile("" : "+v"(x[t][g]));
}

// lgkmcnt(2 FW): scales (2 FW dwords) and the first FW + FW operands done, tied to them.
template <int FW>
__device__ __forceinline__ void lds_wait_first_n(v4u (&a)[FW], v4u (&b)[FW], uint32_t (&c)[FW], uint32_t (&d)[FW]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(2 * FW));
#pragma unroll
    for (int i = 0; i < FW; ++i) asm volatile("" : "+v"(a[i]), "+v"(b[i]), "+v"(c[i]), "+v"(d[i]));
}
// lgkmcnt(N) tied to FW 16-byte results of each of two groups.
template <int N, int FW>
__device__ __forceinline__ void lds_wait_n_of(v4u (&a)[FW], v4u (&b)[FW]) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
#pragma unroll
    for (int i = 0; i < FW; ++i) asm volatile("" : "+v"(a[i]), "+v"(b[i]));
}

// MXFP4 quantization of one 32-value BF16 block (four 16-byte loads, values 8i .. 8i+7 in x[i]) by
// one lane.  Returns the block's 16 code bytes (value 2j in the low nibble of byte j) and sets scale
// to its E8M0 byte: max(E - 2, 0) for the largest exponent field E of the block, 0xFF with zero
// codes if the block holds a NaN or an infinity.  The codes come from gfx950's scaled conversion,
// which divides by the power-of-two scale and rounds to the nearest E2M1 value, ties to the even
// code, saturating at 6 and keeping the sign.
// Largest biased exponent field of eight BF16 values (one 16-byte piece of a block).
__device__ __forceinline__ uint32_t bf16x8_emax(uint4 x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t emax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) emax = max(emax, max((w[j] >> 7) & 0xffu, (w[j] >> 23) & 0xffu));
    return emax;
}
// Maximum of v over the four lanes of a quad (lanes 4j .. 4j + 3), via DPP lane swaps (xor 1, then
// xor 2): no LDS round trip.  Every lane of the quad must be active.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    return v;
}
// E8M0 scale byte of a block from its largest exponent field: max(E - 2, 0), 0xFF for NaN/Inf.
__device__ __forceinline__ uint32_t mx_scale_of_emax(uint32_t emax) {
    return emax == 0xffu ? 0xffu : (emax > 2u ? emax - 2u : 0u);
}
// Eight BF16 values -> eight E2M1 codes (value 2j in the low nibble of byte j) at scale byte `scale`
// (not 0xFF): gfx950's scaled conversion divides by 2^(scale - 127), an FP32 bit pattern that is
// subnormal for scale bytes 0 and 1, and rounds to the nearest E2M1 value (ties to the even code,
// saturating at 6, sign kept).
__device__ __forceinline__ uint32_t bf16x8_codes(uint4 x, uint32_t scale) {
    const float sc = __uint_as_float(scale ? scale << 23 : 1u << 22);  // 2^(scale - 127)
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    uint32_t v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf2, x.x), sc, 0);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, __builtin_bit_cast(bf2, x.y), sc, 1);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, __builtin_bit_cast(bf2, x.z), sc, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(v, __builtin_bit_cast(bf2, x.w), sc, 3);
}

__device__ __forceinline__ uint4 mx_bf16x32_codes(const uint4 (&x)[4], uint32_t& scale) {
    uint32_t emax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) emax = max(emax, bf16x8_emax(x[i]));
    scale = mx_scale_of_emax(emax);
    if (scale == 0xffu) return make_uint4(0u, 0u, 0u, 0u);  // NaN or Inf in the block
    return make_uint4(bf16x8_codes(x[0], scale), bf16x8_codes(x[1], scale), bf16x8_codes(x[2], scale),
                      bf16x8_codes(x[3], scale));
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
// 16-byte load of data used once (non-temporal hint: evict first from the caches).
__device__ __forceinline__ uint4 ldg16_stream(const uint8_t* p) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ int ldg4(const uint8_t* p) { return *reinterpret_cast<const int*>(p); }

}  // namespace mx
