// mfma.h -- gfx950 matrix-core building blocks shared by the prefill and
// multi-row decode kernels: vector types, the 32x32x16 bf16/f16 MFMA with
// packing of fp32 probabilities into its operand type, and the XOR swizzle of
// 16-byte chunks used for K/V tiles in LDS.
#pragma once

#include "common.h"

namespace pa {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

template <class E> struct Mfma;
template <> struct Mfma<BF16> {
    // bf16 probabilities keep 8 bits; P = hi + lo, both bf16, keeps ~16.
    static constexpr bool kSplit = true;
    static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    // Two fp32 values as the element type (round to nearest even), x in the low half.
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        const bf16x2_t v = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ float lo_of(uint32_t w) { return as_f32(w << 16); }
    static __device__ __forceinline__ float hi_of(uint32_t w) { return as_f32(w & 0xffff0000u); }
};
template <> struct Mfma<F16> {
    static constexpr bool kSplit = false;
    static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        const f16x2_t v = {(_Float16)x, (_Float16)y};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ float lo_of(uint32_t) { return 0.f; }
    static __device__ __forceinline__ float hi_of(uint32_t) { return 0.f; }
};

// Position of 16-byte chunk c of row r within an unpadded LDS row of CPR chunks:
// c ^ chunk_swizzle<CPR>(r). For 16 consecutive rows the masks are distinct (a
// K operand read takes one chunk column of 16 rows), and for 4 aligned rows they
// differ in bits 2-3 (a V^T transposing read takes 4 rows x 4 chunks), so
// neither pattern hits one of the 64 LDS banks twice.
template <int CPR> __device__ __forceinline__ int chunk_swizzle(int r) {
    return (((r & 3) << 2) | ((r >> 2) & 3)) & (CPR - 1);
}

}  // namespace pa
