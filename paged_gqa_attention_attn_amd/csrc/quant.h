// quant.h -- the quantisation of the one-byte KV cache (per row, or per channel
// with fixed scales), shared by the quantising append and the decode that fuses
// it, so that both produce the same codes and scales bit for bit.
//
// "LLM 推理全过程的维度变化与核心公式" (research.frankk.site), "KV Cache 的形状与增长":
// the fp16 cache quantised to int8 / fp8 per channel or per token. Read as per-token,
// symmetric absolute-maximum scaling, every step one correctly rounded fp32 operation:
//   amax = max_i |x_i|, scale = amax / QMAX (448 for OCP E4M3, 127 for INT8);
//   scale below the smallest normal float (amax = 0 included): scale = 0, all codes 0;
//   otherwise inv = 1 / scale, y_i = x_i * inv, and the code is the nearest E4M3
//   value of y_i clamped to [-448, 448], or rint(y_i) clamped to [-127, 127].
// The stored value of a code is code * scale.
#pragma once

#include "common.h"

namespace pa {

// Nearest OCP E4M3 code of a finite y with |y| <= 448, ties to the even code: 1
// sign bit, 4 exponent bits (bias 7), 3 fraction bits; exponent field 0 holds the
// subnormals m * 2^-9, and no code past 448 is ever produced.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t sign = __builtin_signbit(y) ? 0x80u : 0u;
    const float a = fabsf(y);
    if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);   // m * 2^-9; 8 is the smallest normal
    int e2;
    const float fr = __builtin_frexpf(a, &e2);   // a = fr * 2^e2, fr in [0.5, 1)
    int e = e2 - 1;
    float q = __builtin_rintf((2.0f * fr - 1.0f) * 8.0f);   // fraction in eighths (exact argument)
    if (q == 8.0f) {
        q = 0.0f;
        ++e;
    }
    return sign | (uint32_t)(((e + 7) << 3) | (int)q);
}

// Element i of a row in the input type, widened exactly to fp32.
template <class SRC> __device__ __forceinline__ float load_f32(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_f32<F32>(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load_f32<BF16>(const void* p, int64_t i) {
    return as_f32((uint32_t) static_cast<const uint16_t*>(p)[i] << 16);
}
template <> __device__ __forceinline__ float load_f32<F16>(const void* p, int64_t i) {
    return (float)__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(p)[i]);
}

// The code of y = x / scale: the nearest E4M3 value of y clamped to [-448, 448], or
// rint(y) clamped to [-127, 127] (one byte, two's complement).
template <bool FP8> __device__ __forceinline__ uint32_t code_of(float y) {
    if constexpr (FP8) {
        return e4m3_code(fminf(fmaxf(y, -448.0f), 448.0f));
    } else {
        return (uint32_t)(int32_t)fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f) & 0xffu;
    }
}

// Per-channel codes (the "per channel" granularity of the same item): element x
// of a channel whose fixed scale s the caller gives. s below the smallest normal
// float stores code 0; otherwise inv = 1 / s, y = x * inv and code_of(y), so a
// value past QMAX * s saturates.
template <bool FP8> __device__ __forceinline__ uint32_t channel_code(float x, float s) {
    if (!(s >= 0x1p-126f)) return 0;
    const float inv = __fdiv_rn(1.0f, s);
    return code_of<FP8>(__fmul_rn(x, inv));
}

// Quantises one row spread over a wave, EPL values per lane (lane l holds row
// elements EPL l .. EPL l + EPL - 1). Returns the row's scale (the same in every
// lane) and this lane's codes, element i in byte i.
template <bool FP8, int EPL>
__device__ __forceinline__ float quantize_row(const float (&x)[EPL], uint32_t& codes) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    constexpr float QMAX = FP8 ? 448.0f : 127.0f;
    float scale = __fdiv_rn(amax, QMAX);
    codes = 0;
    if (scale >= 0x1p-126f) {
        const float inv = __fdiv_rn(1.0f, scale);
#pragma unroll
        for (int i = 0; i < EPL; ++i) codes |= code_of<FP8>(__fmul_rn(x[i], inv)) << (8 * i);
    } else {
        scale = 0.f;
    }
    return scale;
}

}  // namespace pa
