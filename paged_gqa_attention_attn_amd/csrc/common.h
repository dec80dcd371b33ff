// common.h -- device helpers shared by the gfx950 kernels of the paged attention library.
//
// Element types, 16-byte chunk dot products, widening of stored values, and
// wavefront (64-lane) cross-lane reductions built from DPP and the gfx950
// permlane swaps. Nothing here is specific to one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// Element type tags: storage type and the dot product of two packed 16-byte chunks.
struct F32 {
    using storage = float;
};
struct BF16 {
    using storage = uint16_t;
};
struct F16 {
    using storage = uint16_t;
};

// Sliding window over a paged context of ctx positions whose last `rows` are
// query rows: the first position any of them attends to (0 without a window).
// The query at position p sees p - window + 1 .. p, so the earliest row,
// at ctx - rows, reaches back to ctx - rows - window + 1.
__device__ __forceinline__ int window_first(int ctx, int rows, int window) {
    return window > 0 ? max(0, ctx - rows + 1 - window) : 0;
}

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// A read-only value at a wave-uniform address, loaded through the scalar cache
// (s_load) rather than as a vector load: the compiler cannot prove that kernel
// arguments such as a block table stay unwritten, so a plain load becomes a
// vector load and its wait would also wait for every vector memory operation in
// flight (the LDS copies of a prefetch ring). The data must not change during the
// kernel; the scalar cache is invalidated at every launch.
template <class T> __device__ __forceinline__ T load_uniform(const T* ptr) {
    return *reinterpret_cast<const __attribute__((address_space(4))) T*>(reinterpret_cast<uintptr_t>(ptr));
}

// A 16-byte chunk of q with the scale's sign folded in: every word becomes
// (word & q_and) ^ q_xor, which zeroes q for a zero scale (every score is then
// exactly 0) or flips its sign bits for a negative one (q.k negated exactly), so
// the kernels always multiply scores by a positive factor.
__device__ __forceinline__ uint4 q_fold(uint4 v, uint32_t q_and, uint32_t q_xor) {
    return make_uint4((v.x & q_and) ^ q_xor, (v.y & q_and) ^ q_xor, (v.z & q_and) ^ q_xor,
                      (v.w & q_and) ^ q_xor);
}

// acc + sum over the chunk of a[i] * b[i], accumulated in fp32.
template <class E> __device__ __forceinline__ float chunk_dot(uint4 a, uint4 b, float acc);

template <> __device__ __forceinline__ float chunk_dot<BF16>(uint4 a, uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                          __builtin_bit_cast(bf16x2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                          __builtin_bit_cast(bf16x2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                          __builtin_bit_cast(bf16x2_t, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                          __builtin_bit_cast(bf16x2_t, b.w), acc, false);
    return acc;
}

template <> __device__ __forceinline__ float chunk_dot<F16>(uint4 a, uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.x), __builtin_bit_cast(f16x2_t, b.x),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.y), __builtin_bit_cast(f16x2_t, b.y),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.z), __builtin_bit_cast(f16x2_t, b.z),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.w), __builtin_bit_cast(f16x2_t, b.w),
                                 acc, false);
    return acc;
}

template <> __device__ __forceinline__ float chunk_dot<F32>(uint4 a, uint4 b, float acc) {
    acc = fmaf(as_f32(a.x), as_f32(b.x), acc);
    acc = fmaf(as_f32(a.y), as_f32(b.y), acc);
    acc = fmaf(as_f32(a.z), as_f32(b.z), acc);
    acc = fmaf(as_f32(a.w), as_f32(b.w), acc);
    return acc;
}

// Number of elements in one 16-byte chunk.
template <class E> struct chunk_elems {
    static constexpr int value = 16 / (int)sizeof(typename E::storage);
};

// Widen the elements of a 16-byte chunk to fp32 (exact for every type).
template <class E> __device__ __forceinline__ void widen(uint4 a, float* o);

template <> __device__ __forceinline__ void widen<BF16>(uint4 a, float* o) {
    // bf16 is the upper half of a binary32 pattern.
    o[0] = as_f32(a.x << 16);
    o[1] = as_f32(a.x & 0xffff0000u);
    o[2] = as_f32(a.y << 16);
    o[3] = as_f32(a.y & 0xffff0000u);
    o[4] = as_f32(a.z << 16);
    o[5] = as_f32(a.z & 0xffff0000u);
    o[6] = as_f32(a.w << 16);
    o[7] = as_f32(a.w & 0xffff0000u);
}

template <> __device__ __forceinline__ void widen<F16>(uint4 a, float* o) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f16x2_t h = __builtin_bit_cast(f16x2_t, w[i]);
        o[2 * i] = (float)h[0];
        o[2 * i + 1] = (float)h[1];
    }
}

template <> __device__ __forceinline__ void widen<F32>(uint4 a, float* o) {
    o[0] = as_f32(a.x);
    o[1] = as_f32(a.y);
    o[2] = as_f32(a.z);
    o[3] = as_f32(a.w);
}

// Store one fp32 value as element type E (round to nearest even).
template <class E> __device__ __forceinline__ typename E::storage narrow(float x);
template <> __device__ __forceinline__ float narrow<F32>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t narrow<BF16>(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <> __device__ __forceinline__ uint16_t narrow<F16>(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---- LDS staging ---------------------------------------------------------------------
//
// global_load_lds_dwordx4 copies 16 bytes per lane from global memory straight
// into LDS (lane l's bytes land at M0 + 16 * l) without passing through VGPRs.
// The copy is issued from inline asm so the compiler's wait-count pass does not
// see an LDS write behind a vector-memory counter: if it did, it would put a
// full vmcnt(0) wait in front of every LDS read, draining a multi-block ring.
// The caller therefore orders the ring by hand:
//   wait_vmcnt<N>()  before reading a slot (copies complete in issue order),
//   lds_reads_done() before a copy overwrites a slot that was just read.
// Both, and the copy itself, clobber "memory", so the compiler keeps every
// ordinary LDS load of the ring between them.

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_char_t*)p;
}

// Asynchronous copy of 16 bytes per lane from `src` to LDS at lds_dst + 16 * lane.
// lds_dst must be wave-uniform.
__device__ __forceinline__ void copy_to_lds16(const void* src, uint32_t lds_dst) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_dst)), "v"(src)
        : "memory", "m0");
}

// The same copy from the wave-uniform base `sbase` plus this lane's 32-bit byte
// offset `voff` (the scalar-base form: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void copy_to_lds16(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint64_t ub = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_dst)), "v"(voff), "s"(ub)
        : "memory", "m0");
}

// The same copy, with the non-temporal hint when `once` (wave-uniform) says that
// no other workgroup of the launch reads these bytes: a K/V stream read exactly
// once gains about 12% of HBM throughput from it on MI355X (measured on paged
// decode with working sets 8 to 16 times the 256 MB Infinity Cache), while data
// that other workgroups read again should stay in the caches.
__device__ __forceinline__ void copy_to_lds16(const void* src, uint32_t lds_dst, bool once) {
    if (once) {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, off nt"
            :
            : "s"(__builtin_amdgcn_readfirstlane(lds_dst)), "v"(src)
            : "memory", "m0");
    } else {
        copy_to_lds16(src, lds_dst);
    }
}

// Asynchronous copy of 4 bytes per lane from `src` to LDS at lds_dst + 4 * lane.
__device__ __forceinline__ void copy_to_lds4(const void* src, uint32_t lds_dst) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_dst)), "v"(src)
        : "memory", "m0");
}

// The 4-byte copy with the non-temporal hint when `once` (as for copy_to_lds16).
__device__ __forceinline__ void copy_to_lds4(const void* src, uint32_t lds_dst, bool once) {
    if (once) {
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dword %1, off nt"
            :
            : "s"(__builtin_amdgcn_readfirstlane(lds_dst)), "v"(src)
            : "memory", "m0");
    } else {
        copy_to_lds4(src, lds_dst);
    }
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Wait until every LDS read issued so far has returned.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// ---- cross-lane exchange ----------------------------------------------------------

// DPP move of a float within a 16-lane row. CTRL: 0xB1 quad [1,0,3,2], 0x4E quad
// [2,3,0,1], 0x141 half-row mirror, 0x140 row mirror, 0x124 / 0x128 row rotate by 4 / 8.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(x), CTRL, 0xF, 0xF, false));
}

// The values of lanes l and l^16 (order unspecified) via v_permlane16_swap.
__device__ __forceinline__ void pair16(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
    a = as_f32(r[0]);
    b = as_f32(r[1]);
}
// The values of lanes l and l^32 (order unspecified) via v_permlane32_swap.
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
    a = as_f32(r[0]);
    b = as_f32(r[1]);
}

// Sum over the N consecutive lanes of an aligned group (N = 4, 8 or 16). Every
// lane of the group ends with the same bits: each step adds two partial sums
// that both lanes of a pair hold, and IEEE addition is commutative.
template <int N> __device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    if constexpr (N >= 8) x += dpp<0x141>(x);
    if constexpr (N >= 16) x += dpp<0x140>(x);
    return x;
}

// Reduce over the lanes that share lane % N (N = 4, 8, 16 or 32): the result in
// each lane covers all 64 / N lanes of its residue class. Every lane of a class
// holds the same bits for MAX, and for sums when N >= 8; for N == 4 the two
// row-rotate steps associate the four row partials differently per lane.
template <int N, bool MAX> __device__ __forceinline__ float stride_reduce(float x) {
    static_assert(N == 4 || N == 8 || N == 16 || N == 32, "stride of 4, 8, 16 or 32 lanes");
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (N == 4) x = op(x, dpp<0x124>(x));   // + lane (l+4) mod 16 within the row
    if constexpr (N <= 8) x = op(x, dpp<0x128>(x));   // + lane (l+8) mod 16 within the row
    float a, b;
    if constexpr (N <= 16) {
        pair16(x, a, b);
        x = op(a, b);
    }
    pair32(x, a, b);
    return op(a, b);
}

// ---- reduce-scatter across lane bits ---------------------------------------------------
//
// Sum N values per lane over the lanes that differ in lane bits [LO, 6), leaving
// each lane with N / 2^(6-LO) fully reduced values. Bits are reduced from bit 5
// down; at each step a lane keeps the half of its values selected by its own
// lane bit and adds its partner's copy of that half. Afterwards lane l holds
// values j*M .. j*M + M - 1 (M = N / 2^(6-LO)), where j = l >> LO.
//
//   bit 5: v_permlane32_swap(x[k], x[k+H]) gives both halves in one exchange.
//   bit 4: v_permlane16_swap, the same within each 32-lane half.
//   bit 3: DPP row_ror:8 reads lane l^8 inside its 16-lane row.
//   bit 2: ds_bpermute (lane l^4).
template <int N, int BIT> __device__ __forceinline__ void rs_step(const float (&x)[N], float (&y)[N / 2],
                                                                  int lane) {
    constexpr int H = N / 2;
    if constexpr (BIT == 5 || BIT == 4) {
#pragma unroll
        for (int k = 0; k < H; ++k) {
            auto r = BIT == 5 ? __builtin_amdgcn_permlane32_swap(as_u32(x[k]), as_u32(x[k + H]), false, false)
                              : __builtin_amdgcn_permlane16_swap(as_u32(x[k]), as_u32(x[k + H]), false, false);
            y[k] = as_f32(r[0]) + as_f32(r[1]);
        }
    } else {
        const bool hi = (lane >> BIT) & 1;
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const float keep = hi ? x[k + H] : x[k];
            const float send = hi ? x[k] : x[k + H];
            float other;
            if constexpr (BIT == 3)
                other = dpp<0x128>(send);
            else
                other = __shfl_xor(send, 1 << BIT);
            y[k] = keep + other;
        }
    }
}

template <int N, int LO> struct ReduceScatter {
    static constexpr int M = N >> (6 - LO);
    static __device__ __forceinline__ void run(const float (&x)[N], float (&out)[M], int lane) {
        if constexpr (LO == 6) {
#pragma unroll
            for (int k = 0; k < N; ++k) out[k] = x[k];
        } else {
            float y5[N / 2];
            rs_step<N, 5>(x, y5, lane);
            if constexpr (LO == 5) {
#pragma unroll
                for (int k = 0; k < M; ++k) out[k] = y5[k];
            } else {
                float y4[N / 4];
                rs_step<N / 2, 4>(y5, y4, lane);
                if constexpr (LO == 4) {
#pragma unroll
                    for (int k = 0; k < M; ++k) out[k] = y4[k];
                } else {
                    float y3[N / 8];
                    rs_step<N / 4, 3>(y4, y3, lane);
                    if constexpr (LO == 3) {
#pragma unroll
                        for (int k = 0; k < M; ++k) out[k] = y3[k];
                    } else {
                        static_assert(LO == 2, "reduce over lane bits 2..5 at most");
                        rs_step<N / 8, 2>(y3, out, lane);
                    }
                }
            }
        }
    }
};

}  // namespace pa
