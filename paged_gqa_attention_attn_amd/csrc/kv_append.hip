// kv_append.hip -- slot-mapped write of new K/V rows into the paged cache (gfx950).
//
// Token t's K and V rows for every KV head go to flat slot slot_mapping[t] =
// physical_block * block_size + offset (vLLM concepts page, yyzxw.github.io:
// attention backends receive a slot mapping giving each token's physical
// location; "LLM 推理全过程的维度变化与核心公式", research.frankk.site, decode
// step: write the new K/V at position cache_len, prefill: write positions
// 0..S-1). The copy moves 16-byte chunks, so the cache holds the input bits
// exactly. Negative slots (padding) and slots past the pool are skipped.
#include "common.h"
#include "launch.h"
#include "quant.h"

namespace pa {

namespace {

// One thread per 16-byte chunk of a (token, KV head) row; consecutive threads
// cover consecutive chunks of a row, so both the reads of k/v and the writes
// into the (block, head, offset) row are contiguous 16-byte accesses.
__global__ __launch_bounds__(256) void kv_append_kernel(const uint4* __restrict__ k,
                                                        const uint4* __restrict__ v,
                                                        const int64_t* __restrict__ slots,
                                                        int64_t total_chunks, int32_t n_kv,
                                                        int32_t chunks_per_row, int32_t block_size,
                                                        int64_t num_slots, uint4* __restrict__ kc,
                                                        uint4* __restrict__ vc) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total_chunks;
         idx += stride) {
        const int64_t ch = idx % chunks_per_row;
        const int64_t r = idx / chunks_per_row;     // (token, head) row
        const int64_t g = r % n_kv;
        const int64_t t = r / n_kv;
        const int64_t slot = slots[t];
        if (slot < 0 || slot >= num_slots) continue;
        const int64_t blk = slot / block_size;
        const int64_t off = slot % block_size;
        const int64_t dst = ((blk * n_kv + g) * block_size + off) * chunks_per_row + ch;
        kc[dst] = k[idx];
        vc[dst] = v[idx];
    }
}

}  // namespace

hipError_t launch_kv_append(const void* k, const void* v, const int64_t* slots, int32_t num_tokens,
                            int32_t n_kv, int32_t row_bytes, int32_t block_size, int64_t num_slots,
                            void* k_cache, void* v_cache, hipStream_t s) {
    const int32_t chunks = row_bytes / 16;
    const int64_t total = (int64_t)num_tokens * n_kv * chunks;
    if (total == 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const int blocks = (int)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots, total,
                       n_kv, chunks, block_size, num_slots, static_cast<uint4*>(k_cache),
                       static_cast<uint4*>(v_cache));
    return hipGetLastError();
}


// ---- quantised cache: one-byte codes, and one fp32 scale per (token, KV head) row or fixed
// per-channel scales (the quantisation itself is in quant.h)

namespace {

// One wave per (token, KV head, K or V) row: lane l holds elements EPL l .. EPL l + EPL - 1.
// Per row (PC false): the row's scale goes to ks / vs [slots]. Per channel (PC true):
// ks / vs are the fixed channel scales [n_kv][D], read only.
template <class SRC, bool FP8, int D, bool PC>
__global__ __launch_bounds__(256) void kv_append_quant_kernel(const void* k, const void* v,
                                                              const int64_t* __restrict__ slots,
                                                              int64_t rows, int32_t n_kv, int64_t num_slots,
                                                              uint8_t* kc, uint8_t* vc, float* ks, float* vs) {
    constexpr int EPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (r >= rows) return;   // uniform over the wave
    const bool is_v = r & 1;
    const int64_t tg = r >> 1;   // token * n_kv + head
    const int64_t t = tg / n_kv;
    const int64_t g = tg % n_kv;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;   // padding or past the pool: skipped

    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = load_f32<SRC>(is_v ? v : k, tg * D + lane * EPL + i);
    uint32_t codes = 0;
    float scale = 0.f;
    if constexpr (PC) {
        const float* cs = (is_v ? vs : ks) + g * D + lane * EPL;
#pragma unroll
        for (int i = 0; i < EPL; ++i) codes |= channel_code<FP8>(x[i], cs[i]) << (8 * i);
    } else {
        scale = quantize_row<FP8, EPL>(x, codes);
    }
    const int64_t row = ((slot / 16) * n_kv + g) * 16 + slot % 16;
    uint8_t* dst = (is_v ? vc : kc) + row * D + lane * EPL;
    if constexpr (EPL == 2)
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)codes;
    else
        *dst = (uint8_t)codes;
    if (!PC && lane == 0) (is_v ? vs : ks)[row] = scale;
}

template <class SRC, bool FP8, bool PC>
hipError_t launch_quant_typed(const void* k, const void* v, const int64_t* slots, int64_t rows, int32_t n_kv,
                              int32_t head_dim, int64_t num_slots, void* kc, void* vc, float* ks, float* vs,
                              hipStream_t s) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (head_dim == 128)
        hipLaunchKernelGGL((kv_append_quant_kernel<SRC, FP8, 128, PC>), grid, dim3(256), 0, s, k, v, slots, rows,
                           n_kv, num_slots, static_cast<uint8_t*>(kc), static_cast<uint8_t*>(vc), ks, vs);
    else if (head_dim == 64)
        hipLaunchKernelGGL((kv_append_quant_kernel<SRC, FP8, 64, PC>), grid, dim3(256), 0, s, k, v, slots, rows,
                           n_kv, num_slots, static_cast<uint8_t*>(kc), static_cast<uint8_t*>(vc), ks, vs);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <class SRC>
hipError_t launch_quant_src(bool fp8, bool pc, const void* k, const void* v, const int64_t* slots, int64_t rows,
                            int32_t n_kv, int32_t head_dim, int64_t num_slots, void* kc, void* vc, float* ks,
                            float* vs, hipStream_t s) {
    if (pc)
        return fp8 ? launch_quant_typed<SRC, true, true>(k, v, slots, rows, n_kv, head_dim, num_slots, kc, vc, ks, vs, s)
                   : launch_quant_typed<SRC, false, true>(k, v, slots, rows, n_kv, head_dim, num_slots, kc, vc, ks, vs, s);
    return fp8 ? launch_quant_typed<SRC, true, false>(k, v, slots, rows, n_kv, head_dim, num_slots, kc, vc, ks, vs, s)
               : launch_quant_typed<SRC, false, false>(k, v, slots, rows, n_kv, head_dim, num_slots, kc, vc, ks, vs, s);
}

}  // namespace

hipError_t launch_kv_append_quant(const void* k, const void* v, Elem src, QuantFmt fmt, bool per_channel,
                                  const int64_t* slots, int32_t num_tokens, int32_t n_kv, int32_t head_dim,
                                  int64_t num_slots, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                                  hipStream_t s) {
    const int64_t rows = (int64_t)num_tokens * n_kv * 2;
    if (rows == 0) return hipSuccess;
    const bool fp8 = fmt == QuantFmt::FP8_E4M3;
    const bool pc = per_channel;
    switch (src) {
    case Elem::F32:
        return launch_quant_src<F32>(fp8, pc, k, v, slots, rows, n_kv, head_dim, num_slots, k_cache, v_cache, k_scale, v_scale, s);
    case Elem::BF16:
        return launch_quant_src<BF16>(fp8, pc, k, v, slots, rows, n_kv, head_dim, num_slots, k_cache, v_cache, k_scale, v_scale, s);
    case Elem::F16:
        return launch_quant_src<F16>(fp8, pc, k, v, slots, rows, n_kv, head_dim, num_slots, k_cache, v_cache, k_scale, v_scale, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
