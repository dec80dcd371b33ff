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

}  // namespace pa
