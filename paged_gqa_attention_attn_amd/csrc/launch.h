// launch.h -- internal interface between the C-ABI host layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class Elem { F32 = 0, BF16 = 1, F16 = 2 };
// One-byte cache formats (codes plus one fp32 scale per token row).
enum class QuantFmt { FP8_E4M3 = 3, INT8 = 4 };

// Everything a decode launch needs; filled by the host plan in api.hip.
struct DecodeArgs {
    const void* q;               // [B][n_q][D]
    const void* k_cache;         // [num_blocks][n_kv][16][D]
    const void* v_cache;
    const int32_t* block_table;  // [B][max_blocks]
    const int32_t* context_lens; // [B]
    void* out;                   // [B][n_q][D]
    float* ws_m;                 // [B][n_q][nparts_max]      partition running max (log2 units)
    float* ws_l;                 // [B][n_q][nparts_max]      partition softmax denominator
    float* ws_acc;               // [B][n_q][nparts_max][D]   partition numerator
    int32_t batch, n_q, n_kv, num_blocks, max_blocks;
    int32_t group;               // G = n_q / n_kv
    int32_t gw;                  // query heads per wave (template parameter of the kernel)
    int32_t hs_wg;               // head slices (of gw heads) per workgroup
    int32_t hsg;                 // head-slice groups per KV head (grid.y = n_kv * hsg)
    int32_t waves_tok;           // waves that split the partition's blocks
    int32_t blocks_per_wave;     // 16-token blocks one wave takes per partition
    int32_t nparts_max;          // grid.x
    int32_t ring;                // blocks in flight per wave (LDS ring depth: 1 or 2)
    float scale_log2;            // |scale| * log2(e) (log2(e) when scale is 0)
    // Every 32-bit word of q is taken as (word & q_and) ^ q_xor when it is loaded:
    // all ones and 0 for a positive scale, 0 and 0 for scale 0 (every score is then
    // exactly 0), the sign bits for a negative scale (q k negated exactly).
    uint32_t q_and, q_xor;
    int32_t out_f32;             // 1: fp32 output, 0: output in the input type
    // Fused append (all null for a plain decode): new token of each sequence.
    const void* k_new;           // [B][n_kv][D]
    const void* v_new;
    const int64_t* new_slots;    // [B]
    void* k_cache_w;             // writable views of the pools for the append
    void* v_cache_w;
    // Multi-row decode: q_rows new query rows per sequence ([B][q_rows][n_q][D]),
    // served in groups of 32 (query head, row) pairs per KV head (grid.y = n_kv * row_groups).
    int32_t q_rows;
    int32_t row_groups;
    // Sliding window: 0 attends to the whole context; W > 0 lets the query at
    // position p see positions max(0, p - W + 1) .. p only.
    int32_t window;
    // ALiBi: slope m_h per query head [n_q] (nullptr: none); the score of key
    // position j for the query at position i gets -m_h (i - j).
    const float* alibi;
    // Single-row decode on the matrix cores (decode_mfma.hip): gw query heads
    // (4, 8 or 16) per workgroup fill the MFMA columns; hs_wg must be 1.
    int32_t mfma;
    // Quantised cache (decode_quant.hip): per-row scales [num_blocks][n_kv][16], and
    // their writable views for a fused quantising append (k_new / v_new then hold
    // the new rows in q's type, quantised as pa_kv_append_quant does). With
    // chan_scales set, k_scale / v_scale are fixed channel scales [n_kv][D] instead
    // and the append writes codes only.
    const float* k_scale;
    const float* v_scale;
    float* k_scale_w;
    float* v_scale_w;
    int32_t chan_scales;
};

hipError_t launch_decode(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s);
// Single-row decode with the per-block products on the matrix cores (bf16/f16).
hipError_t launch_decode_mfma(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s);
// The log-sum-exp merge of partition partials alone (rows = batch * n_q of `a`).
hipError_t launch_decode_reduce(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s);
// Multi-row decode on the matrix cores (bf16/f16), plus the merge when contexts split.
hipError_t launch_decode_multi(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s);

// Decode over a quantised cache (codes + per-row scales), q in q_type (bf16 or f16).
hipError_t launch_decode_quant(const DecodeArgs& a, Elem q_type, QuantFmt fmt, int head_dim, hipStream_t s);
// LDS bytes one wave of the quantised decode kernel takes for hw heads and a ring of `ring` blocks.
int quant_wave_bytes(int head_dim, int hw, int ring);
// Quantise k/v rows ([T][n_kv][D] in src) into codes at slot_mapping: per row (scales
// written to k_scale / v_scale [slots]) or, per_channel, with the fixed channel scales
// k_scale / v_scale [n_kv][D] (read only).
hipError_t launch_kv_append_quant(const void* k, const void* v, Elem src, QuantFmt fmt, bool per_channel,
                                  const int64_t* slots, int32_t num_tokens, int32_t n_kv, int32_t head_dim,
                                  int64_t num_slots, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                                  hipStream_t s);

hipError_t launch_kv_append(const void* k, const void* v, const int64_t* slots, int32_t num_tokens,
                            int32_t n_kv, int32_t row_bytes, int32_t block_size,
                            int64_t num_slots, void* k_cache, void* v_cache, hipStream_t s);

struct PrefillArgs {
    const void* q;  // [B][S][n_q][D]: S = seq_len query rows per sequence
    const void* k;  // contiguous: [B][S][n_kv][D]; paged: the K pool [num_blocks][n_kv][16][D]
    const void* v;
    void* out;      // [B][S][n_q][D]
    int32_t batch, seq_len, n_q, n_kv;
    int32_t group;
    int32_t causal;
    float scale_log2;             // as for DecodeArgs, with q_and / q_xor applied to q
    uint32_t q_and, q_xor;
    int32_t out_f32;
    // Paged keys (block_table != nullptr): sequence b has context_lens[b] keys in the
    // pools and its S query rows are its last S positions.
    const int32_t* block_table;   // [B][max_blocks]
    const int32_t* context_lens;  // [B]
    int32_t max_blocks, num_blocks;
    int32_t window;   // sliding window (causal only); 0: none
    const float* alibi;   // ALiBi slopes [n_q] (causal only); nullptr: none
    int resident_wgs;     // prefill workgroups the GPU holds at once (set by the launcher)
    int hpw;              // query heads per workgroup (set by the launcher)
    // Contiguous bf16 keys only: an f16 copy of v in v's layout, written by the
    // staging kernel, and one byte per (sequence, KV head, 64-key tile) that is 1
    // where the copy is exact. nullptr: P V stays in bf16 (hi + lo parts).
    void* v16;
    uint8_t* v16_ok;
};

// Prefill work items: a workgroup of 8 waves takes the query heads of one KV group
// that share its K/V tiles, HPW of them (4, 2 or 1: the largest dividing the group
// size), and 256 / HPW query rows of each (32 per wave). One launch has
// ceil(rows / (256 / HPW)) * (n_q / HPW) * batch workgroups in a one-dimensional grid,
// so that count must fit in an int; rows stay 256 below INT32_MAX so that the
// kernels' tile counts cannot overflow.
constexpr int PREFILL_WAVES = 8;
constexpr int PREFILL_PAIRS_PER_WG = 32 * PREFILL_WAVES;   // (head, row) pairs
inline int prefill_heads_per_wg(int group) { return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1; }
inline bool prefill_grid_fits(int rows, int n_q, int batch, int group) {
    const int hpw = prefill_heads_per_wg(group);
    const int64_t rw = PREFILL_PAIRS_PER_WG / hpw;
    return rows <= INT32_MAX - PREFILL_PAIRS_PER_WG &&
           ((int64_t)rows + rw - 1) / rw * (n_q / hpw) * batch <= INT32_MAX;
}

hipError_t launch_prefill(const PrefillArgs& a, Elem e, int head_dim, hipStream_t s);
// fp32 attention of seq_len query rows per sequence (contiguous prefill, or paged
// chunked prefill / multi-row decode when block_table is set) on the fp32 matrix
// cores; hipErrorNotSupported past its grid limits (ceil(seq_len * group / 64)
// workgroups per KV head and sequence at most 2^31 - 1, n_kv and batch at most 65535).
hipError_t launch_attn_f32(const PrefillArgs& a, int head_dim, hipStream_t s);

// Compute units of the current device, queried once per device; 256 (MI355X)
// when no device can be queried.
int device_cus();

}  // namespace pa
