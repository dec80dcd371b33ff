/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged GQA attention library.
 *
 * Scaled dot-product attention softmax(q K^T * scale + M) V over a key/value
 * cache that is stored in fixed-size blocks reached through a block table.
 *
 * Sources (web pages):
 *  [AE] "注意力演进与推理流程", jerryiiii.gitbook.io/llm-review/notes/attention/
 *       attention-evolution-and-inference: section 1.1 (attention formula and
 *       causal mask), section 3.1 (GQA: query head h reads KV group floor(h/G)),
 *       "变革 1" (PagedAttention: fixed blocks such as 16 tokens).
 *  [PD] xinc.fun/index.php/archives/233: section 2 (shapes, causal mask),
 *       section 3 (KV cache append), section 6 (block table over scattered blocks).
 *  [VC] yyzxw.github.io/acknowledge/research/vllm-concepts-deep-dive/section-1.html:
 *       decode attention over K<=t, V<=t; attention kernels take a block table and
 *       a slot mapping instead of contiguous pointers.
 *  [IW] "LLM 推理全过程的维度变化与核心公式", research.frankk.site/notes/
 *       llm-inference-walkthrough: "Decode 阶段维度流转" (append at cache_len, then
 *       read the whole cache; no mask in decode), "Prefill 阶段维度流转",
 *       "KV Cache 的形状与增长" (16-token blocks; sliding window bounding the
 *       cache at W recent positions), "工程优化怎么嵌进公式"
 *       (Flash Attention online softmax; Flash Decoding split + log-sum-exp).
 *
 * Conventions for every entry point
 *  - All data pointers are device pointers owned by the caller (for example
 *    torch allocations). The library keeps no reference after the call returns.
 *  - Every call only enqueues work on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream) and returns before the GPU finishes.
 *  - Data pointers must be 16-byte aligned; rows are contiguous in the stated
 *    layouts. Element offsets are computed in 64-bit arithmetic.
 *  - Return value: PA_OK (0) or a negative pa_status. On failure nothing was
 *    enqueued and pa_last_error() describes the problem.
 *  - Device-resident metadata (block ids, slots, context lengths) is not read
 *    by the host. Kernels bounds-check it: an out-of-range slot is skipped; a
 *    sequence whose context length exceeds max_blocks_per_seq * block_size or
 *    whose block table names a block outside the pool, among the blocks the
 *    call reads, gets a NaN output row instead of an out-of-bounds read.
 *  - Debug mode: with option PA_OPT_VALIDATE on (pa_set_option), kv_append, the decode
 *    calls (single- and multi-row) and chunked prefill also copy that metadata to the host (synchronising `stream`)
 *    and return PA_ERR_INVALID_ARG, enqueuing nothing, for: a slot past the
 *    pool or repeated within one call; a context length outside
 *    [0, max_blocks_per_seq * block_size]; a block id outside the pool among the
 *    table entries the call reads (a sequence's first ceil(ctx / block_size),
 *    less those wholly before a sliding window); and, for
 *    decode_append, a slot other than position ctx - 1 of its own sequence or in
 *    a block another sequence of the call also reads.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. q/k/v and the cache share one type; outputs are f32 or that type.
 * PA_FP8_E4M3 and PA_INT8 describe quantised caches only (one-byte codes plus one
 * fp32 scale per token row, see pa_kv_append_quant); the _PER_CHANNEL forms hold the
 * same codes with one fixed fp32 scale per (KV head, channel) instead. Only the
 * quantised entry points (pa_kv_append_quant, pa_paged_attn_*_quant*) take them;
 * every other entry point rejects them with PA_ERR_UNSUPPORTED. */
typedef enum {
    PA_F32 = 0,
    PA_BF16 = 1,
    PA_F16 = 2,
    PA_FP8_E4M3 = 3,
    PA_INT8 = 4,
    PA_FP8_E4M3_PER_CHANNEL = 5,
    PA_INT8_PER_CHANNEL = 6
} pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, n_q % n_kv != 0 */
    PA_ERR_UNSUPPORTED = -2, /* dtype / head_dim / block_size without a kernel        */
    PA_ERR_HIP = -3          /* a HIP runtime call or launch failed                    */
} pa_status;

/*
 * Paged cache description. Each of the two pools (K and V) is
 *   [num_blocks][n_kv][block_size][head_dim], head_dim fastest,
 * so element (block, kv_head, offset, c) sits at
 *   ((block * n_kv + kv_head) * block_size + offset) * head_dim + c.
 * Supported: block_size 16; head_dim 64 or 128; dtype f32, bf16 or f16 (and,
 * for the quantised entry points, PA_FP8_E4M3 or PA_INT8 or their _PER_CHANNEL
 * forms, one byte per element).
 */
typedef struct {
    int32_t num_blocks;
    int32_t block_size;
    int32_t n_kv;
    int32_t head_dim;
    pa_dtype dtype;
} pa_cache_desc;

/*
 * kv_append -- write new K/V rows into the paged cache through slot_mapping.
 * [VC] (slot mapping given to attention kernels); [IW] decode step: write the
 * new K/V at position cache_len; prefill: write positions 0..S-1; [PD] section 3.
 *
 *   k, v          [num_tokens][n_kv][head_dim] in cache->dtype
 *   slot_mapping  int64 [num_tokens]; token t goes to block slot / block_size,
 *                 offset slot % block_size. slot < 0 marks a padding token
 *                 (skipped); slot >= num_blocks * block_size is skipped too.
 *   k_cache, v_cache  the pools described by `cache`, updated in place.
 * The write is a bit-exact copy. Two tokens with the same slot race (which one
 * lands is unspecified). num_tokens == 0 is a no-op.
 */
int pa_kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                 void* k_cache, void* v_cache, const pa_cache_desc* cache, void* stream);

/*
 * Bytes of scratch memory pa_paged_attn_decode (or, for a quantised cache
 * description, pa_paged_attn_decode_quant) needs for these arguments
 * (partial results of a context split into partitions, [VC]/[IW] Flash Decoding).
 * 0 when every sequence fits in one partition. Returns 0 as well for invalid
 * arguments; the decode call then reports the error. The size covers any
 * window; a windowed call may need less.
 */
size_t pa_decode_workspace_bytes(int32_t batch, int32_t n_q, int32_t max_blocks_per_seq,
                                 const pa_cache_desc* cache);

/*
 * paged_attn_decode -- one query token per sequence attends to its cached
 * context through the block table. [VC] decode attention over K<=t, V<=t;
 * [AE] 3.1 GQA grouping; [IW] "Decode 阶段维度流转" (no causal mask in decode),
 * Flash Attention's running max/sum and Flash Decoding's split + log-sum-exp.
 *
 *   q             [batch][n_q][head_dim] in cache->dtype
 *   k_cache, v_cache  pools described by `cache`
 *   block_table   int32 [batch][max_blocks_per_seq]; entry j = physical block of
 *                 the sequence's logical block j (positions 16j .. 16j+15)
 *   context_lens  int32 [batch]: number of positions attended, counting the
 *                 token appended in the same step (positions 0..ctx-1)
 *   scale         multiplies q.k (usually 1/sqrt(head_dim)); any finite value. 0
 *                 makes every score exactly 0 (with finite q and K), so a row is the
 *                 mean of the V rows it attends to (plus the ALiBi bias, if any); a
 *                 negative scale negates q.k exactly. Not finite: PA_ERR_INVALID_ARG.
 *   window        sliding window ([IW] "KV Cache 的形状与增长", sliding-window item):
 *                 0 attends to all ctx positions; W > 0 to the last W of them,
 *                 positions max(0, ctx - W) .. ctx - 1. Block-table entries of
 *                 blocks wholly before that range are never read, so an engine
 *                 may recycle them. Negative: PA_ERR_INVALID_ARG.
 *   alibi_slopes  NULL, or device fp32 [n_q], 4-byte aligned: ALiBi's slope m_h of
 *                 each query head ([IW] position-encoding section: scores_ij =
 *                 q_i.k_j / sqrt(d) - m_h (i - j)); the score of position t gets
 *                 -m_h (ctx - 1 - t), the query being the newest position ctx - 1.
 *   out           [batch][n_q][head_dim], out_dtype PA_F32 or cache->dtype
 *   workspace     device scratch of at least pa_decode_workspace_bytes(...)
 *                 bytes for the same arguments, or NULL: then the workspace
 *                 given to pa_set_workspace if it is large enough, else one the
 *                 library allocates on the current device at the first call
 *                 that needs it. When a later call needs more, the library
 *                 allocates a buffer at least twice as large and keeps the old
 *                 one too (a call on another thread, or kernels still running,
 *                 may use it), so every library buffer lives until the process
 *                 ends; that call is then not capturable in a HIP graph.
 * Query head h reads KV head h / (n_q / n_kv). ctx == 0 gives a zero row.
 * Results depend only on logical positions, so relabelling physical blocks
 * leaves every output bit unchanged. Calls that share a workspace (the library's
 * own included) must not overlap on the GPU: concurrent streams pass their own.
 * Calls from several host threads on one stream may share the library's own or
 * the pa_set_workspace buffer: each call enqueues all its kernels while holding
 * the library's workspace lock, so their kernels do not interleave.
 */
int pa_paged_attn_decode(const void* q, int32_t batch, int32_t n_q, const void* k_cache,
                         const void* v_cache, const pa_cache_desc* cache,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, float scale, int32_t window,
                         const float* alibi_slopes, void* out,
                         pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_noalloc -- pa_paged_attn_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc. Same arguments, kernels and results (bit for
 * bit) as pa_paged_attn_decode, without the workspace arguments: when contexts
 * are split into partitions, the partial results go to a fixed device array of
 * PA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, that each GPU
 * holds from the library's first use there until the process ends. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   Returns PA_ERR_INVALID_ARG, enqueuing nothing, when the partials would exceed
 * that size (pa_decode_workspace_bytes gives the need for the same arguments).
 * Every call on one GPU shares that GPU's array: calls that overlap on the GPU
 * (on different streams) race and their results are unspecified. Calls from
 * several host threads on one stream are safe: each enqueues its kernels while
 * holding the array's lock. The array keeps whatever the last call left; no part
 * of it needs to start at zero (a merge reads only what its own call wrote).
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_paged_attn_decode_noalloc(const void* q, int32_t batch, int32_t n_q, const void* k_cache,
                                 const void* v_cache, const pa_cache_desc* cache,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, float scale, int32_t window,
                                 const float* alibi_slopes, void* out, pa_dtype out_dtype, void* stream);

/*
 * paged_attn_decode_append -- one decode step in a single launch: kv_append of
 * one new token per sequence followed by paged_attn_decode. [IW] "Decode 阶段维度
 * 流转": write the new K/V at position cache_len, increment it, then attend over
 * the whole cache.
 *
 *   k_new, v_new  [batch][n_kv][head_dim] in cache->dtype: the new token of each sequence
 *   slot_mapping  int64 [batch]: its slot (negative: sequence b appends nothing)
 *   other arguments as for pa_paged_attn_decode; workspace size as reported by
 *   pa_decode_workspace_bytes for the same arguments.
 * The new token must sit at position context_lens[b] - 1, i.e. slot_mapping[b]
 * must be the slot that sequence b's block table gives that position, and no
 * other sequence may attend to that slot in the same call (the engine's
 * copy-on-write rule for shared blocks). The attention then uses k_new/v_new at
 * that position and every output bit equals the two-call sequence
 * pa_kv_append + pa_paged_attn_decode. Otherwise the cache write still lands at
 * slot_mapping[b] (or is skipped if out of range) but the attention result is
 * unspecified; no access goes out of bounds.
 */
int pa_paged_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, int32_t batch, int32_t n_q,
                                void* k_cache, void* v_cache, const pa_cache_desc* cache,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, float scale, int32_t window,
                                const float* alibi_slopes,
                                void* out, pa_dtype out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * paged_attn_prefill -- attention of a whole prompt over itself.
 * [AE] 1.1 / [PD] section 2: A = softmax(Q K^T / sqrt(d) + M), O = A V with the
 * causal mask M_ij = 0 for j <= i and -inf otherwise; [AE] 3.1 GQA grouping;
 * [IW] "Prefill 阶段维度流转".
 *
 *   q     [batch][seq_len][n_q][head_dim]   in dtype (f32, bf16 or f16)
 *   k, v  [batch][seq_len][n_kv][head_dim]  in dtype
 *   causal  1: row i attends to keys 0..i; 0: to all seq_len keys
 *   scale   multiplies q.k (usually 1/sqrt(head_dim)); any finite value, as
 *           for pa_paged_attn_decode
 *   window  0: no window; W > 0 (causal only) narrows row i to keys
 *           max(0, i - W + 1) .. i ([IW] sliding-window item). Negative, or
 *           positive with causal == 0: PA_ERR_INVALID_ARG.
 *   alibi_slopes  NULL, or device fp32 [n_q] (causal only): row i's score for
 *           key j gets -m_h (i - j) (as for pa_paged_attn_decode); with
 *           causal == 0: PA_ERR_INVALID_ARG.
 *   out   [batch][seq_len][n_q][head_dim], out_dtype PA_F32 or dtype
 *   workspace  device scratch of at least pa_prefill_workspace_bytes(...) bytes
 *         (16-byte aligned), or NULL: then the workspace of pa_set_workspace if
 *         large enough, else the library's own (as for pa_paged_attn_decode).
 *         bf16 only: it receives an f16 copy of v, exact for every finite value
 *         below 65520 in magnitude (f16 keeps 11 significant bits to bf16's 8;
 *         values below 2^-14 move by at most 2^-25), so that P V runs with one
 *         11-bit P part on the f16 matrix cores; 64-key tiles holding a larger
 *         finite value keep the bf16 product for the rows that read them.
 *         Option PA_OPT_PREFILL_STAGE_V = 0 turns the staging off.
 *         Calls that share a workspace must not overlap on the GPU.
 * Supported: head_dim 128 (and 64); dtype f32, bf16 or f16. bf16/f16: seq_len
 * at most 2^31 - 257 and the workgroup count, ceil(seq_len / (256 / H)) *
 * (n_q / H) * batch with H = 4, 2 or 1 query heads per workgroup (the largest
 * dividing n_q / n_kv), at most 2^31 - 1. f32 (fp32 matrix-core kernel, one
 * workgroup per 64 (row, head) pairs of a KV head, no workspace): seq_len *
 * n_q / n_kv at most 2^31 - 65, n_kv and batch at most 65535. Otherwise
 * PA_ERR_UNSUPPORTED.
 */
size_t pa_prefill_workspace_bytes(pa_dtype dtype, int32_t batch, int32_t seq_len, int32_t n_kv,
                                  int32_t head_dim);
int pa_paged_attn_prefill(const void* q, const void* k, const void* v, pa_dtype dtype,
                          int32_t batch, int32_t seq_len, int32_t n_q, int32_t n_kv,
                          int32_t head_dim, int32_t causal, float scale, int32_t window,
                          const float* alibi_slopes,
                          void* out, pa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * paged_attn_decode_multi -- q_rows new query rows per sequence (speculative
 * verification of drafted tokens) attend to the paged cache in one step. Row r
 * of sequence b sits at position context_lens[b] - q_rows + r and attends to
 * positions 0 .. that position: [AE] 1.1 causal mask, 3.1 GQA grouping; [VC]
 * block table; [IW] "工程优化怎么嵌进公式" (verifying several drafted tokens at
 * once turns decode's vector products into small matrix products).
 *
 *   q             [batch][q_rows][n_q][head_dim] in cache->dtype (f32, bf16 or f16)
 *   k_cache, v_cache  pools described by `cache`, already holding the rows' own
 *                 K/V (pa_kv_append of the q_rows new tokens first)
 *   block_table, context_lens, scale  as for pa_paged_attn_decode
 *   alibi_slopes  NULL, or device fp32 [n_q]: the row at position p scores key
 *                 position j with -m_h (p - j) added (as for pa_paged_attn_decode)
 *   window        0: none; W > 0: the row at position p attends to positions
 *                 max(0, p - W + 1) .. p only ([IW] sliding-window item); entries
 *                 of blocks wholly before the first row's window are never read
 *   out           [batch][q_rows][n_q][head_dim], out_dtype PA_F32 or cache->dtype
 *   workspace     as for pa_paged_attn_decode, sized by pa_decode_multi_workspace_bytes
 * The (query head, row) pairs of one KV head are the N side of matrix-core
 * products, so each K/V byte is read once per step. Rows at negative positions
 * (context_lens[b] < q_rows) are zero; a context past the block table's reach or
 * an out-of-pool block id among those read gives NaN rows. Results equal
 * pa_paged_attn_chunked_prefill with chunk_len = q_rows up to rounding (bit for
 * bit for f32 caches, which both calls serve with the same fp32 kernel and no
 * workspace). The workspace size covers any window; given a quantised cache
 * description it sizes pa_paged_attn_decode_multi_quant and
 * pa_paged_attn_chunked_prefill_quant (rows = q_rows) instead. Supported:
 * head_dim 64 or 128; f32 within the limits given for pa_paged_attn_prefill.
 */
size_t pa_decode_multi_workspace_bytes(int32_t batch, int32_t q_rows, int32_t n_q,
                                       int32_t max_blocks_per_seq, const pa_cache_desc* cache);
int pa_paged_attn_decode_multi(const void* q, int32_t batch, int32_t q_rows, int32_t n_q,
                               const void* k_cache, const void* v_cache, const pa_cache_desc* cache,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, float scale, int32_t window,
                               const float* alibi_slopes, void* out,
                               pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_chunked_prefill -- a chunk of a prompt attends to the cached prefix
 * and causally to itself, all keys read through the block table. [IW]
 * "工程优化怎么嵌进公式" (chunked prefill: the prompt goes in pieces, the formula
 * is unchanged) and "Prefill 阶段维度流转"; [VC] (kernels take a block table);
 * [AE] 1.1 causal mask, 3.1 GQA grouping.
 *
 *   q             [batch][chunk_len][n_q][head_dim] in cache->dtype (f32, bf16 or f16)
 *   k_cache, v_cache  pools described by `cache`, already holding the chunk's own
 *                 K/V (pa_kv_append first)
 *   block_table   int32 [batch][max_blocks_per_seq]
 *   context_lens  int32 [batch]: keys of sequence b, prefix plus chunk; query row i
 *                 sits at position context_lens[b] - chunk_len + i and attends to
 *                 positions 0 .. that position (causal mask aligned at the bottom
 *                 right; chunk_len == context_lens[b] is a plain causal prefill)
 *   scale         multiplies q.k; any finite value, as for pa_paged_attn_decode
 *   alibi_slopes  NULL, or device fp32 [n_q]: the row at position p scores key
 *                 position j with -m_h (p - j) added (as for pa_paged_attn_decode)
 *   window        0: none; W > 0: the row at position p attends to positions
 *                 max(0, p - W + 1) .. p only ([IW] sliding-window item); entries
 *                 of blocks wholly before the first row's window are never read
 *   out           [batch][chunk_len][n_q][head_dim], out_dtype PA_F32 or cache->dtype
 * Rows at negative positions (context_lens[b] < chunk_len) are zero. A context
 * length past max_blocks_per_seq * block_size, or a block id outside the pool
 * among the ones the sequence's rows read, turns every row of that sequence into
 * NaN instead of an out-of-bounds read. Supported: head_dim 64 or 128; the
 * size limits of pa_paged_attn_prefill with chunk_len in place of seq_len.
 * bf16 caches: when batch * max_blocks_per_seq * n_kv * 16 * head_dim * 2 bytes
 * (plus one byte per block) fit in 256 MiB, the call first copies the V rows it
 * reads to f16 (exact below 65520 in magnitude, as for pa_paged_attn_prefill) in
 * the workspace (below), and P V then runs with one f16 P part; blocks holding a
 * larger value keep the bf16 hi + lo product. Calls that share that workspace
 * must not overlap on the GPU.
 * Option PA_OPT_PREFILL_STAGE_V = 0 turns the copy off.
 *   workspace     device scratch of at least pa_chunked_prefill_workspace_bytes(...)
 *                 bytes for the same batch, max_blocks_per_seq and cache (16-byte
 *                 aligned; 0 bytes: none is used), or NULL: then the workspace of
 *                 pa_set_workspace if large enough, else the library's own (as for
 *                 pa_paged_attn_decode).
 */
size_t pa_chunked_prefill_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq,
                                          const pa_cache_desc* cache);
int pa_paged_attn_chunked_prefill(const void* q, int32_t batch, int32_t chunk_len, int32_t n_q,
                                  const void* k_cache, const void* v_cache, const pa_cache_desc* cache,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, float scale, int32_t window,
                                  const float* alibi_slopes,
                                  void* out, pa_dtype out_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * kv_append_quant -- quantise new K/V rows into a one-byte cache and write them
 * through slot_mapping. [IW] "KV Cache 的形状与增长", INT8 / FP8 item (the fp16
 * cache quantised to int8 or fp8 per channel or per token; one byte per element in
 * the KV-size formula); [VC] slot mapping.
 *
 *   k, v          [num_tokens][n_kv][head_dim] in src_dtype (f32, bf16 or f16)
 *   slot_mapping  int64 [num_tokens], as for pa_kv_append (negative or past the
 *                 pool: skipped)
 *   k_cache, v_cache  code pools [num_blocks][n_kv][block_size][head_dim], one
 *                 byte per element: OCP FP8 E4M3 (cache->dtype PA_FP8_E4M3) or
 *                 two's-complement INT8 (PA_INT8)
 *   k_scale, v_scale  fp32 [num_blocks][n_kv][block_size]: one scale per row,
 *                 written here; for a _PER_CHANNEL cache dtype instead the fixed
 *                 channel scales [n_kv][head_dim] (16-byte aligned), only read
 * Per row: every (token, KV head) row x of K and of V is quantised on its own, with every
 * step one correctly rounded fp32 operation: amax = max |x_i|; scale = amax / QMAX
 * (448 for E4M3, 127 for INT8); a scale below the smallest normal float (amax = 0
 * included) is stored as 0 with all codes 0; otherwise y_i = x_i * (1 / scale) and
 * the code is the nearest E4M3 value of y_i clamped to [-448, 448] (ties to the
 * even code) or rint(y_i) clamped to [-127, 127]. The stored value of a code is
 * code * scale. Per channel ([IW]'s other granularity, read as fixed scales a
 * caller calibrates in advance, since a cache filled one token at a time cannot
 * take a channel's range from tokens still to come): element c of every row of
 * KV head g with s = scale[g][c]: s below the smallest normal float stores code
 * 0; otherwise y = x * (1 / s) and the same code rule, so values past QMAX * s
 * saturate at +-QMAX. The stored value is code * s. Rows must be finite. A
 * scale per KV head, or one for the whole cache, is this form with every
 * channel of a head (or of the cache) given the same scale.
 * num_tokens == 0 is a no-op.
 */
int pa_kv_append_quant(const void* k, const void* v, pa_dtype src_dtype, const int64_t* slot_mapping,
                       int32_t num_tokens, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                       const pa_cache_desc* cache, void* stream);

/*
 * paged_attn_decode_quant -- pa_paged_attn_decode over a quantised cache: K and V
 * values are code * scale of their row ([IW] INT8 / FP8 item), the attention is
 * the same softmax(q K^T * scale + M) V.
 *
 *   q             [batch][n_q][head_dim] in q_dtype (bf16 or f16)
 *   k_cache, v_cache, k_scale, v_scale  as written by pa_kv_append_quant (per row),
 *                 or the codes and the fixed channel scales [n_kv][head_dim]
 *   cache->dtype  PA_FP8_E4M3 or PA_INT8, or their _PER_CHANNEL forms
 *   out           [batch][n_q][head_dim], out_dtype PA_F32 or q_dtype
 *   other arguments as for pa_paged_attn_decode (window, workspace sized by
 *   pa_decode_workspace_bytes with this cache description).
 * Codes are widened exactly to q's type and multiplied on the matrix cores in
 * fp32; unused slots (codes or scales, NaN included) never reach the output.
 * Per channel, q times the K channel scales enters the bf16 matrix cores as a
 * bf16 hi + lo pair (about 16 significant bits) and the V channel scales
 * multiply the output once.
 */
int pa_paged_attn_decode_quant(const void* q, pa_dtype q_dtype, int32_t batch, int32_t n_q,
                               const void* k_cache, const void* v_cache, const float* k_scale,
                               const float* v_scale, const pa_cache_desc* cache,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, float scale, int32_t window,
                               const float* alibi_slopes, void* out,
                               pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_quant_append -- one decode step over a quantised cache in
 * one launch: pa_kv_append_quant of each sequence's new token fused into
 * pa_paged_attn_decode_quant ([IW] decode step: write the new K/V at position
 * cache_len, then attend over the whole cache; [IW] INT8 / FP8 item).
 *
 *   k_new, v_new  [batch][n_kv][head_dim] in q_dtype: the new token of each sequence
 *   slot_mapping  int64 [batch]: its slot (negative: sequence b appends nothing)
 *   k_cache, v_cache, k_scale, v_scale  the pools and per-row scales (written)
 *   other arguments as for pa_paged_attn_decode_quant.
 * The new rows are quantised exactly as pa_kv_append_quant does, so codes,
 * scales and outputs equal those of the two calls bit for bit, under the same
 * conditions as pa_paged_attn_decode_append: each sequence's slot must be its
 * position ctx - 1, in a block no other sequence of the call reads
 * (option PA_OPT_VALIDATE checks both).
 */
int pa_paged_attn_decode_quant_append(const void* q, const void* k_new, const void* v_new, pa_dtype q_dtype,
                                      const int64_t* slot_mapping, int32_t batch, int32_t n_q, void* k_cache,
                                      void* v_cache, float* k_scale, float* v_scale, const pa_cache_desc* cache,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, float scale, int32_t window,
                         const float* alibi_slopes, void* out,
                                      pa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * paged_attn_decode_multi_quant / paged_attn_chunked_prefill_quant -- the
 * several-rows-per-sequence calls over a quantised cache: row r of sequence b
 * sits at position context_lens[b] - rows + r and attends to positions 0 .. that
 * position ([AE] 1.1 causal mask aligned at the bottom right; [IW] chunked
 * prefill and the verification of drafted tokens; [IW] INT8 / FP8 item for the
 * values code * scale of their row).
 *
 *   q             [batch][rows][n_q][head_dim] in q_dtype (bf16 or f16), rows =
 *                 q_rows or chunk_len
 *   k_cache, v_cache, k_scale, v_scale, cache  as for pa_paged_attn_decode_quant,
 *                 already holding the rows' own K/V (pa_kv_append_quant first)
 *   block_table, context_lens, scale, window, alibi_slopes  as for
 *                 pa_paged_attn_decode_multi
 *   out           [batch][rows][n_q][head_dim], out_dtype PA_F32 or q_dtype
 *   workspace     scratch of pa_decode_multi_workspace_bytes(batch, rows, n_q,
 *                 max_blocks_per_seq, cache) bytes (that query takes quantised
 *                 descriptions), or NULL as for pa_paged_attn_decode
 * Both run the quantised-cache decode kernel with the (query head, row) pairs
 * of a KV head as its matrix-core columns, 16 (or 8, 4, 2, 1) per workgroup
 * slice; every slice streams the codes of the keys its rows reach, so the two
 * calls differ only in name. Rows at negative positions are zero; a context
 * past the block table's reach or an out-of-pool block id among those read
 * gives NaN rows. Supported: head_dim 64 or 128, batch at most 65535, and at
 * most 65535 slices, n_kv * G * rows / w with G = n_q / n_kv and w the largest
 * of 16, 8, 4, 2, 1 that divides G * rows; else PA_ERR_UNSUPPORTED.
 * chunk_len == 0 or batch == 0 is a no-op.
 */
int pa_paged_attn_decode_multi_quant(const void* q, pa_dtype q_dtype, int32_t batch, int32_t q_rows, int32_t n_q,
                                     const void* k_cache, const void* v_cache, const float* k_scale,
                                     const float* v_scale, const pa_cache_desc* cache,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, float scale, int32_t window,
                                     const float* alibi_slopes, void* out, pa_dtype out_dtype, void* workspace,
                                     size_t workspace_bytes, void* stream);
int pa_paged_attn_chunked_prefill_quant(const void* q, pa_dtype q_dtype, int32_t batch, int32_t chunk_len,
                                        int32_t n_q, const void* k_cache, const void* v_cache, const float* k_scale,
                                        const float* v_scale, const pa_cache_desc* cache,
                                        const int32_t* block_table, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, float scale, int32_t window,
                                        const float* alibi_slopes, void* out, pa_dtype out_dtype, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Tuning override for the decode partition size, in tokens (a multiple of 16
 * and of the work one workgroup takes per pass). 0 restores the built-in
 * choice. Affects later pa_decode_workspace_bytes and pa_paged_attn_decode
 * calls in this process; returns the previous value, or -1 (and leaves the
 * setting unchanged) for an invalid value.
 */
int32_t pa_set_decode_partition_tokens(int32_t tokens);

/*
 * Kernel-choice options. Each starts at the value of its environment variable
 * (read once, when the library first needs an option; an unset, unparsable or
 * out-of-range variable gives the default) and then changes only through
 * pa_set_option. Process-wide, like the partition size: a call made while
 * another thread changes an option sees the old or the new value, and the
 * *_workspace_bytes queries must be made under the same options as the calls
 * they size.
 */
typedef enum {
    /* PA_DECODE_MFMA: 1 (default) runs bf16/f16 decode, and multi-row decode of
     * at most 16 (head, row) pairs per KV head, on the matrix-core kernel when the
     * pairs per KV head are a multiple of 4; 0 always takes the VALU kernel. */
    PA_OPT_DECODE_MATRIX_CORES = 0,
    /* PA_DECODE_RING: K/V blocks each decode wave keeps in flight, 1 (default) or 2. */
    PA_OPT_DECODE_RING = 1,
    /* PA_DECODE_WAVES: waves per decode workgroup, 1..8; 0 (default) lets the
     * planner choose from the shape and the device's compute units. */
    PA_OPT_DECODE_WAVES = 2,
    /* PA_PREFILL_STAGE_V: 1 (default) stages a bf16 V as f16 for the P V product
     * of prefill and chunked prefill; 0 keeps P V in bf16 hi + lo parts. */
    PA_OPT_PREFILL_STAGE_V = 3,
    /* PA_VALIDATE: 1 turns on the debug-mode checks of device metadata described
     * at the top of this header; 0 (default) leaves them off. */
    PA_OPT_VALIDATE = 4,
    PA_OPT_COUNT = 5
} pa_option;

/* Sets `option` (a pa_option) to `value`; returns the previous value, or -1
 * (changing nothing) for an unknown option or a value outside its range. */
int32_t pa_set_option(int32_t option, int32_t value);

/* Current value of `option`, or -1 for an unknown option. */
int32_t pa_get_option(int32_t option);

/*
 * Default decode workspace for calls that pass workspace == NULL ([VC]/[IW]
 * Flash Decoding partials). `workspace` is caller-owned device memory of
 * `bytes` bytes, 16-byte aligned, that must stay valid while such calls run;
 * NULL (with bytes == 0) clears the setting. Process-wide; returns PA_OK or
 * PA_ERR_INVALID_ARG.
 */
int pa_set_workspace(void* workspace, size_t bytes);

/* Thread-local, NUL-terminated description of the last failure on this thread. */
const char* pa_last_error(void);

/* Library ABI version (major * 100 + minor). */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
