/*
 * oracle.c -- plain, slow, fp64 CPU oracle for paged GQA attention.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It includes nothing
 * from the GPU library and the GPU library includes nothing from here; the
 * two share no headers, helpers, tables or constants.
 *
 * Web pages this follows (tags used below):
 *  [AE] "注意力演进与推理流程" (attention evolution and inference flow),
 *       jerryiiii.gitbook.io/llm-review/notes/attention/attention-evolution-and-inference
 *  [PD] xinc.fun/index.php/archives/233 (prefill vs decode, KV cache, PagedAttention)
 *  [VC] yyzxw.github.io/acknowledge/research/vllm-concepts-deep-dive/section-1.html
 *  [IW] "LLM 推理全过程的维度变化与核心公式" (LLM inference walkthrough),
 *       research.frankk.site/notes/llm-inference-walkthrough
 *
 * What is computed is the textbook definition written out, with no
 * blocking, no online softmax and no split of the context:
 *   s_t   = scale * <q_h, K_{g(h)}[t]>            [VC] self-attention Step 2 (scaled dot product)
 *   w_t   = exp(s_t - max_u s_u)                  [VC] Step 3 (softmax normalisation)
 *   out_h = sum_t w_t V_{g(h)}[t] / sum_t w_t     [VC] Step 4 (weighted aggregation)
 *   g(h)  = floor(h / G), G = n_q / n_kv          [AE] section 3.1 (GQA grouping rule)
 * Subtracting the maximum before exp leaves the softmax value unchanged;
 * it only keeps exp() in range.
 *
 * Decode: one query per sequence attends to context positions [0, ctx_b)
 * ([VC] decode-stage attention over K_{<=t}, V_{<=t}; [IW] "Decode 阶段维度流转":
 * no causal mask is needed in decode). Positions are found through the
 * block table: logical position t of sequence b lives in physical block
 * block_table[b][t / bs] at in-block offset t % bs ([PD] section 6
 * PagedAttention; [IW] "KV Cache 的形状与增长", Paged Attention item, block of
 * 16 tokens). Pool layout: element (phys, g, off, c) sits at
 * ((phys * n_kv + g) * bs + off) * d + c.
 *
 * Prefill: every position i of a contiguous prompt attends to keys j <= i
 * (causal mask M_ij = 0 for j <= i, else -inf: [AE] section 1.1; [PD]
 * section 2), or to all keys when causal == 0.
 *
 * kv_append: token t's K/V rows are stored at flat slot slot_mapping[t] =
 * phys_block * bs + offset ([VC] PagedAttention paragraph: kernels receive a
 * block table and a slot mapping; [IW] decode step "write the KV cache at the
 * next position").
 *
 * Inputs arrive as the exact stored values (fp32, bf16 or fp16 bit
 * patterns) and are widened to fp64 exactly, so input rounding is not
 * counted as error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* element type codes understood by this file */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

/* ---- exact widening of stored values to fp64 ---------------------------- */

/* bfloat16 is the upper half of an IEEE-754 binary32 pattern. */
static double widen_bf16(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double widen_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (e == 0) {
        mag = ldexp((double)frac, -24);            /* subnormal: frac * 2^-24 */
    } else if (e == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), e - 25); /* (1.frac) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

static int elem_bytes_of(int dtype) {
    switch (dtype) {
    case ORACLE_F32: return 4;
    case ORACLE_BF16: return 2;
    case ORACLE_F16: return 2;
    default: return 0;
    }
}

static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    if (dtype == ORACLE_BF16) return widen_bf16(((const uint16_t*)base)[idx]);
    return widen_f16(((const uint16_t*)base)[idx]);
}

int oracle_upcast(const void* src, int dtype, int64_t n, double* dst) {
    if (!src || !dst || n < 0 || elem_bytes_of(dtype) == 0) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, dtype, i);
    return 0;
}

/* ---- kv_append: host model of the slot-mapped cache write ---------------- */

/*
 * For every token t with slot_mapping[t] >= 0: copy k[t][g][:] and
 * v[t][g][:] (all n_kv heads) into the pools at block slot / bs, offset
 * slot % bs. Negative slots mark padding tokens and are skipped. The copy is
 * a byte copy, so the pools hold exactly the input bit patterns.
 * Returns the number of tokens written, or -1 (pools untouched) when an
 * argument is invalid or a slot lies past the end of the pool.
 */
int64_t oracle_kv_append(const void* k, const void* v, const int64_t* slot_mapping,
                         int64_t num_tokens, int32_t n_kv, int32_t head_dim,
                         int32_t elem_bytes, int64_t num_blocks, int32_t block_size,
                         void* k_pool, void* v_pool) {
    if (!k || !v || !slot_mapping || !k_pool || !v_pool) return -1;
    if (num_tokens < 0 || n_kv <= 0 || head_dim <= 0 || elem_bytes <= 0 ||
        num_blocks <= 0 || block_size <= 0)
        return -1;
    const int64_t n_slots = num_blocks * (int64_t)block_size;
    for (int64_t t = 0; t < num_tokens; ++t)
        if (slot_mapping[t] >= n_slots) return -1;

    const size_t row = (size_t)head_dim * (size_t)elem_bytes;
    int64_t written = 0;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        const int64_t blk = slot / block_size;
        const int64_t off = slot % block_size;
        for (int32_t g = 0; g < n_kv; ++g) {
            const size_t src = ((size_t)t * n_kv + g) * row;
            const size_t dst = (((size_t)blk * n_kv + g) * block_size + off) * row;
            memcpy((char*)k_pool + dst, (const char*)k + src, row);
            memcpy((char*)v_pool + dst, (const char*)v + src, row);
        }
        ++written;
    }
    return written;
}

/* ---- softmax-weighted average over a list of key positions -------------- */

/*
 * out[c] = sum_t w_t V[t][c] / sum_t w_t with w_t = exp(s_t - max s),
 * s_t = scale * <q, K[t]>. Key t is fetched through key_index(t), an element
 * offset of K[t][0] (and V[t][0]) in k_base / v_base. n_keys == 0 gives a
 * zero row (an empty context attends to nothing).
 */
typedef struct {
    const void* k_base;
    const void* v_base;
    int dtype;
    int64_t* key_off;     /* element offset of row t, length n_keys */
    int64_t n_keys;
} key_list;

static void attend(const double* q, int32_t d, double scale, const key_list* keys,
                   double* scores, double* out) {
    for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
    if (keys->n_keys == 0) return;

    double m = -INFINITY;
    for (int64_t t = 0; t < keys->n_keys; ++t) {
        double dot = 0.0;
        const int64_t base = keys->key_off[t];
        for (int32_t c = 0; c < d; ++c) dot += q[c] * load_elem(keys->k_base, keys->dtype, base + c);
        scores[t] = scale * dot;
        if (scores[t] > m) m = scores[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < keys->n_keys; ++t) {
        const double w = exp(scores[t] - m);
        den += w;
        const int64_t base = keys->key_off[t];
        for (int32_t c = 0; c < d; ++c) out[c] += w * load_elem(keys->v_base, keys->dtype, base + c);
    }
    for (int32_t c = 0; c < d; ++c) out[c] /= den;
}

static int set_threads(int32_t n_threads) {
#ifdef _OPENMP
    return n_threads > 0 ? n_threads : omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}

/* ---- decode over the paged cache ---------------------------------------- */

/*
 * q            [batch][n_q][head_dim]                      (dtype)
 * k_pool/v_pool[num_blocks][n_kv][block_size][head_dim]    (dtype)
 * block_table  [batch][max_blocks_per_seq] int32
 * context_lens [batch] int32, tokens attended (0 <= ctx <= max_blocks*bs)
 * window       0: all ctx positions; W > 0: only the last W of them, positions
 *              max(0, ctx - W) .. ctx - 1 (sliding-window attention, [IW]
 *              "KV Cache 的形状与增长", sliding-window item: the cache is bounded at
 *              W recent positions)
 * sel          optional list of n_sel (b, h) pairs; NULL means every (b, h)
 * out          [batch][n_q][head_dim] fp64 (or [n_sel][head_dim] with sel)
 * Returns 0, or -1 for invalid arguments or a block id outside the pool.
 */
int oracle_decode(const void* q, const void* k_pool, const void* v_pool, int dtype,
                  int32_t batch, int32_t n_q, int32_t n_kv, int32_t head_dim,
                  int64_t num_blocks, int32_t block_size,
                  const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, double scale, int32_t window,
                  const int32_t* sel, int64_t n_sel, double* out, int32_t n_threads) {
    if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out) return -1;
    if (window < 0) return -1;
    if (elem_bytes_of(dtype) == 0 || batch < 0 || n_q <= 0 || n_kv <= 0 || head_dim <= 0 ||
        num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq < 0)
        return -1;
    if (n_q % n_kv != 0) return -1;
    const int32_t group = n_q / n_kv;
    const int64_t n_items = sel ? n_sel : (int64_t)batch * n_q;

    /* validate everything the loops below will index */
    for (int64_t it = 0; it < n_items; ++it) {
        int32_t b = sel ? sel[2 * it] : (int32_t)(it / n_q);
        int32_t h = sel ? sel[2 * it + 1] : (int32_t)(it % n_q);
        if (b < 0 || b >= batch || h < 0 || h >= n_q) return -1;
        const int32_t ctx = context_lens[b];
        if (ctx < 0 || (int64_t)ctx > (int64_t)max_blocks_per_seq * block_size) return -1;
        for (int32_t j = 0; j < (ctx + block_size - 1) / block_size; ++j) {
            const int32_t phys = block_table[(int64_t)b * max_blocks_per_seq + j];
            if (phys < 0 || phys >= num_blocks) return -1;
        }
    }

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(set_threads(n_threads)) reduction(| : bad)
    for (int64_t it = 0; it < n_items; ++it) {
        const int32_t b = sel ? sel[2 * it] : (int32_t)(it / n_q);
        const int32_t h = sel ? sel[2 * it + 1] : (int32_t)(it % n_q);
        const int32_t g = h / group;                          /* [AE] 3.1: g = floor(h / G) */
        const int32_t ctx = context_lens[b];

        double* qv = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* scores = (double*)malloc(sizeof(double) * (size_t)(ctx > 0 ? ctx : 1));
        int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ctx > 0 ? ctx : 1));
        if (!qv || !scores || !offs) {
            bad |= 1;
        } else {
            for (int32_t c = 0; c < head_dim; ++c)
                qv[c] = load_elem(q, dtype, ((int64_t)b * n_q + h) * head_dim + c);
            const int32_t first = (window > 0 && ctx > window) ? ctx - window : 0;
            for (int32_t t = first; t < ctx; ++t) {
                /* block-table translation: logical t -> (physical block, offset) */
                const int64_t phys = block_table[(int64_t)b * max_blocks_per_seq + t / block_size];
                const int64_t off = t % block_size;
                offs[t - first] = ((phys * n_kv + g) * block_size + off) * head_dim;
            }
            key_list keys = {k_pool, v_pool, dtype, offs, ctx - first};
            attend(qv, head_dim, scale, &keys, scores, out + it * head_dim);
        }
        free(qv);
        free(scores);
        free(offs);
    }
    return bad ? -1 : 0;
}

/* ---- prefill over contiguous Q/K/V --------------------------------------- */

/*
 * q   [batch][seq_len][n_q][head_dim], k/v [batch][seq_len][n_kv][head_dim]
 * sel optional list of n_sel (b, h, i) triples; NULL means every (b, i, h)
 * out [batch][seq_len][n_q][head_dim] fp64 (or [n_sel][head_dim] with sel)
 * Row i attends to keys j <= i when causal, else to all seq_len keys; with
 * window W > 0 (causal only) to keys max(0, i - W + 1) .. i.
 */
int oracle_prefill(const void* q, const void* k, const void* v, int dtype,
                   int32_t batch, int32_t seq_len, int32_t n_q, int32_t n_kv,
                   int32_t head_dim, int32_t causal, double scale, int32_t window,
                   const int32_t* sel, int64_t n_sel, double* out, int32_t n_threads) {
    if (!q || !k || !v || !out) return -1;
    if (window < 0 || (window > 0 && !causal)) return -1;
    if (elem_bytes_of(dtype) == 0 || batch < 0 || seq_len < 0 || n_q <= 0 || n_kv <= 0 ||
        head_dim <= 0)
        return -1;
    if (n_q % n_kv != 0) return -1;
    const int32_t group = n_q / n_kv;
    const int64_t n_items = sel ? n_sel : (int64_t)batch * seq_len * n_q;
    for (int64_t it = 0; sel && it < n_items; ++it) {
        if (sel[3 * it] < 0 || sel[3 * it] >= batch || sel[3 * it + 1] < 0 ||
            sel[3 * it + 1] >= n_q || sel[3 * it + 2] < 0 || sel[3 * it + 2] >= seq_len)
            return -1;
    }

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) num_threads(set_threads(n_threads)) reduction(| : bad)
    for (int64_t it = 0; it < n_items; ++it) {
        int32_t b, h, i;
        if (sel) {
            b = sel[3 * it];
            h = sel[3 * it + 1];
            i = sel[3 * it + 2];
        } else {                                   /* natural order of out: [b][i][h] */
            b = (int32_t)(it / ((int64_t)seq_len * n_q));
            i = (int32_t)((it / n_q) % seq_len);
            h = (int32_t)(it % n_q);
        }
        const int32_t g = h / group;
        const int32_t n_keys = causal ? i + 1 : seq_len;     /* M_ij = -inf for j > i */
        const int32_t first = (window > 0 && i + 1 > window) ? i + 1 - window : 0;

        double* qv = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* scores = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
        int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_keys > 0 ? n_keys : 1));
        if (!qv || !scores || !offs) {
            bad |= 1;
        } else {
            for (int32_t c = 0; c < head_dim; ++c)
                qv[c] = load_elem(q, dtype, (((int64_t)b * seq_len + i) * n_q + h) * head_dim + c);
            for (int32_t j = first; j < n_keys; ++j)
                offs[j - first] = (((int64_t)b * seq_len + j) * n_kv + g) * head_dim;
            key_list keys = {k, v, dtype, offs, n_keys - first};
            attend(qv, head_dim, scale, &keys, scores, out + it * head_dim);
        }
        free(qv);
        free(scores);
        free(offs);
    }
    return bad ? -1 : 0;
}

/* number of OpenMP threads a call with n_threads == 0 would use */
int oracle_max_threads(void) { return set_threads(0); }
