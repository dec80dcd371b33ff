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
 * Quantised cache ([IW] "KV Cache 的形状与增长", INT8 / FP8 item: the fp16
 * cache is quantised to int8 or fp8 per channel or per token; the
 * dimension-walkthrough page's KV-size formula counts FP8 as one byte):
 * each (token, KV head) row of K and of V is stored as one-byte codes, value =
 * code * scale, with the scale taken either per token (one fp32 scale per row,
 * symmetric, absolute maximum; fp32 steps at oracle_quantize_rows) or per
 * channel (one fixed fp32 scale per (KV head, channel), given by the caller;
 * fp32 steps at oracle_quantize_channels). FP8 is the OCP E4M3 ("fn") format: 1 sign bit, 4
 * exponent bits with bias 7, 3 fraction bits, no infinities, one NaN
 * pattern per sign, largest finite value 448.
 *
 * Inputs arrive as the exact stored values (fp32, bf16 or fp16 bit
 * patterns, or one-byte codes) and are widened to fp64 exactly, so input
 * rounding is not counted as error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* element type codes understood by this file */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2, ORACLE_FP8E4M3 = 3, ORACLE_INT8 = 4 };

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

/* OCP FP8 E4M3: sign, exponent e (bias 7), fraction m. e = 0 is subnormal
 * (m * 2^-9); e = 15 with m = 7 is NaN; otherwise (8 + m) * 2^(e - 10). */
static double widen_fp8_e4m3(uint8_t c) {
    const int sign = c >> 7;
    const int e = (c >> 3) & 15;
    const int m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp((double)(8 + m), e - 10);
    return sign ? -mag : mag;
}

static int elem_bytes_of(int dtype) {
    switch (dtype) {
    case ORACLE_F32: return 4;
    case ORACLE_BF16: return 2;
    case ORACLE_F16: return 2;
    case ORACLE_FP8E4M3: return 1;
    case ORACLE_INT8: return 1;
    default: return 0;
    }
}

static int is_quantised(int dtype) { return dtype == ORACLE_FP8E4M3 || dtype == ORACLE_INT8; }

static double load_elem(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case ORACLE_F32: return (double)((const float*)base)[idx];
    case ORACLE_BF16: return widen_bf16(((const uint16_t*)base)[idx]);
    case ORACLE_FP8E4M3: return widen_fp8_e4m3(((const uint8_t*)base)[idx]);
    case ORACLE_INT8: return (double)((const int8_t*)base)[idx];
    default: return widen_f16(((const uint16_t*)base)[idx]);
    }
}

/* ---- per-token quantisation (fp32 steps, as stored) ---------------------- */

/* Nearest E4M3 code of a finite y with |y| <= 448, ties to the even code. */
static uint8_t encode_fp8_e4m3(float y) {
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs((double)y);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: a = m * 2^-9; m = 8 is the smallest normal, code 8 */
        return sign | (uint8_t)nearbyint(ldexp(a, 9));
    }
    int e2;
    const double fr = frexp(a, &e2);          /* a = fr * 2^e2, fr in [0.5, 1) */
    int e = e2 - 1;                           /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double q = nearbyint((2.0 * fr - 1.0) * 8.0);   /* fraction in eighths */
    if (q == 8.0) {
        q = 0.0;
        ++e;
    }
    return sign | (uint8_t)(((e + 7) << 3) | (int)q);
}

int oracle_encode_fp8_e4m3(const float* y, int64_t n, uint8_t* out) {
    if (!y || !out || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        if (!(fabsf(y[i]) <= 448.0f)) return -1;
        out[i] = encode_fp8_e4m3(y[i]);
    }
    return 0;
}

/* The code of y = x / scale (an fp32 value): E4M3, the nearest code of y clamped
 * to [-448, 448]; INT8, y rounded to the nearest integer (ties to even) and
 * clamped to [-127, 127]. */
static uint8_t code_of(float y, int fmt) {
    if (fmt == ORACLE_FP8E4M3) {
        const float c = fminf(fmaxf(y, -448.0f), 448.0f);
        return encode_fp8_e4m3(c);
    }
    const float r = fminf(fmaxf(rintf(y), -127.0f), 127.0f);
    return (uint8_t)(int8_t)r;
}

/*
 * One row x[0..d) of the source type to codes and a scale, all in fp32:
 *   amax  = max_i |x_i|
 *   scale = amax / QMAX                (QMAX = 448 for E4M3, 127 for INT8)
 *   scale below the smallest normal float (amax = 0 included): scale = 0,
 *         every code 0
 *   inv   = 1 / scale,  y_i = x_i * inv
 *   E4M3: code_i = nearest E4M3 value of y_i clamped to [-448, 448]
 *   INT8: code_i = y_i rounded to the nearest integer (ties to even),
 *         clamped to [-127, 127]
 * Every step is one correctly rounded fp32 operation, so the result is a
 * function of the stored inputs alone. Rows must be finite.
 */
static void quantise_row(const void* x, int src_dtype, int64_t row0, int32_t d, int fmt,
                         uint8_t* codes, float* scale_out) {
    float amax = 0.0f;
    for (int32_t i = 0; i < d; ++i) {
        const float a = fabsf((float)load_elem(x, src_dtype, row0 + i));
        if (a > amax) amax = a;
    }
    const float qmax = fmt == ORACLE_FP8E4M3 ? 448.0f : 127.0f;
    volatile float scale = amax / qmax;
    if (!(scale >= 0x1p-126f)) {
        for (int32_t i = 0; i < d; ++i) codes[i] = 0;
        *scale_out = 0.0f;
        return;
    }
    volatile float inv = 1.0f / scale;
    for (int32_t i = 0; i < d; ++i) {
        volatile float y = (float)load_elem(x, src_dtype, row0 + i) * inv;
        codes[i] = code_of(y, fmt);
    }
    *scale_out = scale;
}

/* x [n_rows][d] in src_dtype -> codes [n_rows][d], scales [n_rows]. */
int oracle_quantize_rows(const void* x, int src_dtype, int64_t n_rows, int32_t d, int fmt,
                         uint8_t* codes, float* scales) {
    if (!x || !codes || !scales || n_rows < 0 || d <= 0) return -1;
    if (is_quantised(src_dtype) || elem_bytes_of(src_dtype) == 0 || !is_quantised(fmt)) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        quantise_row(x, src_dtype, r * d, d, fmt, codes + r * d, scales + r);
    return 0;
}

/*
 * Per-channel quantisation (the "per channel" reading of the same item): channel
 * c of KV head g has one fp32 scale s = scales[g * d + c], fixed in advance by
 * the caller (a cache filled one token at a time cannot take a channel's range
 * from tokens that have not arrived yet). Element c of a row of head g:
 *   s below the smallest normal float (0 included): code 0
 *   inv = 1 / s,  y = x * inv,  code = code_of(y): values past QMAX * s saturate
 * each step one correctly rounded fp32 operation, as per token.
 */
static uint8_t quantise_channel_elem(float x, float s, int fmt) {
    if (!(s >= 0x1p-126f)) return 0;
    volatile float inv = 1.0f / s;
    volatile float y = x * inv;
    return code_of(y, fmt);
}

/* x [n_rows][n_kv][d] in src_dtype -> codes [n_rows][n_kv][d] with scales [n_kv][d]. */
int oracle_quantize_channels(const void* x, int src_dtype, int64_t n_rows, int32_t n_kv, int32_t d, int fmt,
                             const float* scales, uint8_t* codes) {
    if (!x || !codes || !scales || n_rows < 0 || n_kv <= 0 || d <= 0) return -1;
    if (is_quantised(src_dtype) || elem_bytes_of(src_dtype) == 0 || !is_quantised(fmt)) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int32_t g = 0; g < n_kv; ++g)
            for (int32_t c = 0; c < d; ++c) {
                const int64_t i = (r * n_kv + g) * d + c;
                codes[i] = quantise_channel_elem((float)load_elem(x, src_dtype, i), scales[(int64_t)g * d + c], fmt);
            }
    return 0;
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

/*
 * kv_append into a quantised cache: every (token, KV head) row of k and v
 * (src_dtype, [num_tokens][n_kv][head_dim]) is quantised per token as in
 * oracle_quantize_rows; codes go to the pools [num_blocks][n_kv][block_size]
 * [head_dim] (one byte each) and scales to k_scale / v_scale
 * [num_blocks][n_kv][block_size], both at block slot / bs, offset slot % bs.
 * Slot rules and the return value are those of oracle_kv_append.
 */
int64_t oracle_kv_append_quant(const void* k, const void* v, int src_dtype,
                               const int64_t* slot_mapping, int64_t num_tokens, int32_t n_kv,
                               int32_t head_dim, int fmt, int64_t num_blocks, int32_t block_size,
                               uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale) {
    if (!k || !v || !slot_mapping || !k_pool || !v_pool || !k_scale || !v_scale) return -1;
    if (is_quantised(src_dtype) || elem_bytes_of(src_dtype) == 0 || !is_quantised(fmt)) return -1;
    if (num_tokens < 0 || n_kv <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
        return -1;
    const int64_t n_slots = num_blocks * (int64_t)block_size;
    for (int64_t t = 0; t < num_tokens; ++t)
        if (slot_mapping[t] >= n_slots) return -1;
    int64_t written = 0;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        const int64_t blk = slot / block_size;
        const int64_t off = slot % block_size;
        for (int32_t g = 0; g < n_kv; ++g) {
            const int64_t src_row = (t * n_kv + g) * (int64_t)head_dim;
            const int64_t dst_row = (blk * n_kv + g) * block_size + off;
            quantise_row(k, src_dtype, src_row, head_dim, fmt, k_pool + dst_row * head_dim,
                         k_scale + dst_row);
            quantise_row(v, src_dtype, src_row, head_dim, fmt, v_pool + dst_row * head_dim,
                         v_scale + dst_row);
        }
        ++written;
    }
    return written;
}

/*
 * kv_append into a per-channel quantised cache: element c of every (token, KV
 * head g) row of k and v is quantised with k_chan[g * d + c] / v_chan[g * d + c]
 * as in oracle_quantize_channels, and the codes go to the pools at block
 * slot / bs, offset slot % bs; nothing else is written. Slot rules and the
 * return value are those of oracle_kv_append.
 */
int64_t oracle_kv_append_quant_channel(const void* k, const void* v, int src_dtype,
                                       const int64_t* slot_mapping, int64_t num_tokens, int32_t n_kv,
                                       int32_t head_dim, int fmt, int64_t num_blocks, int32_t block_size,
                                       uint8_t* k_pool, uint8_t* v_pool, const float* k_chan,
                                       const float* v_chan) {
    if (!k || !v || !slot_mapping || !k_pool || !v_pool || !k_chan || !v_chan) return -1;
    if (is_quantised(src_dtype) || elem_bytes_of(src_dtype) == 0 || !is_quantised(fmt)) return -1;
    if (num_tokens < 0 || n_kv <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
        return -1;
    const int64_t n_slots = num_blocks * (int64_t)block_size;
    for (int64_t t = 0; t < num_tokens; ++t)
        if (slot_mapping[t] >= n_slots) return -1;
    int64_t written = 0;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        const int64_t blk = slot / block_size;
        const int64_t off = slot % block_size;
        for (int32_t g = 0; g < n_kv; ++g) {
            const int64_t src = (t * n_kv + g) * (int64_t)head_dim;
            const int64_t dst = ((blk * n_kv + g) * block_size + off) * head_dim;
            for (int32_t c = 0; c < head_dim; ++c) {
                const int64_t sc = (int64_t)g * head_dim + c;
                k_pool[dst + c] = quantise_channel_elem((float)load_elem(k, src_dtype, src + c), k_chan[sc], fmt);
                v_pool[dst + c] = quantise_channel_elem((float)load_elem(v, src_dtype, src + c), v_chan[sc], fmt);
            }
        }
        ++written;
    }
    return written;
}

/* ---- softmax-weighted average over a list of key positions -------------- */

/*
 * out[c] = sum_t w_t V[t][c] / sum_t w_t with w_t = exp(s_t - max s),
 * s_t = scale * <q, K[t]> - slope * (qpos - kpos_t). Key t is fetched through
 * key_off[t], an element offset of K[t][0] (and V[t][0]) in k_base / v_base, and
 * sits at position kpos_t = kpos0 + t; the query sits at position qpos. The
 * second term is ALiBi's linear bias ("LLM 推理全过程的维度变化与核心公式",
 * research.frankk.site, position-encoding section: scores_ij = q_i.k_j / sqrt(d)
 * - m_h (i - j), one slope m_h per head); slope 0 leaves plain attention.
 * n_keys == 0 gives a zero row (an empty context attends to nothing).
 */
typedef struct {
    const void* k_base;
    const void* v_base;
    int dtype;
    int64_t* key_off;     /* element offset of row t, length n_keys */
    int64_t n_keys;
    const float* k_scale; /* per-token quantised cache: scale of row key_off / head_dim; else NULL */
    const float* v_scale;
    int64_t kpos0;        /* position of key 0 */
    const float* k_chan;  /* per-channel quantised cache: the KV head's d channel scales; else NULL */
    const float* v_chan;
} key_list;

/* Element c of row t of K (or V): the stored value, times its scale in a quantised
 * cache (the row's scale per token, channel c's per channel). */
static double key_elem(const key_list* keys, int is_v, int64_t t, int32_t c, int32_t d) {
    const int64_t base = keys->key_off[t];
    const double x = load_elem(is_v ? keys->v_base : keys->k_base, keys->dtype, base + c);
    const float* ch = is_v ? keys->v_chan : keys->k_chan;
    if (ch) return x * (double)ch[c];
    const float* sc = is_v ? keys->v_scale : keys->k_scale;
    return sc ? x * (double)sc[base / d] : x;
}

static void attend(const double* q, int32_t d, double scale, double slope, int64_t qpos,
                   const key_list* keys, double* scores, double* out) {
    for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
    if (keys->n_keys == 0) return;

    double m = -INFINITY;
    for (int64_t t = 0; t < keys->n_keys; ++t) {
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) dot += q[c] * key_elem(keys, 0, t, c, d);
        scores[t] = scale * dot - slope * (double)(qpos - (keys->kpos0 + t));
        if (scores[t] > m) m = scores[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < keys->n_keys; ++t) {
        const double w = exp(scores[t] - m);
        den += w;
        for (int32_t c = 0; c < d; ++c) out[c] += w * key_elem(keys, 1, t, c, d);
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
 * alibi_slopes optional fp32 [n_q]: ALiBi slope m_h of query head h, adding
 *              -m_h (ctx - 1 - t) to the score of position t (the query is
 *              position ctx - 1); NULL: no bias
 * window       0: all ctx positions; W > 0: only the last W of them, positions
 *              max(0, ctx - W) .. ctx - 1 (sliding-window attention, [IW]
 *              "KV Cache 的形状与增长", sliding-window item: the cache is bounded at
 *              W recent positions)
 * sel          optional list of n_sel (b, h) pairs; NULL means every (b, h)
 * out          [batch][n_q][head_dim] fp64 (or [n_sel][head_dim] with sel)
 * Quantised pools (kv_dtype E4M3 or INT8) come with k_scale / v_scale fp32:
 * per token (per_channel == 0) [num_blocks][n_kv][block_size], element = code *
 * the row's scale; per channel (per_channel == 1) [n_kv][head_dim], element c
 * of KV head g = code * scale[g][c]. q then has its own type q_dtype.
 * Unquantised pools take no scales and q_dtype == kv_dtype.
 * Returns 0, or -1 for invalid arguments or a block id outside the pool.
 */
static int decode_core(const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                       const float* k_scale, const float* v_scale, int per_channel,
                       int32_t batch, int32_t n_q, int32_t n_kv, int32_t head_dim,
                       int64_t num_blocks, int32_t block_size,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, double scale, int32_t window,
                       const float* alibi_slopes,
                       const int32_t* sel, int64_t n_sel, double* out, int32_t n_threads) {
    if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out) return -1;
    if (window < 0) return -1;
    if (elem_bytes_of(q_dtype) == 0 || is_quantised(q_dtype)) return -1;
    if (is_quantised(kv_dtype) ? (!k_scale || !v_scale) : (k_scale || v_scale || q_dtype != kv_dtype))
        return -1;
    if (elem_bytes_of(kv_dtype) == 0 || batch < 0 || n_q <= 0 || n_kv <= 0 || head_dim <= 0 ||
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
                qv[c] = load_elem(q, q_dtype, ((int64_t)b * n_q + h) * head_dim + c);
            const int32_t first = (window > 0 && ctx > window) ? ctx - window : 0;
            for (int32_t t = first; t < ctx; ++t) {
                /* block-table translation: logical t -> (physical block, offset) */
                const int64_t phys = block_table[(int64_t)b * max_blocks_per_seq + t / block_size];
                const int64_t off = t % block_size;
                offs[t - first] = ((phys * n_kv + g) * block_size + off) * head_dim;
            }
            /* the query is the newest position, ctx - 1 */
            key_list keys = {k_pool, v_pool, kv_dtype, offs, ctx - first, k_scale, v_scale, first, NULL, NULL};
            if (per_channel) {
                keys.k_scale = keys.v_scale = NULL;
                keys.k_chan = k_scale + (int64_t)g * head_dim;
                keys.v_chan = v_scale + (int64_t)g * head_dim;
            }
            const double slope = alibi_slopes ? (double)alibi_slopes[h] : 0.0;
            attend(qv, head_dim, scale, slope, (int64_t)ctx - 1, &keys, scores, out + it * head_dim);
        }
        free(qv);
        free(scores);
        free(offs);
    }
    return bad ? -1 : 0;
}

/* Decode over an unquantised cache, or a quantised one with per-token scales. */
int oracle_decode_ex(const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                     const float* k_scale, const float* v_scale,
                     int32_t batch, int32_t n_q, int32_t n_kv, int32_t head_dim,
                     int64_t num_blocks, int32_t block_size,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, double scale, int32_t window,
                     const float* alibi_slopes,
                     const int32_t* sel, int64_t n_sel, double* out, int32_t n_threads) {
    return decode_core(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale, v_scale, 0, batch, n_q, n_kv, head_dim,
                       num_blocks, block_size, block_table, max_blocks_per_seq, context_lens, scale, window,
                       alibi_slopes, sel, n_sel, out, n_threads);
}

/* Decode over a quantised cache with per-channel scales k_chan / v_chan [n_kv][head_dim]. */
int oracle_decode_channel(const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                          const float* k_chan, const float* v_chan,
                          int32_t batch, int32_t n_q, int32_t n_kv, int32_t head_dim,
                          int64_t num_blocks, int32_t block_size,
                          const int32_t* block_table, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, double scale, int32_t window,
                          const float* alibi_slopes,
                          const int32_t* sel, int64_t n_sel, double* out, int32_t n_threads) {
    if (!is_quantised(kv_dtype)) return -1;
    return decode_core(q, q_dtype, k_pool, v_pool, kv_dtype, k_chan, v_chan, 1, batch, n_q, n_kv, head_dim,
                       num_blocks, block_size, block_table, max_blocks_per_seq, context_lens, scale, window,
                       alibi_slopes, sel, n_sel, out, n_threads);
}

/* Decode over an unquantised cache: q and the pools share one type. */
int oracle_decode(const void* q, const void* k_pool, const void* v_pool, int dtype,
                  int32_t batch, int32_t n_q, int32_t n_kv, int32_t head_dim,
                  int64_t num_blocks, int32_t block_size,
                  const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, double scale, int32_t window,
                  const float* alibi_slopes,
                  const int32_t* sel, int64_t n_sel, double* out, int32_t n_threads) {
    if (is_quantised(dtype)) return -1;
    return oracle_decode_ex(q, dtype, k_pool, v_pool, dtype, NULL, NULL, batch, n_q, n_kv, head_dim,
                            num_blocks, block_size, block_table, max_blocks_per_seq, context_lens,
                            scale, window, alibi_slopes, sel, n_sel, out, n_threads);
}

/* ---- prefill over contiguous Q/K/V --------------------------------------- */

/*
 * q   [batch][seq_len][n_q][head_dim], k/v [batch][seq_len][n_kv][head_dim]
 * sel optional list of n_sel (b, h, i) triples; NULL means every (b, i, h)
 * out [batch][seq_len][n_q][head_dim] fp64 (or [n_sel][head_dim] with sel)
 * Row i attends to keys j <= i when causal, else to all seq_len keys; with
 * window W > 0 (causal only) to keys max(0, i - W + 1) .. i. alibi_slopes
 * (causal only; NULL: none) adds -m_h (i - j) to the scores of head h.
 */
int oracle_prefill(const void* q, const void* k, const void* v, int dtype,
                   int32_t batch, int32_t seq_len, int32_t n_q, int32_t n_kv,
                   int32_t head_dim, int32_t causal, double scale, int32_t window,
                   const float* alibi_slopes,
                   const int32_t* sel, int64_t n_sel, double* out, int32_t n_threads) {
    if (!q || !k || !v || !out) return -1;
    if (window < 0 || (window > 0 && !causal)) return -1;
    if (alibi_slopes && !causal) return -1;
    if (is_quantised(dtype)) return -1;
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
            key_list keys = {k, v, dtype, offs, n_keys - first, NULL, NULL, first, NULL, NULL};
            const double slope = alibi_slopes ? (double)alibi_slopes[h] : 0.0;
            attend(qv, head_dim, scale, slope, i, &keys, scores, out + it * head_dim);
        }
        free(qv);
        free(scores);
        free(offs);
    }
    return bad ? -1 : 0;
}

/* number of OpenMP threads a call with n_threads == 0 would use */
int oracle_max_threads(void) { return set_threads(0); }
