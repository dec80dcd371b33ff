// decode_mfma.hip -- paged GQA decode attention on the gfx950 matrix cores.
//
// Same problem and work decomposition as decode.hip (one query token per
// sequence over its 16-token cache blocks, reached through the block table; the
// G query heads of one KV head served by one workgroup so that every K/V byte
// leaves HBM once per step; vLLM concepts page, yyzxw.github.io, decode over
// K<=t, V<=t and the block-table paragraph; "注意力演进与推理流程",
// jerryiiii.gitbook.io, section 3.1 for the head grouping), but the two
// contractions of each block run on the matrix cores instead of the VALU:
//
//  * The G query vectors of a KV head against a block's 16 keys are a real
//    [16 x d] . [d x G] product: S^T = K q^T with v_mfma_f32_16x16x32 (M = the
//    block's 16 keys, N = up to 16 query heads, K = head dims). The query heads
//    of the workgroup are the B operand, loaded once.
//  * O^T += V^T P^T with v_mfma_f32_16x16x16 (M = 16 head dims per tile, N = the
//    heads, K = the block's 16 keys). The S^T accumulator already holds, in each
//    lane, the 4 keys that the P^T operand needs there, so P never moves between
//    lanes. V^T comes from the row-major V tile through ds_read_b64_tr_b16,
//    which hands lane j of a 16-lane group element j % 4 of the 8-byte chunk
//    fetched by lane 4e + j / 4 (e = 0..3).
//  * bf16 probabilities are split into bf16 hi + lo parts and both multiply V
//    (P rounded to 8 bits alone errs by ~0.4% on contexts of a few tokens);
//    the two parts share one v_mfma_f32_16x16x32_bf16, stacked along k with V^T
//    repeated, which issues at twice the rate of two 16x16x16 products. f16
//    keeps 11 bits in one part.
//  * Measured on the 8B-shaped step, the VALU form of these products costs
//    about 7% of the step (its time grows linearly with the VALU instruction
//    count, and the shader clock drops under it); here the VALU only runs the
//    softmax.
//
// Multi-row decode (several new tokens per sequence, draft verification) runs
// here too when the G * NR (head, row) pairs of a KV head are a multiple of 4 up
// to 16: the pairs are the MFMA columns, the row at position ctx - NR + r sees
// keys up to itself, so masks become per column on the blocks that need them.
//
// Tiles reach LDS by global_load_lds_dwordx4 as in decode.hip, each row stored
// unpadded with its 16-byte chunk c at position c ^ swz(row) (the copy picks
// each lane's source chunk so that its destination stays 16 * lane), which
// keeps both operand reads free of bank conflicts. Rows outside the attended
// range are zeroed in LDS before the V^T read: a matrix product would turn the
// 0 * NaN of an unused slot into NaN.
//
// Online softmax in log2 units with the lazy running max of decode.hip; the
// waves of a workgroup merge through LDS, and split contexts write partials for
// decode.hip's log-sum-exp reduce kernel (Flash Decoding, "LLM 推理全过程的维度
// 变化与核心公式", research.frankk.site, "工程优化怎么嵌进公式"). Every
// reduction order depends on logical positions only.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int BS = 16;          // tokens per cache block
constexpr float TAU = 8.0f;     // rescale threshold (log2 units)
constexpr int MAX_WAVES = 8;    // waves per workgroup
constexpr float M_FLOOR = -1e30f; // running-max start (finite)
constexpr float LOG2E = 1.4426950408889634f;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <class E> struct Mfma16;
template <> struct Mfma16<BF16> {
    static __device__ __forceinline__ f32x4_t qk(u32x4_t a, u32x4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                         __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
    }
};
template <> struct Mfma16<F16> {
    static __device__ __forceinline__ f32x4_t qk(u32x4_t a, u32x4_t b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    }
};

template <int D, int HW, int R> struct Layout {
    static constexpr int ROW = D * 2;                 // bytes per token row
    static constexpr int CPR = ROW / 16;              // 16-byte chunks per row
    static constexpr int TILE = BS * ROW;             // one (block, KV head) K or V tile
    static constexpr int NQ = TILE / 1024;            // 1 KB wave copies per tile
    static constexpr int OPS = 2 * NQ;                // vector-memory operations per block
    static constexpr int RING = R * 2 * TILE;         // bytes of a wave's ring
    static constexpr int PITCH = D + 4;               // merge-slot floats per head (padded)
    static constexpr int SLOT = HW * PITCH + 2 * HW;  // acc[HW][PITCH], m[HW], l[HW]
    static constexpr int WAVE_BYTES = ((RING > SLOT * 4 ? RING : SLOT * 4) + 15) / 16 * 16;
    static __device__ __forceinline__ int swz(int r) { return chunk_swizzle<CPR>(r); }
};

template <class E, int D, int HW, int R>
__global__ __launch_bounds__(64 * MAX_WAVES, 2) void decode_mfma_kernel(const DecodeArgs p) {
    using L = Layout<D, HW, R>;
    using S = typename E::storage;
    constexpr int ROW = L::ROW, TILE = L::TILE, NQ = L::NQ, OPS = L::OPS;
    constexpr int KK = D / 32;    // S^T k-steps over the head dimension
    constexpr int MT = D / 16;    // 16-dim O^T tiles
    constexpr int CH = ROW / 16;  // chunks per row: lanes [0, CH) K, [CH, 2 CH) V of a new row
    static_assert(HW == 4 || HW == 8 || HW == 16, "heads per workgroup fill 4, 8 or 16 MFMA columns");
    static_assert(TILE % 1024 == 0 && 1024 % ROW == 0, "tiles move in whole 1 KB copies of whole rows");
    static_assert(OPS * (R - 1) < 64, "outstanding copies must fit the vmcnt counter");
    static_assert(2 * CH <= 64, "a K row and a V row fit in one wave");

    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int part = blockIdx.x;
    const int g = blockIdx.y / p.hsg;
    const int hsgi = blockIdx.y % p.hsg;
    const int b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;    // MFMA column: (head, row) pair hsgi * HW + col
    const int grp = lane >> 4;    // 16-lane group

    // MFMA column col holds (head, row) pair v = hsgi * HW + col of the KV head's
    // G * NR pairs: new-token row v / G of the step's NR (1 outside multi-row
    // decode), query head g * G + v % G. qo_row(v) is its row of q and of out.
    const int G = p.group, NR = p.q_rows;
    auto qo_row = [&](int v) { return ((int64_t)b * NR + v / G) * p.n_q + (int64_t)g * G + v % G; };
    const int v_col = hsgi * HW + (col < HW ? col : 0);

    // Context-independent loads first (q, the table row, the new K/V row), so the
    // start waits for one memory latency rather than a chain.
    const int blk0 = part * p.waves_tok * p.blocks_per_wave + wave * p.blocks_per_wave;
    u32x4_t qreg[KK];
    {
        // Columns past the workgroup's HW pairs stay zero (their scores are 0 and
        // their outputs are never stored).
        const char* qrow = (const char*)p.q + qo_row(v_col) * ROW;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            // B operand of S^T: dims 32 kk + 8 grp .. +8 of column col's q row (the same
            // dims the K operand below takes, which is all the product needs).
            uint4 v = make_uint4(0, 0, 0, 0);
            if (col < HW) v = q_fold(*reinterpret_cast<const uint4*>(qrow + (32 * kk + 8 * grp) * 2), p.q_and, p.q_xor);
            qreg[kk] = u32x4_t{v.x, v.y, v.z, v.w};
        }
    }
    int my_phys = 0;
    if (lane < p.blocks_per_wave && blk0 + lane < p.max_blocks)
        my_phys = p.block_table[(int64_t)b * p.max_blocks + blk0 + lane];

    const bool fused = p.new_slots != nullptr;
    const int64_t new_slot = fused ? p.new_slots[b] : -1;
    uint4 new_row = make_uint4(0, 0, 0, 0);
    if (fused && lane < 2 * CH) {
        const char* src = (const char*)(lane < CH ? p.k_new : p.v_new) +
                          ((int64_t)b * p.n_kv + g) * ROW + (lane % CH) * 16;
        new_row = *reinterpret_cast<const uint4*>(src);
    }

    const int cap = p.max_blocks * BS;
    const int ctx_in = __builtin_amdgcn_readfirstlane(p.context_lens[b]);
    const bool ctx_bad = ctx_in > cap;
    const int ctx = (ctx_in < 0 || ctx_bad) ? 0 : ctx_in;
    const int nblk = (ctx + BS - 1) / BS;
    const int first = window_first(ctx, NR, p.window);   // the earliest position any row sees
    // This column's row sees positions col_lo .. col_hi (causal among the new rows).
    const int col_hi = ctx - NR + v_col / G;
    const int col_lo = p.window > 0 ? col_hi - p.window + 1 : 0;
    // ALiBi: the column's head slope in log2 units; with it, scores are formed in
    // log2 units before the max (c2 = 1), else scaled inside it.
    const bool alibi = p.alibi != nullptr;   // uniform
    const float al2 = alibi ? p.alibi[(int64_t)g * G + v_col % G] * LOG2E : 0.f;
    const float c2 = alibi ? 1.f : p.scale_log2;
    const int fb = first / BS;
    const int bpp = p.waves_tok * p.blocks_per_wave;
    const int nparts = nblk > fb ? (nblk - fb + bpp - 1) / bpp : 1;
    if (part >= nparts) return;  // uniform over the workgroup
    const int wb0 = blk0 + fb;
    if (fb > 0) {
        my_phys = 0;
        if (lane < p.blocks_per_wave && wb0 + lane < p.max_blocks)
            my_phys = p.block_table[(int64_t)b * p.max_blocks + wb0 + lane];
    }
    const int nb = max(0, min(nblk - wb0, p.blocks_per_wave));
    const bool phys_bad = __any(lane < nb && (my_phys < 0 || my_phys >= p.num_blocks));

    const bool slot_ok = new_slot >= 0 && new_slot < (int64_t)p.num_blocks * BS;
    const int last_blk = ctx > 0 ? (ctx - 1) / BS : -1;
    const bool patch_here = fused && slot_ok && last_blk >= wb0 && last_blk < wb0 + nb;
    const bool writer = fused && slot_ok && part == nparts - 1 && hsgi == 0 && wave == 0;

    char* ring = smem + wave * L::WAVE_BYTES;
    const uint32_t ring_lds = lds_addr(ring);
    const int64_t block_bytes = (int64_t)p.n_kv * TILE;
    // Copy qq of a tile fills LDS bytes [1024 qq, +1 KB); lane l writes 16 l of that,
    // i.e. row r = (1024 qq + 16 l) / ROW at chunk position pp, which holds source
    // chunk pp ^ swz(r).
    uint32_t src_off[NQ];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
        const int off = qq * 1024 + 16 * lane;
        const int r = off / ROW;
        src_off[qq] = r * ROW + (((off % ROW) / 16) ^ L::swz(r)) * 16;
    }
    const char* kbase = (const char*)p.k_cache + (int64_t)g * TILE;
    const char* vbase = (const char*)p.v_cache + (int64_t)g * TILE;
    // With one head slice per KV head, no other workgroup reads this wave's tiles:
    // they stream with the non-temporal hint.
    const bool once = p.hsg == 1;
    auto issue = [&](int i) {
        const int64_t phys = __builtin_amdgcn_readlane(my_phys, i);
        const uint32_t dst = ring_lds + (i % R) * 2 * TILE;
        const char* kb = kbase + phys * block_bytes;
        const char* vb = vbase + phys * block_bytes;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) copy_to_lds16(kb + src_off[qq], dst + qq * 1024, once);
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) copy_to_lds16(vb + src_off[qq], dst + TILE + qq * 1024, once);
    };

    // Lane-constant operand offsets inside a ring slot.
    uint32_t k_off[KK];      // K operand: row col, dims 32 kk + 8 grp .. +8
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k_off[kk] = col * ROW + (((4 * kk + grp) ^ L::swz(col)) * 16);
    const int vrow = 4 * grp + (col >> 2);          // V^T operand: this lane fetches row vrow,
    const int vsw = L::swz(vrow);                   // dims 16 t + 4 (col % 4) .. +4
    const int vbyte = 8 * (col & 1);
    const int vchunk = (col & 3) >> 1;

    f32x4_t o[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Running max (log2 units) of column col. It starts finite: with several rows a
    // block can hold no key that some column attends, and 2^(s - m) of a masked s
    // must then be 0, not 2^(-inf + inf).
    float m_run = M_FLOOR;
    float l_run = 0.f;         // this lane's share of its denominator (keys 4 grp .. +4 of each block)

    // q and the new row have landed before the ring starts: were the compiler to
    // wait for them inside the loop, its vmcnt(0) would also drain the ring.
    wait_vmcnt<0>();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : : "v"(qreg[kk]));
    asm volatile("" : : "v"(new_row.x), "v"(new_row.y), "v"(new_row.z), "v"(new_row.w));

    if (!phys_bad && nb > 0) {
        const int pre = min(R, nb);
        for (int i = 0; i < pre; ++i) issue(i);
        for (int i = 0; i < nb; ++i) {
            const int ahead = min(R - 1, nb - 1 - i);
            if constexpr (R >= 3) {
                if (ahead >= 2) wait_vmcnt<2 * OPS>();
            }
            if constexpr (R >= 2) {
                if (ahead == 1) wait_vmcnt<OPS>();
            }
            if (ahead == 0) wait_vmcnt<0>();

            char* base = ring + (i % R) * 2 * TILE;
            const int pos0 = (wb0 + i) * BS;
            if (patch_here && wb0 + i == last_blk) {   // uniform: the new token's block
                if (lane < 2 * CH) {
                    const int r = (ctx - 1) % BS;
                    char* dst = base + (lane < CH ? 0 : TILE) + r * ROW + (((lane % CH) ^ L::swz(r)) * 16);
                    *reinterpret_cast<uint4*>(dst) = new_row;
                }
            }
            // Some key of the block is outside some column's range (uniform).
            const bool edge = pos0 + BS - 1 > ctx - NR || (p.window > 0 && pos0 < ctx - p.window);
            if (edge) {
                // Zero the V rows outside [first, ctx) (whole rows: the swizzle does not matter).
#pragma unroll
                for (int k = 0; k < BS * CH / 64; ++k) {
                    const int idx = k * 64 + lane;
                    const int r = idx / CH;
                    const int pos = pos0 + r;
                    if (pos >= ctx || pos < first)
                        *reinterpret_cast<uint4*>(base + TILE + r * ROW + (idx % CH) * 16) = make_uint4(0, 0, 0, 0);
                }
            }
            u32x4_t ka[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint4 v = *reinterpret_cast<const uint4*>(base + k_off[kk]);
                ka[kk] = u32x4_t{v.x, v.y, v.z, v.w};
            }
            uint2 va[MT];
            lds_char_t* vt = (lds_char_t*)(base + TILE + vrow * ROW);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int pos = ((2 * t + vchunk) ^ vsw) * 16 + vbyte;
                const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + pos));
                va[t] = __builtin_bit_cast(uint2, v);
            }
            lds_reads_done();
            if (i + R < nb) issue(i + R);

            // S^T: s[j] = q_col . K[key 4 grp + j] (raw; scaled inside exp2).
            f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s = Mfma16<E>::qk(ka[kk], qreg[kk], s);
            if (alibi) {   // s = q.k scale log2(e) - m_h log2(e) (i - j), key j = pos0 + 4 grp + j'
                const float b0 = al2 * (float)(pos0 + 4 * grp - col_hi);
#pragma unroll
                for (int j = 0; j < 4; ++j) s[j] = fmaf(s[j], p.scale_log2, fmaf(al2, (float)j, b0));
            }
            if (edge) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int pos = pos0 + 4 * grp + j;
                    s[j] = (pos > col_hi || pos < col_lo) ? -INFINITY : s[j];
                }
            }
            float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * c2;   // c2 > 0
            // The running max moves only when some score passes it by more than TAU;
            // the column max over the four 16-lane groups is taken only then.
            if (__any(bm > m_run + TAU)) {
                const float m_new = fmaxf(m_run, stride_reduce<16, true>(bm));
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < MT; ++t) o[t] *= alpha;
                m_run = m_new;
            }
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pr[j] = __builtin_amdgcn_exp2f(fmaf(s[j], c2, -m_run));
                l_run += pr[j];
            }
            // P^T operand: keys 4 grp .. +4 of column col, exactly where S^T put them.
            const uint2 ph = make_uint2(Mfma<E>::pack(pr[0], pr[1]), Mfma<E>::pack(pr[2], pr[3]));
            if constexpr (Mfma<E>::kSplit) {
                // hi and lo parts stacked along k of one 16x16x32 product (twice the
                // rate of two 16x16x16 products): k slots 8 grp + j hold key 4 grp + j % 4,
                // part j / 4, in both operands.
                const uint2 pl = make_uint2(Mfma<E>::pack(pr[0] - Mfma<E>::lo_of(ph.x), pr[1] - Mfma<E>::hi_of(ph.x)),
                                            Mfma<E>::pack(pr[2] - Mfma<E>::lo_of(ph.y), pr[3] - Mfma<E>::hi_of(ph.y)));
                const u32x4_t pb = u32x4_t{ph.x, ph.y, pl.x, pl.y};
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    o[t] = Mfma16<E>::qk(u32x4_t{va[t].x, va[t].y, va[t].x, va[t].y}, pb, o[t]);
            } else {
#pragma unroll
                for (int t = 0; t < MT; ++t) o[t] = Mfma16<E>::pv(va[t], ph, o[t]);
            }
        }
    }

    // The denominator of column col is spread over the four 16-lane groups; o
    // holds dims 16 t + 4 grp + i of that head, each in exactly one lane.
    l_run = stride_reduce<16, false>(l_run);
    float* mine = reinterpret_cast<float*>(ring);
    if (col < HW) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
            *reinterpret_cast<f32x4_t*>(mine + col * L::PITCH + 16 * t + 4 * grp) = o[t];
        if (grp == 0) {
            mine[HW * L::PITCH + col] = phys_bad ? 0.f : m_run;
            mine[HW * L::PITCH + HW + col] = phys_bad ? NAN : l_run;
        }
    }
    __syncthreads();

    // Merge the waves that split the partition, per query head and dimension.
    for (int idx = threadIdx.x; idx < HW * D; idx += blockDim.x) {
        const int hl = idx / D;
        const int e = idx % D;
        float mw[MAX_WAVES], lw[MAX_WAVES], aw[MAX_WAVES];
#pragma unroll
        for (int w = 0; w < MAX_WAVES; ++w) {
            const bool live = w < p.waves_tok;
            const float* ws = reinterpret_cast<const float*>(smem + (live ? w : 0) * L::WAVE_BYTES);
            mw[w] = live ? ws[HW * L::PITCH + hl] : -INFINITY;
            lw[w] = live ? ws[HW * L::PITCH + HW + hl] : 0.f;
            aw[w] = live ? ws[hl * L::PITCH + e] : 0.f;
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < MAX_WAVES; ++w) M = fmaxf(M, mw[w]);
        float Lsum = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < MAX_WAVES; ++w) {
                const float f = __builtin_amdgcn_exp2f(mw[w] - M);
                Lsum = fmaf(f, lw[w], Lsum);
                A = fmaf(f, aw[w], A);
            }
        }
        const int64_t row = qo_row(hsgi * HW + hl);
        if (nparts == 1) {
            float o1 = (Lsum == 0.f) ? 0.f : A * __builtin_amdgcn_rcpf(Lsum);
            if (ctx_bad) o1 = NAN;
            if (p.out_f32)
                reinterpret_cast<float*>(p.out)[row * D + e] = o1;
            else
                reinterpret_cast<S*>(p.out)[row * D + e] = narrow<E>(o1);
        } else {
            const int64_t pi = row * p.nparts_max + part;
            if (e == 0) {
                p.ws_m[pi] = M;
                p.ws_l[pi] = Lsum;
            }
            p.ws_acc[pi * D + e] = A;
        }
    }

    // The fused append's cache write goes last (a store counts in vmcnt).
    if (writer && lane < 2 * CH) {
        char* dst = (char*)(lane < CH ? p.k_cache_w : p.v_cache_w) +
                    (((new_slot / BS) * p.n_kv + g) * BS + new_slot % BS) * ROW + (lane % CH) * 16;
        *reinterpret_cast<uint4*>(dst) = new_row;
    }
}

template <class E, int D, int HW, int R> hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    const size_t lds = (size_t)a.waves_tok * Layout<D, HW, R>::WAVE_BYTES;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    static const hipError_t opt_in = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_mfma_kernel<E, D, HW, R>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (opt_in != hipSuccess) return opt_in;
    const dim3 grid(a.nparts_max, a.n_kv * a.hsg, a.batch);
    hipLaunchKernelGGL((decode_mfma_kernel<E, D, HW, R>), grid, dim3(64 * a.waves_tok), lds, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.nparts_max <= 1) return err;
    DecodeArgs m = a;
    m.n_q = a.n_q * a.q_rows;   // the reduce kernel's rows: (b, r, h) in [B][q_rows][n_q] order
    return launch_decode_reduce(m, std::is_same<E, BF16>::value ? Elem::BF16 : Elem::F16, D, s);
}

template <class E, int D, int R> hipError_t launch_hw(const DecodeArgs& a, hipStream_t s) {
    switch (a.gw) {
    case 4: return launch_typed<E, D, 4, R>(a, s);
    case 8: return launch_typed<E, D, 8, R>(a, s);
    case 16: return launch_typed<E, D, 16, R>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <class E, int D> hipError_t launch_ring(const DecodeArgs& a, hipStream_t s) {
    switch (a.ring) {
    case 1: return launch_hw<E, D, 1>(a, s);
    case 2: return launch_hw<E, D, 2>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s) {
    if (a.hs_wg != 1 || a.waves_tok < 1 || a.waves_tok > MAX_WAVES) return hipErrorInvalidValue;
    if (a.q_rows < 1 || a.window < 0) return hipErrorInvalidValue;
    // Several new rows per sequence: their pairs must fill whole slices of gw
    // columns, and the fused append serves single-row steps only.
    if (a.q_rows > 1 && ((a.group * a.q_rows) % a.gw != 0 || a.new_slots != nullptr)) return hipErrorInvalidValue;
    if (e == Elem::BF16 && head_dim == 128) return launch_ring<BF16, 128>(a, s);
    if (e == Elem::BF16 && head_dim == 64) return launch_ring<BF16, 64>(a, s);
    if (e == Elem::F16 && head_dim == 128) return launch_ring<F16, 128>(a, s);
    if (e == Elem::F16 && head_dim == 64) return launch_ring<F16, 64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace pa
