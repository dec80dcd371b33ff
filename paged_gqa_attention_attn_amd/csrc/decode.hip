// decode.hip -- paged GQA decode attention for gfx950 (CDNA4, wave64).
//
// One query token per sequence attends to its cached context, which lives in
// 16-token blocks reached through a block table (vLLM concepts page,
// yyzxw.github.io, decode attention over K<=t, V<=t and the block-table
// paragraph; "LLM 推理全过程的维度变化与核心公式", research.frankk.site, "Decode
// 阶段维度流转": no causal mask in decode). Query head h reads KV head
// floor(h / G) ("注意力演进与推理流程", jerryiiii.gitbook.io, section 3.1), and
// the G heads of one KV head are served by the same workgroup, so every K/V
// byte leaves HBM once per step.
//
// Work decomposition
//  * grid = (partitions, n_kv * head-slice groups, batch). A partition is a
//    run of consecutive logical blocks; its waves split it further.
//  * A wave owns `gw` query heads and a contiguous run of blocks. Each 16-token
//    block's 4 KB K tile and 4 KB V tile (bf16, d = 128) are copied into the
//    wave's own LDS ring with global_load_lds_dwordx4: every copy instruction
//    moves one contiguous 1 KB run, and the copies cost no registers, so a
//    wave keeps R blocks in flight while it computes on the current one.
//  * Lane layout for compute: lane = slot * LPT + c. The LPT lanes of a token
//    slot read 16-byte chunks c and c + LPT of the token row from LDS. Scores
//    come from packed dot products (v_dot2 for bf16/f16) and a DPP sum over
//    the LPT lanes.
//  * Softmax runs online (running max m and denominator l per head, the
//    Flash Attention statistics of the walk-through page's "工程优化怎么嵌进公式"
//    section) in log2 units. The running max only moves when some score of
//    the block exceeds it by more than TAU (a one-instruction ballot test), so
//    the wave-wide max and the accumulator rescale are rare; the result is
//    exact either way because acc, l and m stay consistent.
//  * The waves of a workgroup combine through LDS; a workgroup that covers the
//    whole context writes the output, otherwise it writes (m, l, acc) partials
//    and the reduce kernel merges them with log-sum-exp weights (Flash
//    Decoding, same section).
//  * Sliding window (the walk-through's KV-cache section, sliding-window item,
//    which bounds the cache at W recent positions): the query at ctx - 1 sees
//    ctx - W .. ctx - 1. Partitions start at the block holding ctx - W, and
//    positions of that block before it are masked like those past ctx.
// Every reduction order depends only on logical positions, never on physical
// block ids, so relabelling the pool leaves every output bit unchanged.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int BS = 16;         // tokens per cache block
constexpr float TAU = 8.0f;    // rescale threshold (log2 units): p <= 2^TAU between rescales
constexpr float LOG2E = 1.4426950408889634f;
constexpr int MAX_WAVES = 8;   // waves per workgroup
constexpr int MIN_WAVES_PER_SIMD = 3;  // register budget: at most 168 VGPRs per lane

template <int D, int GW> struct WaveSlot {
    static constexpr int floats = GW * D + 2 * GW;   // acc[GW][D], m[GW], l[GW]
};

template <class E, int D, int GW, int R>
__global__ __launch_bounds__(64 * MAX_WAVES, MIN_WAVES_PER_SIMD) void decode_partition_kernel(const DecodeArgs p) {
    using S = typename E::storage;
    constexpr int EB = (int)sizeof(S);
    constexpr int ROW = D * EB;            // bytes per token row
    constexpr int LPT = ROW / 32;          // lanes per token slot (two 16-byte chunks each)
    constexpr int TPP = 64 / LPT;          // token slots per wave
    constexpr int NT = BS / TPP;           // tokens per lane per block
    constexpr int EPC = 16 / EB;           // elements per chunk
    constexpr int EPL = 2 * EPC;           // elements per lane per token
    constexpr int SLOT = WaveSlot<D, GW>::floats;
    constexpr int TILE = BS * ROW;         // bytes of one (block, KV head) K or V tile
    constexpr int NQ = TILE / 1024;        // 1 KB wave copies per tile
    constexpr int OPS = 2 * NQ;            // vector-memory operations per block (K and V)
    constexpr int RING = R * 2 * TILE;     // bytes of this wave's LDS ring
    static_assert(LPT == 4 || LPT == 8 || LPT == 16, "row must split into 4, 8 or 16 lanes");
    static_assert(NT >= 1 && NT * TPP == BS, "block must split evenly over token slots");
    static_assert(TILE % 1024 == 0, "tiles move in whole 1 KB wave copies");
    static_assert(OPS * (R - 1) < 64, "outstanding copies must fit the vmcnt counter");
    static_assert(SLOT * 4 <= RING, "the merge slot reuses the wave's ring");

    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int part = blockIdx.x;
    const int g = blockIdx.y / p.hsg;
    const int hsgi = blockIdx.y % p.hsg;
    const int b = blockIdx.z;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int hs = wave % p.hs_wg;
    const int wt = wave / p.hs_wg;
    const int slot = lane / LPT;
    const int c = lane % LPT;

    // Every load that does not need the context length is issued before it is
    // known, so the start of the kernel waits for one memory latency, not a chain.
    const int hwg0 = g * p.group + hsgi * p.hs_wg * GW;  // first query head of the workgroup
    const int h0 = hwg0 + hs * GW;                        // first query head of this wave
    const int blk0 = part * p.waves_tok * p.blocks_per_wave + wt * p.blocks_per_wave;
    uint4 qv[GW][2];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
        const uint4* qrow =
            reinterpret_cast<const uint4*>((const char*)p.q + (int64_t)(b * p.n_q + h0 + hh) * ROW);
        qv[hh][0] = q_fold(qrow[c], p.q_and, p.q_xor);
        qv[hh][1] = q_fold(qrow[c + LPT], p.q_and, p.q_xor);
    }
    // Lane k holds the physical id of logical block blk0 + k (the table row is
    // read up to the wave's share or the row's end, whatever the context).
    int my_phys = 0;
    if (lane < p.blocks_per_wave && blk0 + lane < p.max_blocks)
        my_phys = p.block_table[(int64_t)b * p.max_blocks + blk0 + lane];

    // Fused append: the wave that owns the block holding position ctx - 1 patches
    // the new K/V row into its LDS copy of that tile, and one wave per
    // (sequence, KV head) writes the row to the cache slot.
    constexpr int CH = ROW / 16;   // 16-byte chunks per row: lanes [0, CH) K, [CH, 2 CH) V
    static_assert(2 * CH <= 64, "a K row and a V row fit in one wave");
    const bool fused = p.new_slots != nullptr;
    const int64_t new_slot = fused ? p.new_slots[b] : -1;
    uint4 new_row = make_uint4(0, 0, 0, 0);
    if (fused && lane < 2 * CH) {
        const char* src = (const char*)(lane < CH ? p.k_new : p.v_new) +
                          ((int64_t)b * p.n_kv + g) * ROW + (lane % CH) * 16;
        new_row = *reinterpret_cast<const uint4*>(src);
    }

    // Context of this sequence. A length past the block table's reach cannot be
    // served without reading out of bounds: that sequence's rows become NaN.
    const int cap = p.max_blocks * BS;
    const int ctx_in = __builtin_amdgcn_readfirstlane(p.context_lens[b]);
    const bool ctx_bad = ctx_in > cap;
    const int ctx = (ctx_in < 0 || ctx_bad) ? 0 : ctx_in;
    const int nblk = (ctx + BS - 1) / BS;
    // Sliding window: the partitions start at the block holding the first
    // attended position; the table entries of earlier blocks are never read.
    const int first = window_first(ctx, 1, p.window);
    const int fb = first / BS;
    const int bpp = p.waves_tok * p.blocks_per_wave;
    const int nparts = nblk > fb ? (nblk - fb + bpp - 1) / bpp : 1;
    if (part >= nparts) return;  // uniform over the workgroup
    const int wb0 = blk0 + fb;   // first logical block of this wave
    if (fb > 0) {                // uniform: the hoisted table read was for blocks from 0
        my_phys = 0;
        if (lane < p.blocks_per_wave && wb0 + lane < p.max_blocks)
            my_phys = p.block_table[(int64_t)b * p.max_blocks + wb0 + lane];
    }
    const int nb = max(0, min(nblk - wb0, p.blocks_per_wave));
    // ALiBi: each head's slope in log2 units; with it, scores are formed in log2
    // units before the max (c2 = 1), else scaled inside it.
    const bool alibi = p.alibi != nullptr;   // uniform
    float al2[GW];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) al2[hh] = alibi ? p.alibi[h0 + hh] * LOG2E : 0.f;
    const float c2 = alibi ? 1.f : p.scale_log2;
    const bool phys_bad = __any(lane < nb && (my_phys < 0 || my_phys >= p.num_blocks));

    const bool slot_ok = new_slot >= 0 && new_slot < (int64_t)p.num_blocks * BS;
    const int last_blk = ctx > 0 ? (ctx - 1) / BS : -1;
    const bool patch_here = fused && slot_ok && last_blk >= wb0 && last_blk < wb0 + nb;
    const bool writer = fused && slot_ok && part == nparts - 1 && hsgi == 0 && wave == 0;

    float m_run[GW], l_run[GW], acc[GW][EPL];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
        m_run[hh] = -INFINITY;
        l_run[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
    }

    char* ring = smem + wave * RING;
    const int64_t block_bytes = (int64_t)p.n_kv * TILE;
    const char* ksrc = (const char*)p.k_cache + (int64_t)g * TILE + lane * 16;
    const char* vsrc = (const char*)p.v_cache + (int64_t)g * TILE + lane * 16;
    const uint32_t off0 = slot * ROW + c * 16;          // chunk c of token `slot`
    const uint32_t off1 = off0 + LPT * 16;              // chunk c + LPT

    // Copy block i's K and V tiles into ring slot i % R (8 KB for bf16, d = 128).
    const uint32_t ring_lds = lds_addr(ring);
    // Tiles no other wave or workgroup reads (one head slice per KV head) stream
    // with the non-temporal hint.
    const bool once = p.hsg == 1 && p.hs_wg == 1;
    auto issue = [&](int i) {
        const int64_t phys = __builtin_amdgcn_readlane(my_phys, i);
        const uint32_t dst = ring_lds + (i % R) * 2 * TILE;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq)
            copy_to_lds16(ksrc + phys * block_bytes + qq * 1024, dst + qq * 1024, once);
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq)
            copy_to_lds16(vsrc + phys * block_bytes + qq * 1024, dst + TILE + qq * 1024, once);
    };

    // q and the block ids have landed before the ring copies start, so the
    // compiler never needs a full vmcnt(0) wait (which would drain the ring)
    // to reach them inside the loop.
    wait_vmcnt<0>();

    if (!phys_bad && nb > 0) {
        const int pre = min(R, nb);
        for (int i = 0; i < pre; ++i) issue(i);
        for (int i = 0; i < nb; ++i) {
            // Block i has landed once at most (blocks issued after it) * OPS copies are pending.
            const int ahead = min(R - 1, nb - 1 - i);
            if constexpr (R >= 4) {
                if (ahead >= 3) wait_vmcnt<3 * OPS>();
            }
            if constexpr (R >= 3) {
                if (ahead == 2) wait_vmcnt<2 * OPS>();
            }
            if (ahead == 1) wait_vmcnt<OPS>();
            if (ahead == 0) wait_vmcnt<0>();

            const char* base = ring + (i % R) * 2 * TILE;
            if (patch_here && wb0 + i == last_blk) {  // uniform: the new token's block
                if (lane < 2 * CH) {
                    char* row = ring + (i % R) * 2 * TILE + (lane < CH ? 0 : TILE) +
                                ((ctx - 1) % BS) * ROW + (lane % CH) * 16;
                    *reinterpret_cast<uint4*>(row) = new_row;
                }
            }
            uint4 kc[NT][2], vc[NT][2];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                kc[t][0] = *reinterpret_cast<const uint4*>(base + t * TPP * ROW + off0);
                kc[t][1] = *reinterpret_cast<const uint4*>(base + t * TPP * ROW + off1);
                vc[t][0] = *reinterpret_cast<const uint4*>(base + TILE + t * TPP * ROW + off0);
                vc[t][1] = *reinterpret_cast<const uint4*>(base + TILE + t * TPP * ROW + off1);
            }
            lds_reads_done();
            // The slot is free again: start the copy R blocks ahead.
            if (i + R < nb) issue(i + R);

            const int pos0 = (wb0 + i) * BS;
            float s[GW][NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
#pragma unroll
                for (int hh = 0; hh < GW; ++hh) {
                    float d = chunk_dot<E>(kc[t][0], qv[hh][0], 0.f);
                    d = chunk_dot<E>(kc[t][1], qv[hh][1], d);
                    s[hh][t] = group_sum<LPT>(d);   // raw q.k; scaled inside exp2 below
                }
            }
            if (alibi) {   // - m_h log2(e) (ctx - 1 - pos) for the key at pos
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float dist = (float)(pos0 + slot + t * TPP - (ctx - 1));
#pragma unroll
                    for (int hh = 0; hh < GW; ++hh) s[hh][t] = fmaf(s[hh][t], p.scale_log2, al2[hh] * dist);
                }
            }
            // Last block: positions >= ctx hold unrelated bytes. First block under a
            // window: positions before `first` are outside it.
            if (pos0 + BS > ctx || pos0 < first) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int pos = pos0 + slot + t * TPP;
                    if (pos >= ctx || pos < first) {
#pragma unroll
                        for (int hh = 0; hh < GW; ++hh) s[hh][t] = -INFINITY;
                        vc[t][0] = make_uint4(0, 0, 0, 0);
                        vc[t][1] = make_uint4(0, 0, 0, 0);
                    }
                }
            }

            float vf[NT][EPL];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                widen<E>(vc[t][0], &vf[t][0]);
                widen<E>(vc[t][1], &vf[t][EPC]);
            }

#pragma unroll
            for (int hh = 0; hh < GW; ++hh) {
                float bm = s[hh][0];
#pragma unroll
                for (int t = 1; t < NT; ++t) bm = fmaxf(bm, s[hh][t]);
                bm *= c2;   // c2 > 0, so scaling commutes with the max
                // The running max moves only when some score in the wave passes it by
                // more than TAU (log2 units); the wave-wide max is taken only then.
                if (__any(bm > m_run[hh] + TAU)) {
                    bm = stride_reduce<LPT, true>(bm);
                    const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - bm);
                    l_run[hh] *= alpha;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
                    m_run[hh] = bm;
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float pr = __builtin_amdgcn_exp2f(fmaf(s[hh][t], c2, -m_run[hh]));
                    l_run[hh] += pr;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pr, vf[t][e], acc[hh][e]);
                }
            }
        }
    }

    // Sum l over the wave's token slots, and reduce-scatter acc over them: each
    // lane ends with M fully summed values (head, dimension pairs) to publish.
    constexpr int LOG_LPT = LPT == 4 ? 2 : LPT == 8 ? 3 : 4;
    constexpr int NV = GW * EPL;
    using RS = ReduceScatter<NV, LOG_LPT>;
    constexpr int M = RS::M;
    static_assert(M >= 1, "at least one value per lane after the reduce-scatter");
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) l_run[hh] = stride_reduce<LPT, false>(l_run[hh]);
    float flat[NV];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh)
#pragma unroll
        for (int e = 0; e < EPL; ++e) flat[hh * EPL + e] = acc[hh][e];
    float mine_vals[M];
    RS::run(flat, mine_vals, lane);

    float* mine = reinterpret_cast<float*>(smem + wave * RING);
#pragma unroll
    for (int k = 0; k < M; ++k) {
        const int kg = slot * M + k;       // index into flat[]
        const int hh = kg / EPL;
        const int e = kg % EPL;
        const int dim = e < EPC ? c * EPC + e : D / 2 + c * EPC + (e - EPC);
        mine[hh * D + dim] = mine_vals[k];
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) {
            mine[GW * D + hh] = phys_bad ? 0.f : m_run[hh];
            mine[GW * D + GW + hh] = phys_bad ? NAN : l_run[hh];
        }
    }
    __syncthreads();

    // Merge the waves that split the partition, per query head and dimension.
    const int nh = p.hs_wg * GW;
    for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x) {
        const int hl = idx / D;
        const int e = idx % D;
        const int hsl = hl / GW;
        const int hh = hl % GW;
        const float* slots = reinterpret_cast<const float*>(smem);
        constexpr int RING_F = RING / 4;
        // All reads are issued before any use, so the merge costs one LDS
        // round trip rather than one per wave.
        float mw[MAX_WAVES], lw[MAX_WAVES], aw[MAX_WAVES];
#pragma unroll
        for (int w = 0; w < MAX_WAVES; ++w) {
            const bool live = w < p.waves_tok;
            const float* ws = slots + (live ? w * p.hs_wg + hsl : 0) * RING_F;
            mw[w] = live ? ws[GW * D + hh] : -INFINITY;
            lw[w] = live ? ws[GW * D + GW + hh] : 0.f;
            aw[w] = live ? ws[hh * D + e] : 0.f;
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < MAX_WAVES; ++w) M = fmaxf(M, mw[w]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < MAX_WAVES; ++w) {
                const float f = __builtin_amdgcn_exp2f(mw[w] - M);
                L = fmaf(f, lw[w], L);
                A = fmaf(f, aw[w], A);
            }
        }
        const int h = hwg0 + hl;
        const int64_t row = (int64_t)b * p.n_q + h;
        if (nparts == 1) {
            float o = (L == 0.f) ? 0.f : A * __builtin_amdgcn_rcpf(L);
            if (ctx_bad) o = NAN;
            if (p.out_f32)
                reinterpret_cast<float*>(p.out)[row * D + e] = o;
            else
                reinterpret_cast<S*>(p.out)[row * D + e] = narrow<E>(o);
        } else {
            const int64_t pi = row * p.nparts_max + part;
            if (e == 0) {
                p.ws_m[pi] = M;
                p.ws_l[pi] = L;
            }
            p.ws_acc[pi * D + e] = A;
        }
    }

    // The fused append's cache write goes last: a store counts in vmcnt, so an
    // earlier one would be waited on by the ring's first full wait.
    if (writer && lane < 2 * CH) {
        char* dst = (char*)(lane < CH ? p.k_cache_w : p.v_cache_w) +
                    (((new_slot / BS) * p.n_kv + g) * BS + new_slot % BS) * ROW + (lane % CH) * 16;
        *reinterpret_cast<uint4*>(dst) = new_row;
    }
}

// Merge the partitions of each (sequence, query head) with log-sum-exp weights:
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
template <class E, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const DecodeArgs p) {
    using S = typename E::storage;
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int cap = p.max_blocks * BS;
    const int ctx_in = p.context_lens[b];
    const int ctx = (ctx_in < 0 || ctx_in > cap) ? 0 : ctx_in;
    const int nblk = (ctx + BS - 1) / BS;
    const int fb = window_first(ctx, p.q_rows, p.window) / BS;   // as in the partition kernels
    const int bpp = p.waves_tok * p.blocks_per_wave;
    const int nparts = nblk > fb ? (nblk - fb + bpp - 1) / bpp : 1;
    if (nparts <= 1) return;  // the partition kernel wrote the output itself

    const int64_t row = (int64_t)b * p.n_q + h;
    const float* pm = p.ws_m + row * p.nparts_max;
    const float* pl = p.ws_l + row * p.nparts_max;
    const float* pa = p.ws_acc + row * p.nparts_max * D;
    float M = -INFINITY;
    for (int i = 0; i < nparts; ++i) M = fmaxf(M, pm[i]);
    const int e = threadIdx.x;
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
        for (int i = 0; i < nparts; ++i) {
            const float f = __builtin_amdgcn_exp2f(pm[i] - M);
            L = fmaf(f, pl[i], L);
            A = fmaf(f, pa[(int64_t)i * D + e], A);
        }
    }
    const float o = (L == 0.f) ? 0.f : A / L;
    if (p.out_f32)
        reinterpret_cast<float*>(p.out)[row * D + e] = o;
    else
        reinterpret_cast<S*>(p.out)[row * D + e] = narrow<E>(o);
}

template <class E, int D, int GW, int R> hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    const int waves = a.hs_wg * a.waves_tok;
    const dim3 grid(a.nparts_max, a.n_kv * a.hsg, a.batch);
    const size_t lds = (size_t)waves * R * 2 * BS * D * sizeof(typename E::storage);
    static bool lds_opt_in = [] {
        return hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_partition_kernel<E, D, GW, R>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    }();
    (void)lds_opt_in;
    hipLaunchKernelGGL((decode_partition_kernel<E, D, GW, R>), grid, dim3(64 * waves), lds, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.nparts_max <= 1) return err;
    hipLaunchKernelGGL((decode_reduce_kernel<E, D>), dim3(a.n_q, a.batch), dim3(D), 0, s, a);
    return hipGetLastError();
}

template <class E, int D, int R> hipError_t launch_gw(const DecodeArgs& a, hipStream_t s) {
    switch (a.gw) {
    case 1: return launch_typed<E, D, 1, R>(a, s);
    case 2: return launch_typed<E, D, 2, R>(a, s);
    case 4: return launch_typed<E, D, 4, R>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <class E, int D> hipError_t launch_ring(const DecodeArgs& a, hipStream_t s) {
    switch (a.ring) {
    case 1: return launch_gw<E, D, 1>(a, s);
    case 2: return launch_gw<E, D, 2>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <class E> hipError_t launch_dim(const DecodeArgs& a, int head_dim, hipStream_t s) {
    switch (head_dim) {
    case 64: return launch_ring<E, 64>(a, s);
    case 128: return launch_ring<E, 128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s) {
    const dim3 grid(a.n_q, a.batch);
    if (e == Elem::BF16 && head_dim == 128) hipLaunchKernelGGL((decode_reduce_kernel<BF16, 128>), grid, dim3(128), 0, s, a);
    else if (e == Elem::BF16 && head_dim == 64) hipLaunchKernelGGL((decode_reduce_kernel<BF16, 64>), grid, dim3(64), 0, s, a);
    else if (e == Elem::F16 && head_dim == 128) hipLaunchKernelGGL((decode_reduce_kernel<F16, 128>), grid, dim3(128), 0, s, a);
    else if (e == Elem::F16 && head_dim == 64) hipLaunchKernelGGL((decode_reduce_kernel<F16, 64>), grid, dim3(64), 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s) {
    if (a.hs_wg * a.waves_tok > MAX_WAVES || a.hs_wg < 1 || a.waves_tok < 1) return hipErrorInvalidValue;
    if (a.q_rows != 1 || a.window < 0) return hipErrorInvalidValue;   // the reduce kernel reads q_rows
    if (a.mfma) return launch_decode_mfma(a, e, head_dim, s);
    switch (e) {
    case Elem::F32: return launch_dim<F32>(a, head_dim, s);
    case Elem::BF16: return launch_dim<BF16>(a, head_dim, s);
    case Elem::F16: return launch_dim<F16>(a, head_dim, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
