// decode_multi.hip -- decode of several new query rows per sequence on the matrix cores.
//
// Speculative verification decodes k new tokens of a sequence in one step: row r
// of the k sits at position ctx - k + r and attends to positions 0 .. that
// position (the causal mask of "注意力演进与推理流程", jerryiiii.gitbook.io,
// section 1.1, over a paged cache as in the vLLM concepts page, yyzxw.github.io;
// the walk-through "LLM 推理全过程的维度变化与核心公式", research.frankk.site,
// notes that verifying several drafted tokens at once is what turns decode into
// a matrix product). The G query heads of a KV head times the k rows are G*k
// rows that all read the same K/V, so they go through v_mfma_f32_32x32x16 as the
// N side of S^T = K Q^T and O^T = V^T P^T, and every K/V byte still leaves HBM
// once per step.
//
// Work decomposition
//  * grid = (partitions, n_kv * row groups, B); a row group is up to 32 virtual
//    rows v = r * G + j (token r, query head j of the group); lane l32 of every
//    wave owns row v = 32 * group + l32.
//  * The workgroup's 4 waves split the partition's blocks into contiguous runs
//    and stream them independently: each wave copies 32-key tiles (two cache
//    blocks) of K and V into its own double-buffered LDS ring with
//    global_load_lds_dwordx4 (no workgroup barrier until the end). Tiles use
//    the XOR chunk swizzle of mfma.h; V^T operands come from the row-major tile
//    through ds_read_b64_tr_b16.
//  * Online softmax in log2 units with the lazy running max of the prefill
//    kernel (one ballot per tile); for bf16, P = hi + lo (see mfma.h).
//  * The waves merge (m, l, O) through LDS; a workgroup that covers the whole
//    context writes the output, otherwise it writes the partition partials that
//    the decode reduce kernel merges with log-sum-exp weights.
//  * Sliding window: row r sees positions my_pos - W + 1 .. my_pos; the
//    partitions start at the block holding the earliest row's window start.
// Reductions depend only on logical positions, so relabelling physical blocks
// leaves every output bit unchanged.
#include "launch.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int BS = 16;            // tokens per cache block
constexpr int MR = 32;            // virtual rows per workgroup (the MFMA N side)
constexpr int BN = 32;            // keys per tile: two cache blocks
constexpr int WAVES = 4;          // waves per workgroup, each streaming its own run of blocks
constexpr int RING = 2;           // tiles in flight per wave
constexpr float TAU = 8.0f;       // rescale threshold (log2 units)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float M_FLOOR = -1e30f; // running-max start: finite, so 2^(s - m) of a masked s is 0

template <int D> struct MTile {
    static constexpr int ROWB = D * 2;             // bytes per K or V row
    static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
    static constexpr int BYTES = BN * ROWB;        // one K or V tile
    static constexpr int COPIES = BYTES / 1024;    // 1 KB copies per K (or V) tile
    static constexpr int ROWS_PER_COPY = 1024 / ROWB;
    static constexpr int SLOT = 2 * BYTES;         // K tile, then V tile
    static constexpr int WAVE_BYTES = RING * SLOT; // one wave's ring
    static_assert(BS % ROWS_PER_COPY == 0, "a copy stays inside one cache block");
    static_assert(WAVE_BYTES >= (MR * D + 2 * MR) * 4, "the merge reuses the wave's ring");
    static __device__ __forceinline__ int swz(int r) { return chunk_swizzle<CPR>(r); }
};

template <class E, int D>
__global__ __launch_bounds__(64 * WAVES, 1) void decode_multi_kernel(const DecodeArgs p) {
    using T = MTile<D>;
    using S = typename E::storage;
    constexpr int KK = D / 16;     // MFMA k-steps over the head dimension
    constexpr int MT = D / 32;     // 32-dim output tiles
    constexpr int OPS = 2 * T::COPIES;   // vector-memory operations per tile (K and V)
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int part = blockIdx.x;
    const int g = blockIdx.y / p.row_groups;
    const int rg = blockIdx.y % p.row_groups;
    const int b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int G = p.group;
    const int R = p.q_rows;
    const int v = rg * MR + l32;                   // this lane's virtual row
    const bool v_ok = v < G * R;
    const int r = v / G;                           // new-token index of the row
    const int jh = v % G;                          // query head within the group

    // Loads that do not need the context length go out before it is known, so
    // the start waits for one memory latency rather than a chain.
    const int blk0 = part * WAVES * p.blocks_per_wave + wave * p.blocks_per_wave;
    // Q^T operand: lane holds dims 16 kk + 8 half .. +8 of its row.
    // (Padding lanes past the G * R rows load row 0 and are zeroed below.)
    const int64_t qrow = v_ok ? ((int64_t)b * R + r) * p.n_q + (int64_t)g * G + jh : (int64_t)b * R * p.n_q;
    u32x4_t qreg[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const uint4 x = q_fold(*reinterpret_cast<const uint4*>(reinterpret_cast<const S*>(p.q) + qrow * D +
                                                               16 * kk + 8 * half), p.q_and, p.q_xor);
        qreg[kk] = u32x4_t{x.x, x.y, x.z, x.w};
    }
    // Lane k holds the physical id of logical block blk0 + k.
    int my_phys = 0;
    if (lane < p.blocks_per_wave && blk0 + lane < p.max_blocks)
        my_phys = p.block_table[(int64_t)b * p.max_blocks + blk0 + lane];

    // Context; a length past the block table's reach gives NaN rows.
    const int cap = p.max_blocks * BS;
    const int ctx_in = __builtin_amdgcn_readfirstlane(p.context_lens[b]);
    const bool ctx_bad = ctx_in > cap;
    const int ctx = (ctx_in < 0 || ctx_bad) ? 0 : ctx_in;
    const int nblk = (ctx + BS - 1) / BS;
    // Sliding window: partitions start at the block holding the first position
    // any row attends to; earlier table entries are never read.
    const int first = window_first(ctx, R, p.window);
    const int fb = first / BS;
    const int bpp = WAVES * p.blocks_per_wave;
    const int nparts = nblk > fb ? (nblk - fb + bpp - 1) / bpp : 1;
    if (part >= nparts) return;  // uniform over the workgroup
    const int wb0 = blk0 + fb;   // first logical block of this wave
    if (fb > 0) {                // uniform: the hoisted table read was for blocks from 0
        my_phys = 0;
        if (lane < p.blocks_per_wave && wb0 + lane < p.max_blocks)
            my_phys = p.block_table[(int64_t)b * p.max_blocks + wb0 + lane];
    }
    const int nb = max(0, min(nblk - wb0, p.blocks_per_wave));
    const int wave_end = min((wb0 + nb) * BS, ctx);    // keys of this wave: [wb0 * 16, wave_end)
    const int my_pos = ctx - R + r;                      // this row sees keys <= my_pos
    const bool phys_bad = __any(lane < nb && (my_phys < 0 || my_phys >= p.num_blocks));
    // The copies below are invisible to the compiler's wait counting: have it
    // wait for q and the block ids here, before the first copy.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (!v_ok) qreg[kk] = u32x4_t{0u, 0u, 0u, 0u};
        asm volatile("" : : "v"(qreg[kk]));
    }
    asm volatile("" : : "v"(my_phys));

    const int ntile = (nb + 1) / 2;
    char* ring = smem + wave * T::WAVE_BYTES;
    const uint32_t ring_lds = lds_addr(ring);
    const int64_t block_bytes = (int64_t)p.n_kv * BS * T::ROWB;
    const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)g * BS * T::ROWB;
    const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)g * BS * T::ROWB;
    const int last_local = (wave_end - 1) / BS - wb0;    // last block of the run holding a key

    // Tile t of the run (keys wb0 * 16 + 32 t ..) into ring slot t % RING. Copy c
    // holds rows c * ROWS_PER_COPY .. of the tile; a row past the run reads the
    // run's last key instead (its score is masked and its V row stays finite).
    const bool once = p.row_groups == 1;   // no other workgroup reads these tiles: non-temporal
    auto issue = [&](int t) {
        const uint32_t dst = ring_lds + (t % RING) * T::SLOT;
#pragma unroll
        for (int c = 0; c < T::COPIES; ++c) {
            const int row0 = c * T::ROWS_PER_COPY;                     // first row of the copy
            const int lb = min(2 * t + row0 / BS, last_local);        // uniform block index
            const int64_t phys = __builtin_amdgcn_readlane(my_phys, lb);
            const int off = c * 1024 + 16 * lane;
            const int row = off / T::ROWB;
            const int chunk = ((off % T::ROWB) / 16) ^ T::swz(row);
            const int key = min(wb0 * BS + 32 * t + row, wave_end - 1);
            const int64_t src = phys * block_bytes + (int64_t)(key % BS) * T::ROWB + chunk * 16;
            copy_to_lds16(kbase + src, dst + c * 1024, once);
            copy_to_lds16(vbase + src, dst + T::BYTES + c * 1024, once);
        }
    };

    f32x16_t o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16_t{};
    float m_run = M_FLOOR;
    float l_run = 0.f;
    // ALiBi: this row's head slope in log2 units; with it, scores are formed in log2
    // units before the max (c2 = 1), else scaled inside it.
    const bool alibi = p.alibi != nullptr;   // uniform
    const float al2 = alibi ? p.alibi[(int64_t)g * G + jh] * LOG2E : 0.f;
    const float c2 = alibi ? 1.f : p.scale_log2;
    const int ksw = T::swz(l32);
    const int g16 = lane >> 4, r16 = lane & 15;
    const int vkey = 4 * half + r16 / 4;               // + 16 jg + 8 tt
    const int vchunk = 2 * (g16 & 1) + (r16 & 3) / 2;  // + 4 mt
    const int vbyte = 8 * (r16 & 1);
    const int row_lim = min(my_pos, wave_end - 1);     // last key this row may use in this run
    // First key this row may use: its window start (no lower limit without a window).
    const int row_lo = p.window > 0 ? my_pos - p.window + 1 : 0;
    const int lo_max = p.window > 0 ? ctx - p.window : 0;   // the last row's window start

    if (!phys_bad && ntile > 0) {
        const int pre = min(RING, ntile);
        for (int t = 0; t < pre; ++t) issue(t);
        for (int t = 0; t < ntile; ++t) {
            if (t + 1 < ntile) wait_vmcnt<OPS>();   // tile t landed, t + 1 may be in flight
            else wait_vmcnt<0>();
            const char* kl = ring + (t % RING) * T::SLOT;
            lds_char_t* vl = (lds_char_t*)(kl + T::BYTES);
            const int key0 = wb0 * BS + 32 * t;

            f32x16_t sc = f32x16_t{};
            const char* krow = kl + l32 * T::ROWB;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint4 a = *reinterpret_cast<const uint4*>(krow + ((2 * kk + half) ^ ksw) * 16);
                sc = Mfma<E>::run(u32x4_t{a.x, a.y, a.z, a.w}, qreg[kk], sc);
            }
            if (alibi) {   // - m_h log2(e) (my_pos - key)
                const float b0 = al2 * (float)(key0 + half * 4 - my_pos);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sc[i] = fmaf(sc[i], p.scale_log2, fmaf(al2, (float)((i / 4) * 8 + (i % 4)), b0));
            }
            // Mask keys past the run, past this row's position or before its window.
            if (key0 + BN > wave_end || key0 + BN - 1 > ctx - R || key0 < lo_max) {   // uniform
                const int lim = row_lim - key0;
                const int lo = row_lo - key0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = (i / 4) * 8 + half * 4 + (i % 4);
                    sc[i] = (key > lim || key < lo) ? -INFINITY : sc[i];
                }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[i]);
            {
                float a2, b2;
                pair32(tmax, a2, b2);
                tmax = fmaxf(a2, b2) * c2;   // scale > 0, so scaling commutes with the max
            }
            if (__any(tmax > m_run + TAU)) {
                const float m_new = fmaxf(m_run, tmax);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
            }
            u32x4_t ph[2], pl[2];
            float lsum = 0.f;
#pragma unroll
            for (int jg = 0; jg < 2; ++jg) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[8 * jg + 2 * w], c2, -m_run));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[8 * jg + 2 * w + 1], c2, -m_run));
                    hw[w] = Mfma<E>::pack(p0, p1);
                    if constexpr (Mfma<E>::kSplit)
                        lw[w] = Mfma<E>::pack(p0 - Mfma<E>::lo_of(hw[w]), p1 - Mfma<E>::hi_of(hw[w]));
                    lsum += p0 + p1;
                }
                ph[jg] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
                if constexpr (Mfma<E>::kSplit) pl[jg] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
            }
            l_run += lsum;
#pragma unroll
            for (int jg = 0; jg < 2; ++jg) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    uint32_t av[4];
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        const int key = jg * 16 + 8 * tt + vkey;
                        const int pos = ((4 * mt + vchunk) ^ T::swz(key)) * 16 + vbyte;
                        const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vl + key * T::ROWB + pos));
                        av[2 * tt] = __builtin_bit_cast(uint2, x).x;
                        av[2 * tt + 1] = __builtin_bit_cast(uint2, x).y;
                    }
                    const u32x4_t a = u32x4_t{av[0], av[1], av[2], av[3]};
                    o[mt] = Mfma<E>::run(a, ph[jg], o[mt]);
                    if constexpr (Mfma<E>::kSplit) o[mt] = Mfma<E>::run(a, pl[jg], o[mt]);
                }
            }
            lds_reads_done();                     // the slot is free again
            if (t + RING < ntile) issue(t + RING);
        }
    }

    // Lanes l and l ^ 32 covered complementary keys of the same row.
    {
        float a2, b2;
        pair32(l_run, a2, b2);
        l_run = a2 + b2;
    }
    // Publish (m, l, O) in the wave's ring: O [row][dim], then m [row], l [row].
    float* mine = reinterpret_cast<float*>(ring);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            mine[l32 * D + mt * 32 + (i / 4) * 8 + half * 4 + (i % 4)] = o[mt][i];
    if (half == 0) {
        mine[MR * D + l32] = m_run;
        mine[MR * D + MR + l32] = phys_bad ? NAN : l_run;
    }
    __syncthreads();

    // Merge the waves: thread -> (row, 16 consecutive dims).
    constexpr int PER = MR * D / (64 * WAVES);
    const int row = threadIdx.x / (D / PER);
    const int d0 = (threadIdx.x % (D / PER)) * PER;
    const int vr = rg * MR + row;
    if (vr >= G * R) return;
    const float* slots = reinterpret_cast<const float*>(smem);
    constexpr int WF = T::WAVE_BYTES / 4;
    float mw[WAVES], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        mw[w] = slots[w * WF + MR * D + row];
        M = fmaxf(M, mw[w]);
    }
    float L = 0.f, A[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) A[e] = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - M);
        L = fmaf(f, slots[w * WF + MR * D + MR + row], L);
#pragma unroll
        for (int e = 0; e < PER; ++e) A[e] = fmaf(f, slots[w * WF + row * D + d0 + e], A[e]);
    }
    const int rr = vr / G, jj = vr % G;
    const int64_t orow = ((int64_t)b * R + rr) * p.n_q + (int64_t)g * G + jj;
    if (nparts == 1) {
        const float inv = ctx_bad ? NAN : (L == 0.f ? 0.f : 1.f / L);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const float x = A[e] * inv;
            if (p.out_f32)
                reinterpret_cast<float*>(p.out)[orow * D + d0 + e] = x;
            else
                reinterpret_cast<S*>(p.out)[orow * D + d0 + e] = narrow<E>(x);
        }
    } else {
        const int64_t pi = orow * p.nparts_max + part;
        if (d0 == 0) {
            p.ws_m[pi] = M;
            p.ws_l[pi] = L;
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) p.ws_acc[pi * D + d0 + e] = A[e];
    }
}

template <class E, int D> hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    const size_t lds = (size_t)WAVES * MTile<D>::WAVE_BYTES;
    static const hipError_t opt_in = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_multi_kernel<E, D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (opt_in != hipSuccess) return opt_in;
    const dim3 grid(a.nparts_max, a.n_kv * a.row_groups, a.batch);
    hipLaunchKernelGGL((decode_multi_kernel<E, D>), grid, dim3(64 * WAVES), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_multi(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s) {
    if (a.waves_tok != WAVES || a.blocks_per_wave < 1 || a.blocks_per_wave > 64) return hipErrorInvalidValue;
    hipError_t err;
    if (e == Elem::BF16 && head_dim == 128) err = launch_typed<BF16, 128>(a, s);
    else if (e == Elem::BF16 && head_dim == 64) err = launch_typed<BF16, 64>(a, s);
    else if (e == Elem::F16 && head_dim == 128) err = launch_typed<F16, 128>(a, s);
    else if (e == Elem::F16 && head_dim == 64) err = launch_typed<F16, 64>(a, s);
    else return hipErrorNotSupported;
    if (err != hipSuccess || a.nparts_max <= 1) return err;
    DecodeArgs m = a;
    m.n_q = a.n_q * a.q_rows;   // the reduce kernel's rows: (b, r, h) in [B][q_rows][n_q] order
    return launch_decode_reduce(m, e, head_dim, s);
}

}  // namespace pa
