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
//  * A wave owns `gw` query heads and a contiguous run of blocks. Per 16-token
//    block it loads the 4 KB K tile and the 4 KB V tile straight into
//    registers (two 16-byte loads per lane per token it owns), with the next
//    block's loads issued before the current block is computed.
//  * Lane layout inside a block: lane = slot * LPT + c. The LPT lanes of a
//    token slot each hold 16-byte chunks c and c + LPT of the token row, so
//    every load instruction of the wave reads whole 16-byte-aligned
//    half-rows. Scores come from packed dot products (v_dot2 for bf16/f16)
//    and a DPP sum over the LPT lanes.
//  * Softmax runs online (running max m and denominator l per head, the
//    Flash Attention statistics of the walk-through page's "工程优化怎么嵌进公式"
//    section) in log2 units. The running max only moves when a block's max
//    exceeds it by more than TAU, so the accumulator is rarely rescaled; the
//    result is exact either way because acc, l and m stay consistent.
//  * The waves of a workgroup combine through LDS; a workgroup that covers the
//    whole context writes the output, otherwise it writes (m, l, acc) partials
//    and the reduce kernel merges them with log-sum-exp weights (Flash
//    Decoding, same section).
// Every reduction order depends only on logical positions, never on physical
// block ids, so relabelling the pool leaves every output bit unchanged.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int BS = 16;         // tokens per cache block
constexpr float TAU = 8.0f;    // rescale threshold (log2 units): p <= 2^TAU between rescales
constexpr int MAX_WAVES = 8;   // waves per workgroup

template <int D, int GW> struct WaveSlot {
    static constexpr int floats = GW * D + 2 * GW;   // acc[GW][D], m[GW], l[GW]
};

template <class E, int D, int GW>
__global__ __launch_bounds__(64 * MAX_WAVES) void decode_partition_kernel(const DecodeArgs p) {
    using S = typename E::storage;
    constexpr int EB = (int)sizeof(S);
    constexpr int ROW = D * EB;            // bytes per token row
    constexpr int LPT = ROW / 32;          // lanes per token slot (two 16-byte chunks each)
    constexpr int TPP = 64 / LPT;          // token slots per wave
    constexpr int NT = BS / TPP;           // tokens per lane per block
    constexpr int EPC = 16 / EB;           // elements per chunk
    constexpr int EPL = 2 * EPC;           // elements per lane per token
    constexpr int SLOT = WaveSlot<D, GW>::floats;
    static_assert(LPT == 4 || LPT == 8 || LPT == 16, "row must split into 4, 8 or 16 lanes");
    static_assert(NT >= 1 && NT * TPP == BS, "block must split evenly over token slots");

    extern __shared__ float smem[];

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

    // Context of this sequence. A length past the block table's reach cannot be
    // served without reading out of bounds: that sequence's rows become NaN.
    const int cap = p.max_blocks * BS;
    const int ctx_in = p.context_lens[b];
    const bool ctx_bad = ctx_in > cap;
    const int ctx = (ctx_in < 0 || ctx_bad) ? 0 : ctx_in;
    const int nblk = (ctx + BS - 1) / BS;
    const int bpp = p.waves_tok * p.blocks_per_wave;
    const int nparts = nblk > 0 ? (nblk + bpp - 1) / bpp : 1;
    if (part >= nparts) return;  // uniform over the workgroup

    const int blk0 = part * bpp + wt * p.blocks_per_wave;
    const int nb = max(0, min(nblk - blk0, p.blocks_per_wave));
    const int hwg0 = g * p.group + hsgi * p.hs_wg * GW;  // first query head of the workgroup
    const int h0 = hwg0 + hs * GW;                        // first query head of this wave

    // Lane k holds the physical id of logical block blk0 + k.
    int my_phys = 0;
    if (lane < nb) my_phys = p.block_table[(int64_t)b * p.max_blocks + blk0 + lane];
    const bool phys_bad = __any(lane < nb && (my_phys < 0 || my_phys >= p.num_blocks));

    uint4 qv[GW][2];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
        const uint4* qrow =
            reinterpret_cast<const uint4*>((const char*)p.q + (int64_t)(b * p.n_q + h0 + hh) * ROW);
        qv[hh][0] = qrow[c];
        qv[hh][1] = qrow[c + LPT];
    }

    float m_run[GW], l_run[GW], acc[GW][EPL];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
        m_run[hh] = -INFINITY;
        l_run[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
    }

    const char* kbase = (const char*)p.k_cache;
    const char* vbase = (const char*)p.v_cache;
    const int64_t tile_bytes = (int64_t)BS * ROW;              // one (block, KV head) tile
    const int64_t block_bytes = (int64_t)p.n_kv * tile_bytes;
    const int64_t off0 = (int64_t)slot * ROW + c * 16;          // chunk c of token `slot`
    const int64_t off1 = off0 + LPT * 16;                       // chunk c + LPT

    if (!phys_bad && nb > 0) {
        uint4 kc[NT][2], vc[NT][2], kn[NT][2], vn[NT][2];
        auto load = [&](int i, uint4 (&kr)[NT][2], uint4 (&vr)[NT][2]) {
            const int phys = __builtin_amdgcn_readlane(my_phys, i);
            const int64_t tile = (int64_t)phys * block_bytes + (int64_t)g * tile_bytes;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int64_t o = tile + (int64_t)t * TPP * ROW;
                kr[t][0] = *reinterpret_cast<const uint4*>(kbase + o + off0);
                kr[t][1] = *reinterpret_cast<const uint4*>(kbase + o + off1);
                vr[t][0] = *reinterpret_cast<const uint4*>(vbase + o + off0);
                vr[t][1] = *reinterpret_cast<const uint4*>(vbase + o + off1);
            }
        };

        load(0, kc, vc);
        for (int i = 0; i < nb; ++i) {
            if (i + 1 < nb) load(i + 1, kn, vn);

            const int pos0 = (blk0 + i) * BS;
            float s[GW][NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
#pragma unroll
                for (int hh = 0; hh < GW; ++hh) {
                    float d = chunk_dot<E>(kc[t][0], qv[hh][0], 0.f);
                    d = chunk_dot<E>(kc[t][1], qv[hh][1], d);
                    s[hh][t] = group_sum<LPT>(d) * p.scale_log2;
                }
            }
            if (pos0 + BS > ctx) {  // last block: positions >= ctx hold unrelated bytes
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (pos0 + slot + t * TPP >= ctx) {
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
                bm = stride_reduce<LPT, true>(bm);
                if (bm > m_run[hh] + TAU) {  // wave-uniform
                    const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - bm);
                    l_run[hh] *= alpha;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
                    m_run[hh] = bm;
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float pr = __builtin_amdgcn_exp2f(s[hh][t] - m_run[hh]);
                    l_run[hh] += pr;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pr, vf[t][e], acc[hh][e]);
                }
            }

#pragma unroll
            for (int t = 0; t < NT; ++t) {
                kc[t][0] = kn[t][0];
                kc[t][1] = kn[t][1];
                vc[t][0] = vn[t][0];
                vc[t][1] = vn[t][1];
            }
        }
    }

    // Sum l and acc over the wave's token slots; lanes of slot 0 publish to LDS.
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
        l_run[hh] = stride_reduce<LPT, false>(l_run[hh]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] = stride_reduce<LPT, false>(acc[hh][e]);
    }
    float* mine = smem + wave * SLOT;
    if (lane < LPT) {
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                mine[hh * D + c * EPC + e] = acc[hh][e];
                mine[hh * D + (c + LPT) * EPC + e] = acc[hh][EPC + e];
            }
        }
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
        float M = -INFINITY;
        for (int w = 0; w < p.waves_tok; ++w)
            M = fmaxf(M, smem[(w * p.hs_wg + hsl) * SLOT + GW * D + hh]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
            for (int w = 0; w < p.waves_tok; ++w) {
                const float* ws = smem + (w * p.hs_wg + hsl) * SLOT;
                const float f = __builtin_amdgcn_exp2f(ws[GW * D + hh] - M);
                L = fmaf(f, ws[GW * D + GW + hh], L);
                A = fmaf(f, ws[hh * D + e], A);
            }
        }
        const int h = hwg0 + hl;
        const int64_t row = (int64_t)b * p.n_q + h;
        if (nparts == 1) {
            float o = (L == 0.f) ? 0.f : A / L;
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
    const int bpp = p.waves_tok * p.blocks_per_wave;
    const int nparts = nblk > 0 ? (nblk + bpp - 1) / bpp : 1;
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

template <class E, int D, int GW> hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    const int waves = a.hs_wg * a.waves_tok;
    const dim3 grid(a.nparts_max, a.n_kv * a.hsg, a.batch);
    const size_t lds = (size_t)waves * WaveSlot<D, GW>::floats * sizeof(float);
    hipLaunchKernelGGL((decode_partition_kernel<E, D, GW>), grid, dim3(64 * waves), lds, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.nparts_max <= 1) return err;
    hipLaunchKernelGGL((decode_reduce_kernel<E, D>), dim3(a.n_q, a.batch), dim3(D), 0, s, a);
    return hipGetLastError();
}

template <class E, int D> hipError_t launch_gw(const DecodeArgs& a, hipStream_t s) {
    switch (a.gw) {
    case 1: return launch_typed<E, D, 1>(a, s);
    case 2: return launch_typed<E, D, 2>(a, s);
    case 4: return launch_typed<E, D, 4>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <class E> hipError_t launch_dim(const DecodeArgs& a, int head_dim, hipStream_t s) {
    switch (head_dim) {
    case 64: return launch_gw<E, 64>(a, s);
    case 128: return launch_gw<E, 128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, Elem e, int head_dim, hipStream_t s) {
    if (a.hs_wg * a.waves_tok > MAX_WAVES || a.hs_wg < 1 || a.waves_tok < 1) return hipErrorInvalidValue;
    switch (e) {
    case Elem::F32: return launch_dim<F32>(a, head_dim, s);
    case Elem::BF16: return launch_dim<BF16>(a, head_dim, s);
    case Elem::F16: return launch_dim<F16>(a, head_dim, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
