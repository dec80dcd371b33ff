// attn_f32.hip -- fp32 attention of several query rows per sequence on the fp32
// matrix cores: contiguous prefill (causal or full), chunked prefill over the
// paged cache, and multi-row decode (the same computation with q_rows rows).
//
// What is computed: softmax(q K^T * scale + M) V per query row ("注意力演进与推理流程",
// jerryiiii.gitbook.io, section 1.1, causal mask M; section 3.1, query head h reads
// KV group floor(h / G)), over keys reached through a block table for the paged
// forms (the vLLM concepts page, yyzxw.github.io) with the rows of a sequence
// aligned at the bottom right of its context (the inference walk-through,
// research.frankk.site, chunked prefill keeps the formula unchanged), the online
// softmax of Flash Attention (same walk-through, "工程优化怎么嵌进公式"), and the
// sliding window and ALiBi bias of its KV-cache and position-encoding sections.
//
// Work decomposition
//  * A "virtual row" v = i * G + j is query row i, query head j of a KV group; the
//    grid is (row tiles of 64 virtual rows, n_kv, batch), heaviest causal
//    tiles first. Each wave owns 16 virtual rows, which are the 16 columns of
//    v_mfma_f32_16x16x4_f32: S^T = K Q^T and O^T = V^T P^T. In both products a
//    lane keeps its own row (column l % 16) and four keys or four dims
//    (4 (l / 16) + r), so the probabilities of S^T are already the B operand of
//    O^T and the per-row softmax statistics never leave the lane's 16-lane column
//    (two cross-lane steps reduce over the 16 keys of a tile).
//  * The workgroup streams 16-key tiles (one cache block) of K and V through a
//    double-buffered LDS stage: each thread loads its share of tile t + 1 into
//    registers while tile t is multiplied, one barrier per tile.
//  * Masking is by select, never by arithmetic: key positions past the context,
//    before a row's window or after its position (causal) get a score of -inf;
//    V rows the workgroup does not own (past the context, before the earliest
//    window) are zeroed in LDS so that unwritten slots cannot leak NaN.
//  * A context past the block table's reach, or a block id outside the pool among
//    the blocks any row of the sequence reads, makes every row of the sequence NaN.
// fp32 throughout: products and sums in fp32, exp2 on the VALU; the result is
// within 1e-5 (norm-wise relative) of the exact one for the test shapes.
#include "launch.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int BK = 16;            // keys per tile (one cache block)
constexpr int ROWS = 16;          // virtual rows per wave (MFMA columns)
constexpr int WAVES = 4;          // waves past the last row only stage tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float M_FLOOR = -1e30f; // running-max start: finite, so 2^(s - m) of a masked s is 0

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D> struct F32Tile {
    static constexpr int STRIDE = D + 4;             // floats per LDS row (bank spread)
    static constexpr int MAT = BK * STRIDE;          // one K or V tile
    static constexpr int BUF = 2 * MAT;              // K then V
    static constexpr int LDS = 2 * BUF * 4;          // double-buffered, bytes
    static constexpr int F4 = BK * D / 4;            // float4s per tile and matrix
};

template <int D, bool PAGED>
__global__ __launch_bounds__(64 * WAVES) void attn_f32_kernel(const PrefillArgs p) {
    using T = F32Tile<D>;
    constexpr int NT = D / 16;    // 16-dim steps of S^T, 16-dim output blocks of O^T
    extern __shared__ __attribute__((aligned(16))) float fsm[];

    constexpr int nthreads = 64 * WAVES;
    constexpr int tile_rows = ROWS * WAVES;
    const int tile = gridDim.x - 1 - blockIdx.x;      // the longest causal tiles first
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;                        // this lane's row within the wave
    const int quad = lane >> 4;                       // its keys / dims 4 quad .. 4 quad + 3
    const int G = p.group;
    const int R = p.seq_len;                          // query rows per sequence
    const int VR = R * G;

    // Keys of the sequence and the position of query row 0.
    const int S_len = R;
    int ctx = S_len;
    bool bad = false;
    if constexpr (PAGED) {
        ctx = load_uniform(p.context_lens + b);
        if (ctx < 0 || ctx > p.max_blocks * BK) {
            bad = ctx > 0;
            ctx = 0;
        }
        // Every block any row of the sequence reads must lie in the pool.
        const int nblk = (ctx + BK - 1) / BK;
        for (int j = window_first(ctx, R, p.window) / BK + (int)threadIdx.x; j < nblk; j += nthreads) {
            const int phys = p.block_table[(int64_t)b * p.max_blocks + j];
            bad = bad || phys < 0 || phys >= p.num_blocks;
        }
        bad = __syncthreads_or(bad);
    }
    const int qbase = ctx - R;

    // This lane's virtual row.
    const int v0 = tile * tile_rows;
    const int v = v0 + wave * ROWS + col;
    const bool v_ok = v < VR;
    const int qi = v_ok ? v / G : 0;
    const int h = g * G + (v_ok ? v % G : 0);
    const int pos = qbase + qi;
    const int64_t orow = ((int64_t)b * R + qi) * p.n_q + h;
    float* out = static_cast<float*>(p.out) + orow * D;

    if (bad) {   // uniform over the workgroup
        if (v_ok)
#pragma unroll
            for (int k = 0; k < NT; ++k)
                *reinterpret_cast<float4*>(out + 16 * k + 4 * quad) = make_float4(NAN, NAN, NAN, NAN);
        return;
    }

    // Keys the workgroup's rows attend to: [k_lo, k_hi).
    const int v_last = min(v0 + tile_rows, VR) - 1;
    const int pos_first = qbase + v0 / G;
    const int pos_last = qbase + v_last / G;
    int k_lo = 0, k_hi = ctx;
    if (p.causal) {
        k_hi = min(ctx, pos_last + 1);
        if (p.window > 0) k_lo = max(0, pos_first - p.window + 1);
    }
    // This lane's keys: [r_lo, r_hi).
    const int r_hi = !v_ok ? 0 : p.causal ? max(0, pos + 1) : ctx;
    const int r_lo = (p.causal && p.window > 0) ? max(0, pos - p.window + 1) : 0;

    // Q^T operand: lane holds q[row][16 k + 4 quad .. + 3] for k < NT.
    f32x4_t qreg[NT];
    {
        const float* qp = static_cast<const float*>(p.q) + orow * D + 4 * quad;
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            uint4 w = *reinterpret_cast<const uint4*>(qp + 16 * k);
            w = q_fold(w, p.q_and, p.q_xor);
            const f32x4_t x = {as_f32(w.x), as_f32(w.y), as_f32(w.z), as_f32(w.w)};
            qreg[k] = v_ok ? x : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    const bool alibi = p.alibi != nullptr;                      // uniform
    const float al2 = alibi && v_ok ? p.alibi[h] * LOG2E : 0.f; // slope in log2 units

    // Staging: thread t copies float4s t, t + nthreads, ... of each matrix of a tile.
    constexpr int PER = (T::F4 + nthreads - 1) / nthreads;   // float4s per thread and matrix
    const int64_t kv_row = PAGED ? D : (int64_t)p.n_kv * D;   // floats between key rows
    const float* kbase;
    const float* vbase;
    if constexpr (PAGED) {
        kbase = static_cast<const float*>(p.k) + (int64_t)g * BK * D;
        vbase = static_cast<const float*>(p.v) + (int64_t)g * BK * D;
    } else {
        kbase = static_cast<const float*>(p.k) + ((int64_t)b * S_len * p.n_kv + g) * D;
        vbase = static_cast<const float*>(p.v) + ((int64_t)b * S_len * p.n_kv + g) * D;
    }
    float4 kst[PER], vst[PER];
    auto load_tile = [&](int t) {
        const int key0 = t * BK;
        int64_t blk_off = 0;
        if constexpr (PAGED) {
            const int phys = load_uniform(p.block_table + (int64_t)b * p.max_blocks + t);
            blk_off = (int64_t)phys * p.n_kv * BK * D;   // checked above
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int f = (int)threadIdx.x + i * nthreads;
            const int r = f / (D / 4), c4 = f % (D / 4);
            const int key = key0 + r;
            kst[i] = vst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            // Keys the workgroup owns; the others stay zero (never read past a
            // contiguous sequence; unwritten paged slots never reach P V).
            if (f < T::F4 && key >= k_lo && key < k_hi) {
                const int64_t off = blk_off + (int64_t)(PAGED ? r : key) * kv_row + 4 * c4;
                kst[i] = *reinterpret_cast<const float4*>(kbase + off);
                vst[i] = *reinterpret_cast<const float4*>(vbase + off);
            }
        }
    };
    auto store_tile = [&](int buf) {
        float* kl = fsm + buf * T::BUF;
        float* vl = kl + T::MAT;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int f = (int)threadIdx.x + i * nthreads;
            if (f < T::F4) {
                const int r = f / (D / 4), c4 = f % (D / 4);
                *reinterpret_cast<float4*>(kl + r * T::STRIDE + 4 * c4) = kst[i];
                *reinterpret_cast<float4*>(vl + r * T::STRIDE + 4 * c4) = vst[i];
            }
        }
    };

    float m_run = M_FLOOR, l_run = 0.f;
    f32x4_t acc[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const bool wave_live = __builtin_amdgcn_readfirstlane(v0 + wave * ROWS < VR ? 1 : 0) != 0;

    const int t0 = k_lo / BK;
    const int t1 = k_hi > k_lo ? (k_hi + BK - 1) / BK : t0;
    if (t0 < t1) load_tile(t0);
    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        store_tile(buf);
        __syncthreads();
        if (t + 1 < t1) load_tile(t + 1);
        if (!wave_live) continue;   // uniform: a wave past the last row only stages
        const float* kl = fsm + buf * T::BUF;
        const float* vl = kl + T::MAT;

        // S^T[key 4 quad + r][row col] over the head dimension.
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kl + col * T::STRIDE + 16 * k + 4 * quad);
#pragma unroll
            for (int c = 0; c < 4; ++c) s = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[c], qreg[k][c], s, 0, 0, 0);
        }
        // Scores in log2 units, masked, and the tile's row max.
        float sc[4];
        float mx = M_FLOOR;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = t * BK + 4 * quad + r;
            float x = alibi ? fmaf(s[r], p.scale_log2, al2 * (float)(key - pos)) : s[r] * p.scale_log2;
            x = (key >= r_lo && key < r_hi) ? x : -INFINITY;
            sc[r] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sc[r] = __builtin_amdgcn_exp2f(sc[r] - m_new);
            ps += sc[r];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        // O^T[dim 16 k + 4 quad + r][row col] += V^T P^T: this lane's probabilities
        // for keys 4 quad + c are the B operand as they stand.
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            f32x4_t o = acc[k] * alpha;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o = __builtin_amdgcn_mfma_f32_16x16x4f32(vl[(4 * quad + c) * T::STRIDE + 16 * k + col], sc[c], o,
                                                         0, 0, 0);
            acc[k] = o;
        }
    }

    if (!v_ok) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;   // a row with no keys is zero
    // Lane holds O[row][16 k + 4 quad + r]: gather the four dims of each block
    // from the lanes of its column that computed them.
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        *reinterpret_cast<float4*>(out + 16 * k + 4 * quad) =
            make_float4(acc[k][0] * inv, acc[k][1] * inv, acc[k][2] * inv, acc[k][3] * inv);
    }
}

template <int D, bool PAGED> hipError_t launch_typed(const PrefillArgs& a, hipStream_t s) {
    const int64_t vr = (int64_t)a.seq_len * a.group;   // virtual rows, an int in the kernel
    const int64_t tiles = (vr + ROWS * WAVES - 1) / (ROWS * WAVES);
    if (vr > INT32_MAX - ROWS * WAVES || a.n_kv > 65535 || a.batch > 65535) return hipErrorNotSupported;
    const dim3 grid((unsigned)tiles, (unsigned)a.n_kv, (unsigned)a.batch);
    hipLaunchKernelGGL((attn_f32_kernel<D, PAGED>), grid, dim3(64 * WAVES), F32Tile<D>::LDS, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const PrefillArgs& a, int head_dim, hipStream_t s) {
    const bool paged = a.block_table != nullptr;
    if (head_dim == 128) return paged ? launch_typed<128, true>(a, s) : launch_typed<128, false>(a, s);
    if (head_dim == 64) return paged ? launch_typed<64, true>(a, s) : launch_typed<64, false>(a, s);
    return hipErrorNotSupported;
}

}  // namespace pa
