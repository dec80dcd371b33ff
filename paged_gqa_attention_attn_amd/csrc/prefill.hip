// prefill.hip -- causal (or full) prefill attention with bf16/f16 MFMA for gfx950.
//
// O = softmax(Q K^T * scale + M) V for every query position of a prompt, with
// the causal mask M_ij = 0 for j <= i and -inf otherwise ("注意力演进与推理流程",
// jerryiiii.gitbook.io, section 1.1; xinc.fun/index.php/archives/233, section 2),
// query head h reading KV head floor(h / G) (same first page, section 3.1).
// The S x S score matrix is never stored: key tiles stream through LDS and a
// running max / sum rescales the output ("LLM 推理全过程的维度变化与核心公式",
// research.frankk.site, Flash Attention paragraph of "工程优化怎么嵌进公式").
//
// Tiling (per workgroup: 4 waves, 128 query rows of one head, 32 per wave)
//  * Key/value tiles of 64 positions are double-buffered in LDS: K row-major
//    (rows padded to 272 B), V transposed to [dim][key] (rows padded to 136 B)
//    because the PV product needs 8 consecutive keys per lane for one dim.
//  * S^T = K Q^T with v_mfma_f32_32x32x16 (M = keys, N = queries, K = dims):
//    each lane then holds 16 keys of ONE query per 32-key half-tile, so the
//    row max needs only one v_permlane32_swap.
//  * O^T = V^T P^T (M = dims, N = queries, K = keys): each lane's output
//    column also belongs to one query, so the online-softmax rescale is a
//    lane-local multiply. P is split into bf16 (or f16) hi + lo parts and both
//    are multiplied, which keeps the result within ~1e-5 of exact (P rounded
//    to 8 bits alone errs by up to ~3e-3 on rows with few keys).
//  * The K/V-position permutation inside one MFMA is shared by both operands
//    (it only has to be the same on A and B): lane half h = lane/32 holds keys
//    {16j + 8(i/4) + 4h + i%4 : i = 0..7} of 16-key group j, which is exactly
//    where the S^T accumulator put them.
//  * Causal: a workgroup visits key tiles up to its last query; tiles past a
//    wave's last query are skipped by that wave; the heavy (late) query tiles
//    are launched first.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int WM = 32;    // query rows per wave
constexpr int NWAVES = BM / WM;

template <class E> struct Mfma;
template <> struct Mfma<BF16> {
    static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    // Pack two fp32 values as the element type (round to nearest even), low half first.
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        return (uint32_t)narrow<BF16>(x) | ((uint32_t)narrow<BF16>(y) << 16);
    }
    static __device__ __forceinline__ float lo_of(uint32_t w) { return as_f32(w << 16); }
    static __device__ __forceinline__ float hi_of(uint32_t w) { return as_f32(w & 0xffff0000u); }
};
template <> struct Mfma<F16> {
    static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        return (uint32_t)narrow<F16>(x) | ((uint32_t)narrow<F16>(y) << 16);
    }
    static __device__ __forceinline__ float lo_of(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi_of(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
};

template <int D> struct Layout {
    static constexpr int KROW = D * 2 + 16;          // padded bytes per K row in LDS
    static constexpr int VTROW = BN * 2 + 8;         // padded bytes per V^T row (one dim)
    static constexpr int K_BYTES = BN * KROW;
    static constexpr int VT_BYTES = D * VTROW;
    static constexpr int BUF = K_BYTES + VT_BYTES;   // one tile buffer
    static constexpr int CHUNKS = BN * D / 8;        // 16-byte chunks per K (or V) tile
    static constexpr int PER_THREAD = CHUNKS / (64 * NWAVES);
    static_assert(PER_THREAD * 64 * NWAVES == CHUNKS, "tile splits evenly over the workgroup");
};

template <class E, int D>
__global__ __launch_bounds__(64 * NWAVES, 2) void prefill_kernel(const PrefillArgs p) {
    using L = Layout<D>;
    using S = typename E::storage;
    constexpr int KK = D / 16;     // MFMA k-steps over the head dimension
    constexpr int MT = D / 32;     // 32-dim output tiles
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int nqt = (p.seq_len + BM - 1) / BM;
    const int qt = p.causal ? nqt - 1 - (int)blockIdx.x : (int)blockIdx.x;  // heavy tiles first
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = h / p.group;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;    // 0 or 1
    const int l32 = lane & 31;
    const int q0 = qt * BM + wave * WM;           // first query row of this wave
    const int my_q = q0 + l32;                    // the query this lane's columns belong to
    const int S_len = p.seq_len;

    const int64_t q_stride = (int64_t)p.n_q * D;       // elements between query positions
    const int64_t kv_stride = (int64_t)p.n_kv * D;     // elements between key positions
    const S* Qg = reinterpret_cast<const S*>(p.q) + (int64_t)b * S_len * q_stride + (int64_t)h * D;
    const S* Kg = reinterpret_cast<const S*>(p.k) + (int64_t)b * S_len * kv_stride + (int64_t)g * D;
    const S* Vg = reinterpret_cast<const S*>(p.v) + (int64_t)b * S_len * kv_stride + (int64_t)g * D;

    // Q^T operand: lane holds dims 16*kk + 8*half .. +8 of its query, for every kk.
    u32x4_t qreg[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (my_q < S_len) {
            const uint4 v = *reinterpret_cast<const uint4*>(Qg + (int64_t)my_q * q_stride + 16 * kk + 8 * half);
            qreg[kk] = u32x4_t{v.x, v.y, v.z, v.w};
        } else {
            qreg[kk] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    // Key tiles this workgroup visits.
    const int q_last_wg = min(qt * BM + BM, S_len) - 1;
    const int n_tiles = p.causal ? q_last_wg / BN + 1 : (S_len + BN - 1) / BN;
    const int q_last_wave = min(q0 + WM, S_len) - 1;

    // Tile loads: K chunk r of this thread covers (key row, 16-byte column) of the
    // tile; V chunks are assigned so that one wave's 64 lanes hold 64 consecutive
    // keys of the same 8 dims, which makes the transposed LDS stores contiguous.
    uint4 kbuf[L::PER_THREAD], vbuf[L::PER_THREAD];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int r = 0; r < L::PER_THREAD; ++r) {
            const int id = threadIdx.x + 64 * NWAVES * r;
            const int krow = id / (D / 8), kcol = id % (D / 8);
            const int kpos = j * BN + krow;
            kbuf[r] = kpos < S_len ? *reinterpret_cast<const uint4*>(Kg + (int64_t)kpos * kv_stride + kcol * 8)
                                   : make_uint4(0, 0, 0, 0);
            const int vkey = id % BN, vcol = id / BN;
            const int vpos = j * BN + vkey;
            vbuf[r] = vpos < S_len ? *reinterpret_cast<const uint4*>(Vg + (int64_t)vpos * kv_stride + vcol * 8)
                                   : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int buf) {
        char* kl = smem + buf * L::BUF;
        char* vl = kl + L::K_BYTES;
#pragma unroll
        for (int r = 0; r < L::PER_THREAD; ++r) {
            const int id = threadIdx.x + 64 * NWAVES * r;
            const int krow = id / (D / 8), kcol = id % (D / 8);
            *reinterpret_cast<uint4*>(kl + krow * L::KROW + kcol * 16) = kbuf[r];
            const int vkey = id % BN, vcol = id / BN;
            const uint32_t w[4] = {vbuf[r].x, vbuf[r].y, vbuf[r].z, vbuf[r].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t val = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
                *reinterpret_cast<uint16_t*>(vl + (vcol * 8 + e) * L::VTROW + vkey * 2) = val;
            }
        }
    };

    f32x16_t o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16_t{};
    float m_run = -INFINITY;   // running max (log2 units) of this lane's query
    float l_run = 0.f;         // this lane's share of the softmax denominator

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        if (j + 1 < n_tiles) load_tile(j + 1);
        const char* kl = smem + (j & 1) * L::BUF;
        const char* vl = kl + L::K_BYTES;
        const int key0 = j * BN;

        if (!p.causal || key0 <= q_last_wave) {
            // S^T for two 32-key halves of the tile.
            f32x16_t sc[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sc[st] = f32x16_t{};
                const char* krow = kl + (st * 32 + l32) * L::KROW + half * 16;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const uint4 a = *reinterpret_cast<const uint4*>(krow + kk * 32);
                    sc[st] = Mfma<E>::run(u32x4_t{a.x, a.y, a.z, a.w}, qreg[kk], sc[st]);
                }
            }
            // Scale, mask, and the tile max of this lane's query.
            const bool need_mask = key0 + BN > S_len || (p.causal && key0 + BN - 1 > q0);
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = sc[st][i] * p.scale_log2;
                    if (need_mask) {
                        const int key = key0 + st * 32 + (i / 4) * 8 + half * 4 + (i % 4);
                        if (key >= S_len || (p.causal && key > my_q)) x = -INFINITY;
                    }
                    sc[st][i] = x;
                    tmax = fmaxf(tmax, x);
                }
            }
            {
                float a2, b2;
                pair32(tmax, a2, b2);
                tmax = fmaxf(a2, b2);
            }
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;

            // P = 2^(s - m), split as hi + lo in the element type; PV on both parts.
            u32x4_t ph[2][2], pl[2][2];   // [half-tile][16-key group]
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int jg = 0; jg < 2; ++jg) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const float x0 = sc[st][8 * jg + 2 * w], x1 = sc[st][8 * jg + 2 * w + 1];
                        const float p0 = (x0 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x0 - m_new);
                        const float p1 = (x1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x1 - m_new);
                        hw[w] = Mfma<E>::pack(p0, p1);
                        const float r0 = p0 - Mfma<E>::lo_of(hw[w]);
                        const float r1 = p1 - Mfma<E>::hi_of(hw[w]);
                        lw[w] = Mfma<E>::pack(r0, r1);
                        l_run += p0 + p1;
                    }
                    ph[st][jg] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
                    pl[st][jg] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const char* vrow = vl + (mt * 32 + l32) * L::VTROW;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
#pragma unroll
                    for (int jg = 0; jg < 2; ++jg) {
                        const int kb = st * 32 + jg * 16 + half * 4;   // keys kb..kb+3 and kb+8..kb+11
                        const uint2 a0 = *reinterpret_cast<const uint2*>(vrow + kb * 2);
                        const uint2 a1 = *reinterpret_cast<const uint2*>(vrow + (kb + 8) * 2);
                        const u32x4_t a = u32x4_t{a0.x, a0.y, a1.x, a1.y};
                        o[mt] = Mfma<E>::run(a, ph[st][jg], o[mt]);
                        o[mt] = Mfma<E>::run(a, pl[st][jg], o[mt]);
                    }
                }
            }
        }

        if (j + 1 < n_tiles) store_tile((j + 1) & 1);
        __syncthreads();
    }

    // Denominator: this lane and its partner (lane ^ 32) covered complementary keys.
    {
        float a2, b2;
        pair32(l_run, a2, b2);
        l_run = a2 + b2;
    }
    if (my_q >= S_len) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t orow = ((int64_t)b * S_len + my_q) * p.n_q + h;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int dim = mt * 32 + grp * 8 + half * 4;
            const float v0 = o[mt][4 * grp] * inv, v1 = o[mt][4 * grp + 1] * inv;
            const float v2 = o[mt][4 * grp + 2] * inv, v3 = o[mt][4 * grp + 3] * inv;
            if (p.out_f32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + orow * D + dim) =
                    make_float4(v0, v1, v2, v3);
            } else {
                S* dst = reinterpret_cast<S*>(p.out) + orow * D + dim;
                dst[0] = narrow<E>(v0);
                dst[1] = narrow<E>(v1);
                dst[2] = narrow<E>(v2);
                dst[3] = narrow<E>(v3);
            }
        }
    }
}

template <class E, int D> hipError_t launch_typed(const PrefillArgs& a, hipStream_t s) {
    const size_t lds = 2 * (size_t)Layout<D>::BUF;
    static bool opt_in = [] {
        return hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<E, D>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    }();
    (void)opt_in;
    const dim3 grid((a.seq_len + BM - 1) / BM, a.n_q, a.batch);
    hipLaunchKernelGGL((prefill_kernel<E, D>), grid, dim3(64 * NWAVES), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, Elem e, int head_dim, hipStream_t s) {
    if (e == Elem::BF16 && head_dim == 128) return launch_typed<BF16, 128>(a, s);
    if (e == Elem::BF16 && head_dim == 64) return launch_typed<BF16, 64>(a, s);
    if (e == Elem::F16 && head_dim == 128) return launch_typed<F16, 128>(a, s);
    if (e == Elem::F16 && head_dim == 64) return launch_typed<F16, 64>(a, s);
    return hipErrorNotSupported;
}

}  // namespace pa
