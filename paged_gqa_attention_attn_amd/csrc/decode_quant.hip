// decode_quant.hip -- paged GQA decode over a quantised (FP8 E4M3 or INT8) KV cache,
// on the gfx950 matrix cores.
//
// The cache keeps every (token, KV head) row of K and of V as one-byte codes and
// one fp32 scale, value = code * scale ("LLM 推理全过程的维度变化与核心公式",
// research.frankk.site, "KV Cache 的形状与增长": the fp16 cache quantised to
// int8 / fp8 per token; the dimension-walkthrough page counts FP8 as one byte
// per element). Decode reads half the bytes of a bf16 cache for the same
// context. The work decomposition is that of decode_mfma.hip (one workgroup per
// head slice of a KV head and partition, each wave a contiguous run of 16-token
// blocks through its own LDS ring, cross-wave merge in LDS, partials for the
// log-sum-exp reduce kernel when a context is split); what changes per block:
//
//  * Each block brings a D-byte-per-row K tile, a V tile and the two 16-float
//    scale vectors, all by global_load_lds (the scales with one dword copy whose
//    lanes 0-15 fetch K scales and 16-31 V scales).
//  * The K operand of S^T = K q^T is 8 codes per lane widened in registers to
//    the query's type (FP8: v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 1, an
//    exact conversion; INT8: through fp32, exact), so the product runs on the
//    bf16/f16 matrix cores; the K scale multiplies the 4 scores each lane holds.
//  * The V scale folds into P (P' = P * v_scale per key; the softmax
//    denominator keeps P). V^T comes from the row-major code tile in dwords (4
//    dims of one key); the dwords of a lane's 4 keys are byte-transposed in
//    registers (8 v_perm per 64 dims), so O^T tile t = 4 h + m takes dims
//    64 h + 4 r + m as its rows r, and widened like K.
//  * Codes of rows outside [first, ctx) are zeroed in LDS and their P' is
//    selected to 0: an unused slot may hold a NaN code or a NaN scale.
//  * A decode step may carry its own append: the new token's K and V rows are
//    quantised in registers exactly as the quantising append does (quant.h),
//    patched into the LDS copy of their block, and written to the cache by one
//    wave at the end, so the step equals the append followed by the decode.
//  * Per-channel scales (one fixed fp32 scale per (KV head, channel), the other
//    granularity of the same item): no scale copies. The K scales multiply q
//    once, q * sk held as a bf16 hi + lo pair (so S^T runs on the bf16 matrix
//    cores with about 16 significant bits of q * sk, two products per k-step);
//    the V scales multiply the O^T rows (dims) once at the end; P is not scaled.
//  * Several query rows per sequence (multi-row decode, chunked prefill): the
//    (query head, row) pairs of a KV head take the columns; a row at position
//    ctx - NR + r sees keys up to that position.
// Rows are stored with their 16-byte chunk c at position c ^ swz(row), swz
// chosen for one-byte rows so that both operand reads stay conflict-free.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "quant.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int BS = 16;
constexpr float TAU = 8.0f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float M_FLOOR = -1e30f; // running-max start: finite, so 2^(s - m) of a masked s is 0
constexpr int MAX_WAVES = 8;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

struct QFp8 {
    static constexpr bool kFp8 = true;
};
struct QInt8 {
    static constexpr bool kFp8 = false;
};

// Four one-byte codes (bytes 0..3 of w) as four elements of a 16-bit operand of type E.
template <class Q, class E> __device__ __forceinline__ uint2 widen4(uint32_t w);
template <> __device__ __forceinline__ uint2 widen4<QFp8, BF16>(uint32_t w) {
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
}
template <> __device__ __forceinline__ uint2 widen4<QFp8, F16>(uint32_t w) {
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
}
// A signed byte is exact in fp32 and has at most 7 significant bits, so the
// packed fp32 -> bf16 conversion (one instruction per pair) rounds nothing.
template <> __device__ __forceinline__ uint2 widen4<QInt8, BF16>(uint32_t w) {
    const bf16x2_t a = {(__bf16)(float)(int8_t)w, (__bf16)(float)(int8_t)(w >> 8)};
    const bf16x2_t b = {(__bf16)(float)(int8_t)(w >> 16), (__bf16)(float)(int8_t)(w >> 24)};
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}
template <> __device__ __forceinline__ uint2 widen4<QInt8, F16>(uint32_t w) {
    f16x2_t a, b;
    a[0] = (_Float16)(float)(int8_t)w;
    a[1] = (_Float16)(float)(int8_t)(w >> 8);
    b[0] = (_Float16)(float)(int8_t)(w >> 16);
    b[1] = (_Float16)(float)(int8_t)(w >> 24);
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// A 16-bit element of q's type (bits in the low half) as fp32, exactly.
template <class E> __device__ __forceinline__ float half_to_f32(uint32_t bits);
template <> __device__ __forceinline__ float half_to_f32<BF16>(uint32_t bits) { return as_f32(bits << 16); }
template <> __device__ __forceinline__ float half_to_f32<F16>(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

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

template <int D, int HW, int R, bool PC = false> struct QLayout {
    static constexpr int ROW = D;                     // bytes per token row (one-byte codes)
    static constexpr int CPR = ROW / 16;              // 16-byte chunks per row: 8 or 4
    static constexpr int TILE = BS * ROW;             // one (block, KV head) code tile
    static constexpr int NQ = TILE / 1024;            // 1 KB wave copies per tile
    static constexpr int SC = 256;                    // scale copy: K scales, V scales, repeat
    static constexpr int SLOTB = 2 * TILE + SC;       // one ring slot
    static constexpr int OPS = 2 * NQ + (PC ? 0 : 1); // vector-memory operations per block (no scale copy per channel)
    static constexpr int RING = R * SLOTB;            // R blocks in flight per wave
    static constexpr int PITCH = D + 4;
    static constexpr int SLOT = HW * PITCH + 2 * HW;  // merge slot floats
    static constexpr int WAVE_BYTES = ((RING > SLOT * 4 ? RING : SLOT * 4) + 15) / 16 * 16;
    // Rows of the 16 keys share 256-byte bank lines 256 / ROW at a time; rows of one
    // line get distinct chunk masks and rows of the same line position distinct ones.
    static __device__ __forceinline__ int swz(int r) { return (r / (16 / CPR)) & (CPR - 1); }
};

template <class Q, class E, int D, int HW, int R, bool PC>
__global__ __launch_bounds__(64 * MAX_WAVES, 2) void decode_quant_kernel(const DecodeArgs p) {
    using L = QLayout<D, HW, R, PC>;
    using S = typename E::storage;
    // Matrix-core operand type: q's own, or bf16 per channel, where q arrives
    // multiplied by the K channel scales as a bf16 hi + lo pair.
    using M = typename std::conditional<PC, BF16, E>::type;
    constexpr int ROW = L::ROW, TILE = L::TILE, NQ = L::NQ, OPS = L::OPS;
    constexpr int KK = D / 32;    // S^T k-steps
    constexpr int MT = D / 16;    // O^T tiles
    static_assert(HW == 1 || HW == 2 || HW == 4 || HW == 8 || HW == 16, "1 to 16 MFMA columns");
    static_assert(TILE % 1024 == 0, "tiles move in whole 1 KB copies");
    static_assert(OPS * R < 64, "a ring's copies fit the vmcnt counter");

    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int part = blockIdx.x;
    const int g = blockIdx.y / p.hsg;
    const int hsgi = blockIdx.y % p.hsg;
    const int b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // MFMA column col holds (head, row) pair v = hsgi * HW + col of the KV head's
    // G * NR pairs: new-token row v / G of the step's NR (1 for single-row decode),
    // query head g * G + v % G. qo_row(v) is its row of q and of out.
    const int G = p.group, NR = p.q_rows;
    auto qo_row = [&](int v) { return ((int64_t)b * NR + v / G) * p.n_q + (int64_t)g * G + v % G; };
    const int v_col = hsgi * HW + (col < HW ? col : 0);
    const int blk0 = part * p.waves_tok * p.blocks_per_wave + wave * p.blocks_per_wave;
    u32x4_t qreg[KK];
    u32x4_t qlo[PC ? KK : 1];   // per channel: the lo part of q * K scale
    {
        const char* qrow = (const char*)p.q + qo_row(v_col) * (D * 2);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (col < HW) v = q_fold(*reinterpret_cast<const uint4*>(qrow + (32 * kk + 8 * grp) * 2), p.q_and, p.q_xor);
            if constexpr (PC) {
                // Dims 32 kk + 8 grp + i: q_i * sk_i in fp32, then hi = bf16(x), lo = bf16(x - hi).
                const float* sk = p.k_scale + (int64_t)g * D + 32 * kk + 8 * grp;
                const float4 s0 = *reinterpret_cast<const float4*>(sk);
                const float4 s1 = *reinterpret_cast<const float4*>(sk + 4);
                const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = half_to_f32<E>(w[i] & 0xffffu) * sc[2 * i];
                    const float x1 = half_to_f32<E>(w[i] >> 16) * sc[2 * i + 1];
                    hi[i] = Mfma<BF16>::pack(x0, x1);
                    lo[i] = Mfma<BF16>::pack(x0 - Mfma<BF16>::lo_of(hi[i]), x1 - Mfma<BF16>::hi_of(hi[i]));
                }
                qreg[kk] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
                qlo[kk] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
            } else {
                qreg[kk] = u32x4_t{v.x, v.y, v.z, v.w};
            }
        }
    }
    int my_phys = 0;
    if (lane < p.blocks_per_wave && blk0 + lane < p.max_blocks)
        my_phys = p.block_table[(int64_t)b * p.max_blocks + blk0 + lane];

    const int cap = p.max_blocks * BS;
    const int ctx_in = __builtin_amdgcn_readfirstlane(p.context_lens[b]);
    const bool ctx_bad = ctx_in > cap;
    const int ctx = (ctx_in < 0 || ctx_bad) ? 0 : ctx_in;
    const int nblk = (ctx + BS - 1) / BS;
    const int first = window_first(ctx, NR, p.window);   // the earliest position any row sees
    // This column's row sees positions col_lo .. col_hi (causal among the new rows).
    const int col_hi = ctx - NR + v_col / G;
    const int col_lo = p.window > 0 ? col_hi - p.window + 1 : 0;
    const int fb = first / BS;
    const int bpp = p.waves_tok * p.blocks_per_wave;
    const int nparts = nblk > fb ? (nblk - fb + bpp - 1) / bpp : 1;
    if (part >= nparts) return;
    const int wb0 = blk0 + fb;
    if (fb > 0) {
        my_phys = 0;
        if (lane < p.blocks_per_wave && wb0 + lane < p.max_blocks)
            my_phys = p.block_table[(int64_t)b * p.max_blocks + wb0 + lane];
    }
    const int nb = max(0, min(nblk - wb0, p.blocks_per_wave));
    // ALiBi: the column's head slope in log2 units; with it, scores are formed in
    // log2 units before the max (c2 = 1), else scaled inside it.
    const bool alibi = p.alibi != nullptr;   // uniform
    const float al2 = alibi ? p.alibi[(int64_t)g * G + v_col % G] * LOG2E : 0.f;
    const float c2 = alibi ? 1.f : p.scale_log2;
    const bool phys_bad = __any(lane < nb && (my_phys < 0 || my_phys >= p.num_blocks));

    // Fused append: the wave whose run holds position ctx - 1 patches the new
    // token's codes and scales into its LDS copy of that block, and one wave of
    // the sequence's last partition writes them to the cache at the end. Both
    // quantise the new rows exactly as the quantising append does.
    constexpr int EPL = D / 64;   // row bytes (codes) per lane
    const bool fused = p.new_slots != nullptr;
    const int64_t new_slot = fused ? p.new_slots[b] : -1;
    const bool slot_ok = new_slot >= 0 && new_slot < (int64_t)p.num_blocks * BS;
    const int last_blk = ctx > 0 ? (ctx - 1) / BS : -1;
    const bool patch_here = fused && slot_ok && last_blk >= wb0 && last_blk < wb0 + nb;
    const bool writer = fused && slot_ok && part == nparts - 1 && hsgi == 0 && wave == 0;
    uint32_t new_kc = 0, new_vc = 0;
    float new_ks = 0.f, new_vs = 0.f;
    if (patch_here || writer) {   // uniform over the wave
        float xk[EPL], xv[EPL];
        const int64_t e0 = ((int64_t)b * p.n_kv + g) * D + lane * EPL;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            xk[i] = load_f32<E>(p.k_new, e0 + i);
            xv[i] = load_f32<E>(p.v_new, e0 + i);
        }
        if constexpr (PC) {
            const int64_t c0 = (int64_t)g * D + lane * EPL;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                new_kc |= channel_code<Q::kFp8>(xk[i], p.k_scale[c0 + i]) << (8 * i);
                new_vc |= channel_code<Q::kFp8>(xv[i], p.v_scale[c0 + i]) << (8 * i);
            }
        } else {
            new_ks = quantize_row<Q::kFp8, EPL>(xk, new_kc);
            new_vs = quantize_row<Q::kFp8, EPL>(xv, new_vc);
        }
    }

    char* ring = smem + wave * L::WAVE_BYTES;
    const uint32_t ring_lds = lds_addr(ring);
    const int64_t block_bytes = (int64_t)p.n_kv * TILE;
    uint32_t src_off[NQ];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
        const int off = qq * 1024 + 16 * lane;
        const int r = off / ROW;
        src_off[qq] = r * ROW + (((off % ROW) / 16) ^ L::swz(r)) * 16;
    }
    const char* kbase = (const char*)p.k_cache + (int64_t)g * TILE;
    const char* vbase = (const char*)p.v_cache + (int64_t)g * TILE;
    // Scale copy: lanes 0-15 the K scales of the block's 16 rows, 16-31 the V
    // scales, 32-63 the same again (landing in the unused half of the slot).
    const float* sbase = ((lane >> 4) & 1 ? p.v_scale : p.k_scale) + (int64_t)g * BS + (lane & 15);
    const bool once = p.hsg == 1;   // no other workgroup reads these tiles: non-temporal
    auto issue = [&](int i) {
        const int64_t phys = __builtin_amdgcn_readlane(my_phys, i);
        const uint32_t dst = ring_lds + (i % R) * L::SLOTB;
        const char* kb = kbase + phys * block_bytes;
        const char* vb = vbase + phys * block_bytes;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) copy_to_lds16(kb + src_off[qq], dst + qq * 1024, once);
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) copy_to_lds16(vb + src_off[qq], dst + TILE + qq * 1024, once);
        if constexpr (!PC) copy_to_lds4(sbase + phys * p.n_kv * BS, dst + 2 * TILE, once);
    };

    uint32_t k_off[KK];   // K operand: row col, bytes 32 kk + 8 grp .. +8
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const int c = 2 * kk + (grp >> 1);
        k_off[kk] = col * ROW + ((c ^ L::swz(col)) * 16) + 8 * (grp & 1);
    }
    // V^T operand: O^T tile t = 4 h + m takes dims 64 h + 4 r + m as its rows r, so
    // one dword of key row 4 grp + e at dims 64 h + 4 col .. +3 feeds four tiles; a
    // 4 x 4 byte transpose of the four keys' dwords gives each tile its 4 keys.
    constexpr int VH = D / 64;   // halves of 64 dims
    uint32_t v_off[VH][4];
#pragma unroll
    for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * grp + e;
            v_off[h][e] = TILE + r * ROW + (((4 * h + col / 4) ^ L::swz(r)) * 16) + 4 * (col % 4);
        }

    f32x4_t o[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Running max (log2 units) of column col. It starts finite: with several rows a
    // block can hold no key that some column attends, and 2^(s - m) of a masked s
    // must then be 0, not 2^(-inf + inf).
    float m_run = M_FLOOR;
    float l_run = 0.f;

    wait_vmcnt<0>();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : : "v"(qreg[kk]));

    if (!phys_bad && nb > 0) {
        const int pre = min(R, nb);
        for (int i = 0; i < pre; ++i) issue(i);
        for (int i = 0; i < nb; ++i) {
            // Block i has landed once at most (blocks issued after it) * OPS copies are pending.
            const int ahead = min(R - 1, nb - 1 - i);
            if constexpr (R >= 2) {
                if (ahead == 1) wait_vmcnt<OPS>();
            }
            if (ahead == 0) wait_vmcnt<0>();
            char* base = ring + (i % R) * L::SLOTB;
            const int pos0 = (wb0 + i) * BS;
            if (patch_here && wb0 + i == last_blk) {   // uniform: the new token's block
                const int r = (ctx - 1) % BS;
                const int at = r * ROW + ((((lane * EPL) / 16) ^ L::swz(r)) * 16) + (lane * EPL) % 16;
                if constexpr (EPL == 2) {
                    *reinterpret_cast<uint16_t*>(base + at) = (uint16_t)new_kc;
                    *reinterpret_cast<uint16_t*>(base + TILE + at) = (uint16_t)new_vc;
                } else {
                    *reinterpret_cast<uint8_t*>(base + at) = (uint8_t)new_kc;
                    *reinterpret_cast<uint8_t*>(base + TILE + at) = (uint8_t)new_vc;
                }
                if (!PC && lane == 0) {
                    *reinterpret_cast<float*>(base + 2 * TILE + 4 * r) = new_ks;
                    *reinterpret_cast<float*>(base + 2 * TILE + 64 + 4 * r) = new_vs;
                }
            }
            // Some key of the block is outside some column's range (uniform).
            const bool edge = pos0 + BS - 1 > ctx - NR || (p.window > 0 && pos0 < ctx - p.window);
            if (edge) {
                // Zero the V code rows outside [first, ctx) (whole rows).
#pragma unroll
                for (int k = 0; k < BS * L::CPR / 64; ++k) {
                    const int idx = k * 64 + lane;
                    const int r = idx / L::CPR;
                    const int pos = pos0 + r;
                    if (pos >= ctx || pos < first)
                        *reinterpret_cast<uint4*>(base + TILE + r * ROW + (idx % L::CPR) * 16) = make_uint4(0, 0, 0, 0);
                }
            }
            u32x4_t ka[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint2 c8 = *reinterpret_cast<const uint2*>(base + k_off[kk]);
                const uint2 lo = widen4<Q, M>(c8.x), hi = widen4<Q, M>(c8.y);
                ka[kk] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
            }
            uint2 va[MT];
#pragma unroll
            for (int h = 0; h < VH; ++h) {
                uint32_t w[4];   // key 4 grp + e, dims 64 h + 4 col + m in byte m
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const uint32_t*>(base + v_off[h][e]);
                // Byte transpose: x[m] holds dim 64 h + 4 col + m of keys e = 0..3 in byte e.
                const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
                const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
                const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
                const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
                va[4 * h + 0] = widen4<Q, M>(__builtin_amdgcn_perm(lo23, lo01, 0x05040100u));
                va[4 * h + 1] = widen4<Q, M>(__builtin_amdgcn_perm(lo23, lo01, 0x07060302u));
                va[4 * h + 2] = widen4<Q, M>(__builtin_amdgcn_perm(hi23, hi01, 0x05040100u));
                va[4 * h + 3] = widen4<Q, M>(__builtin_amdgcn_perm(hi23, hi01, 0x07060302u));
            }
            float4 ks = make_float4(1.f, 1.f, 1.f, 1.f), vs = ks;   // per channel: scales applied outside
            if constexpr (!PC) {
                ks = *reinterpret_cast<const float4*>(base + 2 * TILE + 16 * grp);
                vs = *reinterpret_cast<const float4*>(base + 2 * TILE + 64 + 16 * grp);
            }
            lds_reads_done();
            if (i + R < nb) issue(i + R);

            f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                s = Mfma16<M>::qk(ka[kk], qreg[kk], s);
                if constexpr (PC) s = Mfma16<M>::qk(ka[kk], qlo[kk], s);
            }
            if constexpr (!PC) {
                s[0] *= ks.x;
                s[1] *= ks.y;
                s[2] *= ks.z;
                s[3] *= ks.w;
            }
            if (alibi) {   // - m_h log2(e) (i - j) for the column's row i and key j = pos0 + 4 grp + j'
                const float b0 = al2 * (float)(pos0 + 4 * grp - col_hi);
#pragma unroll
                for (int j = 0; j < 4; ++j) s[j] = fmaf(s[j], p.scale_log2, fmaf(al2, (float)j, b0));
            }
            bool live[4] = {true, true, true, true};
            if (edge) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int pos = pos0 + 4 * grp + j;
                    live[j] = pos <= col_hi && pos >= col_lo;
                    s[j] = live[j] ? s[j] : -INFINITY;
                }
            }
            float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * c2;
            if (__any(bm > m_run + TAU)) {
                const float m_new = fmaxf(m_run, stride_reduce<16, true>(bm));
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < MT; ++t) o[t] *= alpha;
                m_run = m_new;
            }
            const float vsc[4] = {vs.x, vs.y, vs.z, vs.w};
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pj = __builtin_amdgcn_exp2f(fmaf(s[j], c2, -m_run));
                l_run += pj;
                pr[j] = live[j] ? (PC ? pj : pj * vsc[j]) : 0.f;   // per row: V scale folded into P
            }
            const uint2 ph = make_uint2(Mfma<M>::pack(pr[0], pr[1]), Mfma<M>::pack(pr[2], pr[3]));
            if constexpr (Mfma<M>::kSplit) {
                // hi and lo parts stacked along k of one 16x16x32 product (twice the
                // rate of two 16x16x16 products): k slots 8 grp + j hold key 4 grp + j % 4,
                // part j / 4, in both operands.
                const uint2 pl = make_uint2(Mfma<M>::pack(pr[0] - Mfma<M>::lo_of(ph.x), pr[1] - Mfma<M>::hi_of(ph.x)),
                                            Mfma<M>::pack(pr[2] - Mfma<M>::lo_of(ph.y), pr[3] - Mfma<M>::hi_of(ph.y)));
                const u32x4_t pb = u32x4_t{ph.x, ph.y, pl.x, pl.y};
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    o[t] = Mfma16<M>::qk(u32x4_t{va[t].x, va[t].y, va[t].x, va[t].y}, pb, o[t]);
            } else {
#pragma unroll
                for (int t = 0; t < MT; ++t) o[t] = Mfma16<M>::pv(va[t], ph, o[t]);
            }
        }
    }

    l_run = stride_reduce<16, false>(l_run);
    // o[4 h + m][j] is dim 64 h + 16 grp + 4 j + m of column col: gather the four m.
    float* mine = reinterpret_cast<float*>(ring);
    if (col < HW) {
#pragma unroll
        for (int h = 0; h < VH; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dim = 64 * h + 16 * grp + 4 * j;
                f32x4_t x = {o[4 * h][j], o[4 * h + 1][j], o[4 * h + 2][j], o[4 * h + 3][j]};
                if constexpr (PC) {   // times the V channel scales of those dims
                    const float4 sv = *reinterpret_cast<const float4*>(p.v_scale + (int64_t)g * D + dim);
                    x *= f32x4_t{sv.x, sv.y, sv.z, sv.w};
                }
                *reinterpret_cast<f32x4_t*>(mine + col * L::PITCH + dim) = x;
            }
        if (grp == 0) {
            mine[HW * L::PITCH + col] = phys_bad ? 0.f : m_run;
            mine[HW * L::PITCH + HW + col] = phys_bad ? NAN : l_run;
        }
    }
    __syncthreads();

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
    if (writer) {
        const int64_t row = ((new_slot / BS) * p.n_kv + g) * BS + new_slot % BS;
        uint8_t* kd = static_cast<uint8_t*>(p.k_cache_w) + row * D + lane * EPL;
        uint8_t* vd = static_cast<uint8_t*>(p.v_cache_w) + row * D + lane * EPL;
        if constexpr (EPL == 2) {
            *reinterpret_cast<uint16_t*>(kd) = (uint16_t)new_kc;
            *reinterpret_cast<uint16_t*>(vd) = (uint16_t)new_vc;
        } else {
            *kd = (uint8_t)new_kc;
            *vd = (uint8_t)new_vc;
        }
        if (!PC && lane == 0) {
            p.k_scale_w[row] = new_ks;
            p.v_scale_w[row] = new_vs;
        }
    }
}

template <class Q, class E, int D, int HW, int R, bool PC> hipError_t launch_pc(const DecodeArgs& a, hipStream_t s) {
    const size_t lds = (size_t)a.waves_tok * QLayout<D, HW, R, PC>::WAVE_BYTES;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    static const hipError_t opt_in = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_quant_kernel<Q, E, D, HW, R, PC>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (opt_in != hipSuccess) return opt_in;
    const dim3 grid(a.nparts_max, a.n_kv * a.hsg, a.batch);
    hipLaunchKernelGGL((decode_quant_kernel<Q, E, D, HW, R, PC>), grid, dim3(64 * a.waves_tok), lds, s, a);
    return hipGetLastError();
}

template <class Q, class E, int D, int HW, int R> hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    const hipError_t err = a.chan_scales ? launch_pc<Q, E, D, HW, R, true>(a, s) : launch_pc<Q, E, D, HW, R, false>(a, s);
    if (err != hipSuccess || a.nparts_max <= 1) return err;
    DecodeArgs m = a;
    m.n_q = a.n_q * a.q_rows;   // the reduce kernel's rows: (b, r, h) in [B][q_rows][n_q] order
    return launch_decode_reduce(m, std::is_same<E, BF16>::value ? Elem::BF16 : Elem::F16, D, s);
}

template <class Q, class E, int D, int R> hipError_t launch_hw(const DecodeArgs& a, hipStream_t s) {
    switch (a.gw) {
    case 1: return launch_typed<Q, E, D, 1, R>(a, s);
    case 2: return launch_typed<Q, E, D, 2, R>(a, s);
    case 4: return launch_typed<Q, E, D, 4, R>(a, s);
    case 8: return launch_typed<Q, E, D, 8, R>(a, s);
    case 16: return launch_typed<Q, E, D, 16, R>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <class Q, class E, int D> hipError_t launch_ring(const DecodeArgs& a, hipStream_t s) {
    if (a.ring == 2) return launch_hw<Q, E, D, 2>(a, s);
    if (a.ring == 1) return launch_hw<Q, E, D, 1>(a, s);
    return hipErrorInvalidValue;
}

template <class Q, class E> hipError_t launch_dim(const DecodeArgs& a, int head_dim, hipStream_t s) {
    if (head_dim == 128) return launch_ring<Q, E, 128>(a, s);
    if (head_dim == 64) return launch_ring<Q, E, 64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

int quant_wave_bytes(int head_dim, int hw, int ring) {
    const int tile = BS * head_dim;
    const int slotb = ring * (2 * tile + 256);
    const int slot = (hw * (head_dim + 4) + 2 * hw) * 4;
    return ((slotb > slot ? slotb : slot) + 15) / 16 * 16;
}

hipError_t launch_decode_quant(const DecodeArgs& a, Elem q_type, QuantFmt fmt, int head_dim, hipStream_t s) {
    if (a.hs_wg != 1 || a.waves_tok < 1 || a.waves_tok > MAX_WAVES) return hipErrorInvalidValue;
    if (a.q_rows < 1 || a.window < 0 || !a.k_scale || !a.v_scale) return hipErrorInvalidValue;
    // Several new rows per sequence: their pairs fill whole slices of gw columns,
    // and no append rides along.
    if (a.q_rows > 1 && ((a.group * a.q_rows) % a.gw != 0 || a.new_slots != nullptr)) return hipErrorInvalidValue;
    if (fmt == QuantFmt::FP8_E4M3 && q_type == Elem::BF16) return launch_dim<QFp8, BF16>(a, head_dim, s);
    if (fmt == QuantFmt::FP8_E4M3 && q_type == Elem::F16) return launch_dim<QFp8, F16>(a, head_dim, s);
    if (fmt == QuantFmt::INT8 && q_type == Elem::BF16) return launch_dim<QInt8, BF16>(a, head_dim, s);
    if (fmt == QuantFmt::INT8 && q_type == Elem::F16) return launch_dim<QInt8, F16>(a, head_dim, s);
    return hipErrorInvalidValue;
}

}  // namespace pa
