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
// Tiling (per workgroup: 8 waves of 32 query rows, one KV head)
//  * A workgroup takes the HPW query heads of one KV group that share its K/V tiles
//    (4, 2 or 1: the largest dividing the group size) and 256 / HPW query rows of
//    each, so every K/V tile staged in LDS feeds 256 (head, row) pairs. At HPW = 4
//    the waves' rows (two runs of 32) end in the same 64-key tile, so all eight
//    do the same causal work between barriers.
//  * Key/value tiles of 64 positions stream through a ring of NBUF tiles in LDS
//    (one workgroup per compute unit holds it), NBUF - 1 tiles ahead of the one in
//    use. Each wave copies 8 rows of the next K and V tiles with
//    global_load_lds_dwordx4, so tile data never passes through registers. Rows
//    are stored unpadded, with the 16-byte chunk c of row r at position c ^ swz(r)
//    of the row, which keeps the operand reads below free of LDS bank conflicts
//    (the copy picks its source chunk so that each lane's destination stays the
//    contiguous 16 * lane the copy instruction writes).
//  * S^T = K Q^T with v_mfma_f32_32x32x16 (M = keys, N = queries, K = dims):
//    each lane then holds 16 keys of ONE query per 32-key half-tile, so the
//    row max needs only one v_permlane32_swap.
//  * O^T = V^T P^T (M = dims, N = queries, K = keys): each lane's output column
//    also belongs to one query, so the online-softmax rescale is lane-local.
//    The V^T operand (8 keys of one dim per lane) is read from the row-major V
//    tile with ds_read_b64_tr_b16, which hands lane j of a 16-lane group
//    element j % 4 of the 8-byte chunk fetched by lane 4e + j / 4, for e = 0..3.
//  * P rounded to bf16's 8 bits errs by up to ~3e-3 on rows with few keys, so
//    bf16 P V runs either on an f16 copy of V (written by stage_v_f16_kernel,
//    or by stage_paged_v_f16_kernel for paged keys; exact for every finite
//    bf16 value below 65520 in magnitude) with one 11-bit f16 P, or, where a
//    tile or block holds a larger value or no copy was made, with P split into
//    bf16 hi + lo parts (within ~1e-5 of exact). f16 inputs keep one f16 P.
//  * The K/V-position permutation inside one MFMA is shared by both operands
//    (it only has to be the same on A and B): lane half h = lane/32 holds keys
//    {16j + 8(i/4) + 4h + i%4 : i = 0..7} of 16-key group j, which is exactly
//    where the S^T accumulator put them.
//  * The running max only moves when a score passes it by more than TAU
//    (log2 units, checked with one ballot per tile), so the output rescale is
//    rare; p stays below 2^TAU and acc, l and m stay consistent either way.
//  * Causal: a workgroup visits key tiles up to its last query; tiles past a
//    wave's last query are skipped by that wave. Each XCD gets an equal,
//    contiguous share of the (head, query tile) items and starts the heaviest
//    (latest) query tiles of its share first.
//  * Sliding window (the walk-through's KV-cache section, sliding-window item,
//    which bounds the cache at W recent positions): the row at position p sees
//    p - W + 1 .. p. A workgroup starts at the tile holding its first row's
//    window start, and a wave skips tiles wholly before its first row's.
//  * ALiBi (the walk-through's position-encoding section): the score of row i
//    and key j gets -m_h (i - j), added in unscaled units with one
//    multiply-add per score.
#include <atomic>
#include <type_traits>

#include "launch.h"
#include "mfma.h"

namespace pa {

namespace {

constexpr int BN = 64;    // keys per tile
constexpr int WM = 32;    // query rows per wave
constexpr int NWAVES = PREFILL_WAVES;
constexpr int NBUF = 4;   // K/V tiles in the LDS ring
constexpr float TAU = 8.0f;        // rescale threshold (log2 units)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float M_FLOOR = -1e30f;  // running-max start: finite, so 2^(s - m) of a masked s is 0

template <int D> struct Tile {
    static constexpr int ROWB = D * 2;                  // bytes per K or V row
    static constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
    static constexpr int BYTES = BN * ROWB;             // one K or V tile
    static constexpr int COPIES = BYTES / (1024 * NWAVES);  // 1 KB copies per wave per tile
    static constexpr int BUF = 2 * BYTES;               // K tile, then V tile
    static constexpr int LDS = NBUF * BUF;              // the ring
    static_assert(COPIES * 1024 * NWAVES == BYTES, "a tile splits into whole 1 KB wave copies");
    static_assert(LDS <= 160 * 1024, "the ring fits one compute unit's LDS");
    static __device__ __forceinline__ int swz(int r) { return chunk_swizzle<CPR>(r); }
};

template <class E, int D, bool PAGED>
__global__ __launch_bounds__(64 * NWAVES, 1) void prefill_kernel(const PrefillArgs p) {
    using T = Tile<D>;
    using S = typename E::storage;
    constexpr int KK = D / 16;     // MFMA k-steps over the head dimension
    constexpr int MT = D / 32;     // 32-dim output tiles
    constexpr bool kStage = std::is_same<E, BF16>::value;   // V may come staged as f16
    extern __shared__ __attribute__((aligned(16))) char smem[];

    // Work item of this workgroup: query tile qt (RW = 256 / HPW rows) of head block hb
    // (HPW heads of one KV group) of sequence b. Items are numbered hb * nqt + r
    // (hb = b * n_q / HPW + head block; rank r = 0 is the heaviest causal tile, the last
    // rows). Workgroups go to the 8 XCDs in turn (XCD = id mod 8), so XCD k takes the
    // k-th contiguous eighth [a, e) of the items: whole head blocks apart from the two
    // ends, so every XCD gets the same mix of causal tile costs, and a KV head's work
    // stays on one XCD's L2. On its XCD, the j-th workgroup takes the j-th item of
    // [a, e) in (rank, head block) order: all heaviest tiles first, as in longest-first
    // scheduling. C(r), the number of items of [a, e) with rank below r, is
    // (e / nqt - a / nqt) r + min(r, e % nqt) - min(r, a % nqt); the rank is the
    // largest r with C(r) <= j, and the head blocks holding rank r are consecutive
    // from ceil((a - r) / nqt).
    const int HPW = p.hpw;
    const int RW = NWAVES * WM / HPW;             // query rows per workgroup
    const int nqt = p.seq_len / RW + (p.seq_len % RW != 0);
    const int n_items = gridDim.x;
    const int wg = blockIdx.x;
    const int per_xcd = n_items / 8, xcd = wg % 8;
    const int ia = xcd * per_xcd + min(xcd, n_items % 8);
    const int ie = ia + per_xcd + (xcd < n_items % 8);
    int jx = wg / 8;
    // When the whole grid is resident at once, the second half of an XCD's share goes
    // lightest first, so that workgroups that share the chip at the end pair heavy
    // tiles with light ones.
    if (n_items <= p.resident_wgs && jx >= (ie - ia) / 2) jx = (ie - ia) - 1 - (jx - (ie - ia) / 2);
    const int fa = ia / nqt, ra = ia % nqt, fe = ie / nqt, re = ie % nqt;
    auto below = [&](int r) { return (fe - fa) * r + min(r, re) - min(r, ra); };
    int qr = 0;
    for (int hi = nqt - 1; qr < hi;) {   // uniform: a binary search on scalars
        const int mid = (qr + hi + 1) / 2;
        if (below(mid) <= jx) qr = mid; else hi = mid - 1;
    }
    const int hb = fa + (qr < ra ? 1 : 0) + (jx - below(qr));
    const int qt = p.causal ? nqt - 1 - qr : qr;
    const int n_hb = p.n_q / HPW;                 // head blocks per sequence
    const int b = hb / n_hb;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = (hb % n_hb) * HPW + wave % HPW;   // this wave's query head
    const int g = (hb % n_hb) * HPW / p.group;      // the workgroup's KV head
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;    // 0 or 1
    const int l32 = lane & 31;
    const int q0 = qt * RW + (wave / HPW) * WM;   // first query row of this wave
    const int my_q = q0 + l32;                    // the query row this lane's columns belong to
    const int S_len = p.seq_len;                  // query rows per sequence

    // Keys: contiguous K/V hold exactly the S_len positions of the rows; paged
    // K/V hold ctx positions reached through the block table, and the rows are
    // the last S_len of them (causal, aligned at the bottom right). A context
    // past the block table's reach or a block id outside the pool makes every
    // row of the sequence NaN instead of reading out of bounds.
    int ctx = S_len;
    bool bad = false;
    if constexpr (PAGED) {
        ctx = load_uniform(p.context_lens + b);
        if (ctx < 0 || ctx > p.max_blocks * 16) {
            bad = ctx > 0;
            ctx = 0;
        }
    }
    const int qbase = ctx - S_len;                // position of query row 0
    const int pos0 = qbase + q0;                  // position of this wave's first row
    const int my_pos = qbase + my_q;              // position of this lane's query

    const int64_t q_stride = (int64_t)p.n_q * D;       // elements between query positions
    const int64_t kv_row = (int64_t)p.n_kv * D * 2;    // bytes between key positions
    const S* Qg = reinterpret_cast<const S*>(p.q) + (int64_t)b * S_len * q_stride + (int64_t)h * D;
    // Contiguous rows interleave the KV heads; a pool block holds one 16-row tile per KV head.
    const int64_t head_off = PAGED ? (int64_t)g * 16 * D * 2 : (int64_t)g * D * 2 + (int64_t)b * S_len * kv_row;
    const char* Kg = reinterpret_cast<const char*>(p.k) + head_off;
    const char* Vg = reinterpret_cast<const char*>(p.v) + head_off;   // the f16 copy when staged (below)

    // Q^T operand: lane holds dims 16*kk + 8*half .. +8 of its query, for every kk.
    // (Rows past the prompt load its last row, all loads in flight together, and are zeroed.)
    u32x4_t qreg[KK];
    const int q_row = min(my_q, S_len - 1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const uint4 v = q_fold(*reinterpret_cast<const uint4*>(Qg + (int64_t)q_row * q_stride + 16 * kk + 8 * half),
                               p.q_and, p.q_xor);
        qreg[kk] = u32x4_t{v.x, v.y, v.z, v.w};
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        if (my_q >= S_len) qreg[kk] = u32x4_t{0u, 0u, 0u, 0u};

    // Key tiles this workgroup visits (none when its last query sees no key).
    const int pos_last_wg = qbase + min(qt * RW + RW, S_len) - 1;
    const int n_tiles = ctx == 0 ? 0
                        : p.causal ? (pos_last_wg < 0 ? 0 : min(pos_last_wg, ctx - 1) / BN + 1)
                                   : (ctx + BN - 1) / BN;
    const int pos_last_wave = qbase + min(q0 + WM, S_len) - 1;
    // Sliding window (causal): row at position p sees p - W + 1 .. p. Tiles wholly
    // before the workgroup's first row's window are skipped, and no block before
    // it is read (their table entries may be stale).
    const int W = p.window;
    const int wg_lo = W > 0 ? max(0, qbase + qt * RW - W + 1) : 0;
    const int j0 = min(wg_lo / BN, n_tiles);
    const int lo_blk = wg_lo / 16;
    const int wave_lo = pos0 - W + 1;             // window start of this wave's first row
    const int wave_lo_max = pos_last_wave - W + 1; // ... and of its last row

    // bf16 values staged as f16 (exact where this sequence's flags say so): the
    // P V product then runs on the f16 matrix cores with one 11-bit P part
    // instead of two bf16 parts. Every wave checks the same tiles, so the choice
    // is uniform over the workgroup.
    // Paged keys: the copy holds the blocks this call reads, indexed by (sequence,
    // logical block), with one flag per block; the blocks a workgroup reads are
    // those from its first tile (or window block) to the context's last.
    bool use16 = false;
    if constexpr (kStage) {
        if (p.v16 != nullptr) {
            bool fits = true;
            if constexpr (PAGED) {
                const uint8_t* ok = p.v16_ok + ((int64_t)b * p.n_kv + g) * p.max_blocks;
                const int blo = max(j0 * (BN / 16), lo_blk);
                const int bhi = min(n_tiles * (BN / 16), (ctx + 15) / 16);
                for (int jb = blo + lane; jb < bhi; jb += 64) fits = fits && ok[jb] != 0;
            } else {
                const uint8_t* ok = p.v16_ok + ((int64_t)b * p.n_kv + g) * (S_len / BN + (S_len % BN != 0));
                for (int j = j0 + lane; j < n_tiles; j += 64) fits = fits && ok[j] != 0;
            }
            use16 = __all(fits);
        }
    }
    if (use16) Vg = reinterpret_cast<const char*>(p.v16) + head_off;
    const bool v_logical = PAGED && use16;   // V blocks addressed by logical index

    // This wave's copies of tile j into ring slot `buf`: copy c fills bytes
    // [(wave * COPIES + c) KB, +1 KB) of the K tile and of the V tile, lane l
    // the 16 bytes at 16 l of that, which hold source chunk pos ^ swz(row).
    // A wave's copies cover rows 8 wave .. 8 wave + 7 of the tile, i.e. half of
    // one 16-token cache block when the keys are paged. Rows past the context
    // read its last row instead, and rows of blocks wholly before the window
    // read the window's first row (each in the block the clamped block index
    // names): their keys are masked, and their V rows must be finite because
    // the P V product multiplies them by exactly 0.
    static_assert(T::COPIES * 1024 == 8 * T::ROWB, "a wave copies 8 rows of a tile");
    const uint32_t lds0 = lds_addr(smem);
    // Tiles that need no row clamp (wholly inside [window start, ctx)) copy from a
    // wave-uniform base plus lane offsets fixed for the whole kernel: row r of the
    // tile is key key0 + r, at r * kv_row from the tile's first key (contiguous),
    // or at (r % 16) * ROWB inside the wave's block (paged).
    uint32_t lane_src[T::COPIES];
#pragma unroll
    for (int c = 0; c < T::COPIES; ++c) {
        const int off = (wave * T::COPIES + c) * 1024 + 16 * lane;
        const int r = off / T::ROWB;
        const int chunk = ((off % T::ROWB) / 16) ^ T::swz(r);
        lane_src[c] = PAGED ? (uint32_t)((r % 16) * T::ROWB + chunk * 16) : (uint32_t)(r * kv_row + chunk * 16);
    }
    const bool lane_src_fits = PAGED || (int64_t)BN * kv_row < ((int64_t)1 << 31);
    auto issue_tile = [&](int j, int buf) {
        const int key0 = j * BN;
        int64_t block_src = 0, vblock_src = 0;
        if constexpr (PAGED) {
            const int jb = max(min(key0 / 16 + wave / 2, (ctx - 1) / 16), lo_blk);   // uniform over the wave
            int phys = load_uniform(p.block_table + (int64_t)b * p.max_blocks + jb);
            if (phys < 0 || phys >= p.num_blocks) {
                bad = true;
                phys = 0;
            }
            block_src = (int64_t)phys * p.n_kv * 16 * T::ROWB;
            vblock_src = v_logical ? ((int64_t)b * p.max_blocks + jb) * p.n_kv * 16 * T::ROWB : block_src;
        }
        if (lane_src_fits && key0 >= wg_lo && key0 + BN <= ctx) {   // uniform
            const int64_t base = PAGED ? block_src : (int64_t)key0 * kv_row;
            const int64_t vbase = PAGED ? vblock_src : base;
#pragma unroll
            for (int c = 0; c < T::COPIES; ++c) {
                const uint32_t dst = lds0 + buf * T::BUF + (wave * T::COPIES + c) * 1024;
                copy_to_lds16(Kg + base, lane_src[c], dst);
                copy_to_lds16(Vg + vbase, lane_src[c], dst + T::BYTES);
            }
            return;
        }
#pragma unroll
        for (int c = 0; c < T::COPIES; ++c) {
            const int off = (wave * T::COPIES + c) * 1024 + 16 * lane;
            const int r = off / T::ROWB;
            const int chunk = ((off % T::ROWB) / 16) ^ T::swz(r);
            // The key this lane's row holds: rows past the context read its last
            // key, rows before the window its first (both masked, both finite).
            const int t = max(min(key0 + r, ctx - 1), wg_lo);
            const int64_t in_blk = (int64_t)(t % 16) * T::ROWB + chunk * 16;
            const int64_t src = PAGED ? block_src + in_blk : (int64_t)t * kv_row + chunk * 16;
            const int64_t vsrc = PAGED ? vblock_src + in_blk : src;
            const uint32_t dst = lds0 + buf * T::BUF + (wave * T::COPIES + c) * 1024;
            copy_to_lds16(Kg + src, dst);
            copy_to_lds16(Vg + vsrc, dst + T::BYTES);
        }
    };

    // The tile copies are invisible to the compiler's wait counting: make it
    // wait for q here, before the first copy, rather than inside the loop where
    // its wait would also drain the prefetch of the next tile.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : : "v"(qreg[kk]));

    f32x16_t o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16_t{};
    float m_run = M_FLOOR;     // running max (log2 units) of this lane's query
    float l_run = 0.f;         // this lane's share of the softmax denominator
    // ALiBi: the bias -m_h (i - j) is a (j - i) in unscaled score units, a = m_h / scale.
    // For the element at offset c of a lane's tile, j - i = (key0 + 4 half - my_pos) + c:
    // the part a c (c a compile-time constant) is one multiply-add per score, and the
    // lane's part a (key0 + 4 half - my_pos) shifts its tile max and exponent instead.
    const bool alibi = p.alibi != nullptr;   // uniform
    const float a_sl = alibi ? p.alibi[h] * LOG2E / p.scale_log2 : 0.f;
    const float c2 = p.scale_log2;

    // Lane-constant parts of the operand addresses (the swizzle of a row depends on
    // its index mod 16 only, so key 32 st + 16 jg + 8 t + vkey shares it with 8 t + vkey).
    const int ksw = T::swz(l32);                 // rows l32 and 32 + l32 share it
    const int g16 = lane >> 4, r16 = lane & 15;  // 16-lane group and lane within it
    const int vkey = 4 * half + r16 / 4;         // + 16 jg + 8 t + 32 st
    const int vchunk = 2 * (g16 & 1) + (r16 & 3) / 2;  // + 4 mt
    const int vbyte = 8 * (r16 & 1);
    // K operand: row l32, 16-byte chunk 2 kk + half, stored at chunk (2 kk + half) ^ ksw.
    // As 2 kk + half = 2 kk ^ half, its byte offset is k_base ^ 32 kk (the XOR only
    // touches bits 5..7, below the row's bits).
    const uint32_t k_base = l32 * T::ROWB + ((half ^ ksw) * 16);
    auto k_off = [&](int kk) { return k_base ^ (uint32_t)(32 * kk); };
    // V^T operand: key 8 t + vkey, chunk 4 mt + vchunk (vchunk < 4, so that sum is an XOR),
    // stored at chunk (4 mt + vchunk) ^ swz(8 t + vkey): byte offset vt_base[t] ^ 64 mt.
    uint32_t vt_base[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        vt_base[t] = (8 * t + vkey) * T::ROWB + ((vchunk ^ T::swz(8 * t + vkey)) * 16) + vbyte;
    auto vt_off = [&](int t, int mt) { return vt_base[t] ^ (uint32_t)(64 * mt); };

    // The tile loop, for P V in the input type (PE = E) or on the staged f16 V.
    auto tile_loop = [&](auto staged) {
        using PE = typename std::conditional<decltype(staged)::value, F16, E>::type;
        // Ring: tiles j0 .. j0 + NBUF - 2 are copied first; step j then waits for tile j,
        // and once every wave is done with tile j - 1 copies tile j + NBUF - 1 into its
        // slot. Copies complete in issue order, so tile j has landed when at most the
        // copies of the tiles issued after it are outstanding.
        for (int t = 0; t < NBUF - 1; ++t)
            if (j0 + t < n_tiles) issue_tile(j0 + t, (j0 + t) % NBUF);
        for (int j = j0; j < n_tiles; ++j) {
            const int ahead = min(n_tiles - 1, j + NBUF - 2) - j;   // tiles issued after j
            static_assert(NBUF == 4, "the waits below cover up to two tiles in flight after j");
            if (ahead >= 2) wait_vmcnt<4 * T::COPIES>();
            else if (ahead == 1) wait_vmcnt<2 * T::COPIES>();
            else wait_vmcnt<0>();
            __syncthreads();   // the other waves' copies of tile j landed; all are done with tile j - 1
            if (j + NBUF - 1 < n_tiles) issue_tile(j + NBUF - 1, (j + NBUF - 1) % NBUF);
            const int key0 = j * BN;
            if (p.causal && key0 > pos_last_wave) continue;   // uniform over the wave
            if (W > 0 && key0 + BN - 1 < wave_lo) continue;   // wholly before every row's window

            const char* kl = smem + (j % NBUF) * T::BUF;
            lds_char_t* vl_lds = (lds_char_t*)(smem + (j % NBUF) * T::BUF + T::BYTES);

            // S^T for the two 32-key halves, interleaved so each MFMA hides the other's latency.
            // Operands of k-step kk + 2 are read before the products of k-step kk, so two
            // steps of LDS reads are in flight behind the matrix cores.
            f32x16_t sc[2] = {f32x16_t{}, f32x16_t{}};
            uint4 ka[3][2];
            auto k_read = [&](int kk, uint4 (&a)[2]) {
                a[0] = *reinterpret_cast<const uint4*>(kl + k_off(kk));
                a[1] = *reinterpret_cast<const uint4*>(kl + k_off(kk) + 32 * T::ROWB);
            };
            k_read(0, ka[0]);
            k_read(1, ka[1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if (kk + 2 < KK) k_read(kk + 2, ka[(kk + 2) % 3]);
                const uint4 a0 = ka[kk % 3][0], a1 = ka[kk % 3][1];
                sc[0] = Mfma<E>::run(u32x4_t{a0.x, a0.y, a0.z, a0.w}, qreg[kk], sc[0]);
                sc[1] = Mfma<E>::run(u32x4_t{a1.x, a1.y, a1.z, a1.w}, qreg[kk], sc[1]);
                __builtin_amdgcn_sched_barrier(0);
            }

            float lane_bias = 0.f;   // ALiBi bias shared by the lane's scores (unscaled units)
            if (alibi) {   // key = key0 + 32 st + 8 (i / 4) + 4 half + i % 4
                lane_bias = a_sl * (float)(key0 + 4 * half - my_pos);
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        sc[st][i] = fmaf(a_sl, (float)(32 * st + (i / 4) * 8 + (i % 4)), sc[st][i]);
            }
            // Mask keys past this lane's query (causal), past the prompt, or before
            // this lane's window.
            if (key0 + BN > ctx || (p.causal && key0 + BN - 1 > pos0) || (W > 0 && key0 < wave_lo_max)) {   // uniform
                const int lim = (p.causal ? min(my_pos, ctx - 1) : ctx - 1) - key0;
                const int lo = (W > 0 ? my_pos - W + 1 : 0) - key0;
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = st * 32 + (i / 4) * 8 + half * 4 + (i % 4);
                        sc[st][i] = (key > lim || key < lo) ? -INFINITY : sc[st][i];
                    }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[st][i]);
            {
                float a2, b2;
                pair32(tmax + lane_bias, a2, b2);
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

            // P = 2^((s + lane_bias) scale - m) in the element type (bf16: hi + lo parts).
            const float nm = fmaf(lane_bias, c2, -m_run);
            auto v_read = [&](int st, int jg, int mt) -> u32x4_t {   // V^T operand, see vt_off
                uint32_t a[4];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4_t*)(vl_lds + (st * 32 + jg * 16) * T::ROWB + vt_off(t, mt)));
                    a[2 * t] = __builtin_bit_cast(uint2, v).x;
                    a[2 * t + 1] = __builtin_bit_cast(uint2, v).y;
                }
                return u32x4_t{a[0], a[1], a[2], a[3]};
            };
            if constexpr (!Mfma<PE>::kSplit) {
                // One f16 P part: group u = 2 st + jg of 16 keys; its P words are made on the
                // VALU while the P V products of group u - 1 run, and each V^T operand is
                // read two products ahead.
                float lsum = 0.f;
                auto p_word = [&](int u, int w) {
                    const int st = u / 2, jg = u % 2;
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[st][8 * jg + 2 * w], c2, nm));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[st][8 * jg + 2 * w + 1], c2, nm));
                    const uint32_t hw = Mfma<PE>::pack(p0, p1);
                    // the denominator of the rounded weights the product uses
                    lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, hw),
                                                  f16x2_t{(_Float16)1.f, (_Float16)1.f}, lsum, false);
                    return hw;
                };
                u32x4_t pw[2];
                {
                    uint32_t w4[4];
#pragma unroll
                    for (int w = 0; w < 4; ++w) w4[w] = p_word(0, w);
                    pw[0] = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
                }
                constexpr int NU = 4 * MT;   // products: (group u, dims mt)
                u32x4_t vv[3];
                static_assert(MT >= 2, "the first two products are (group 0, dims 0) and (group 0, dims 32)");
                vv[0] = v_read(0, 0, 0);
                vv[1] = v_read(0, 0, 1);
                __builtin_amdgcn_sched_barrier(0);
                uint32_t nxt[4];
#pragma unroll
                for (int i = 0; i < NU; ++i) {
                    const int u = i / MT, mt = i % MT;
                    if (i + 2 < NU) {
                        const int i2 = i + 2, u2 = i2 / MT, m2 = i2 % MT;
                        vv[i2 % 3] = v_read(u2 / 2, u2 % 2, m2);
                    }
                    o[mt] = Mfma<PE>::run(vv[i % 3], pw[u % 2], o[mt]);
                    // P words of group u + 1, spread over group u's products
                    if (u + 1 < 4) {
#pragma unroll
                        for (int w = mt * 4 / MT; w < (mt + 1) * 4 / MT; ++w) nxt[w] = p_word(u + 1, w);
                        if (mt == MT - 1) pw[(u + 1) % 2] = u32x4_t{nxt[0], nxt[1], nxt[2], nxt[3]};
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                l_run += lsum;
            } else {
                u32x4_t ph[2][2], pl[2][2];   // [half-tile][16-key group]
                float lsum = 0.f;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
#pragma unroll
                    for (int jg = 0; jg < 2; ++jg) {
                        uint32_t hw[4], lw[4];
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[st][8 * jg + 2 * w], c2, nm));
                            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[st][8 * jg + 2 * w + 1], c2, nm));
                            hw[w] = Mfma<PE>::pack(p0, p1);
                            lw[w] = Mfma<PE>::pack(p0 - Mfma<PE>::lo_of(hw[w]), p1 - Mfma<PE>::hi_of(hw[w]));
                            lsum += p0 + p1;
                        }
                        ph[st][jg] = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
                        pl[st][jg] = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
                    }
                }
                l_run += lsum;
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int jg = 0; jg < 2; ++jg)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            const u32x4_t av = v_read(st, jg, mt);
                            o[mt] = Mfma<PE>::run(av, ph[st][jg], o[mt]);
                            o[mt] = Mfma<PE>::run(av, pl[st][jg], o[mt]);
                        }
            }
        }
    };
    if constexpr (kStage) {
        if (use16)
            tile_loop(std::true_type{});
        else
            tile_loop(std::false_type{});
    } else {
        tile_loop(std::false_type{});
    }

    // Denominator: this lane and its partner (lane ^ 32) covered complementary keys.
    {
        float a2, b2;
        pair32(l_run, a2, b2);
        l_run = a2 + b2;
    }
    if constexpr (PAGED) bad = __syncthreads_or(bad);   // a bad block anywhere spoils the tiles
    if (my_q >= S_len) return;
    const float inv = bad ? NAN : l_run > 0.f ? 1.f / l_run : 0.f;
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

// f16 copy of bf16 V for the staged P V product: f16 keeps 11 significant bits
// to bf16's 8, so every finite bf16 value below 65520 in magnitude converts
// exactly, except those below f16's normal range (2^-14), which move by at most
// 2^-25. One workgroup per (64-key tile, KV head, sequence) also records whether
// any finite value of its tile overflowed (flag 0: the prefill keeps bf16 there).
// Eight bf16 values (one 16-byte chunk) as f16. `bad` is set when a finite value
// overflows f16; every other finite bf16 value converts exactly (values below
// 2^-14 move by at most 2^-25).
__device__ __forceinline__ uint4 bf16x8_to_f16(const uint4 w, bool& bad) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t o16[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x0 = as_f32(in[i] << 16), x1 = as_f32(in[i] & 0xffff0000u);
        const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
        bad = bad || (__builtin_isinf((float)h0) && !__builtin_isinf(x0)) ||
              (__builtin_isinf((float)h1) && !__builtin_isinf(x1));
        const f16x2_t hv = {h0, h1};
        o16[i] = __builtin_bit_cast(uint32_t, hv);
    }
    return make_uint4(o16[0], o16[1], o16[2], o16[3]);
}

// Contiguous bf16 V: one workgroup per (64-key tile, KV head, sequence) writes the
// f16 copy of its tile in V's layout and flags whether the copy is exact. Each
// thread loads all its chunks before it stores any, so the loads overlap.
template <int D> __global__ __launch_bounds__(256) void stage_v_f16_kernel(const PrefillArgs p) {
    constexpr int CPR = D * 2 / 16;                // 16-byte chunks (8 values) per row
    constexpr int PER = BN * CPR / 256;            // chunks per thread
    static_assert(PER * 256 == BN * CPR, "a tile splits evenly over 256 threads");
    const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int S_len = p.seq_len;
    int64_t off[PER];
    uint4 w[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int t = tile * BN + c / CPR;
        off[i] = t < S_len ? (((int64_t)b * S_len + t) * p.n_kv + g) * D + (c % CPR) * 8 : -1;
        if (off[i] >= 0) w[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.v) + off[i]);
    }
    bool bad = false;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if (off[i] >= 0)
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.v16) + off[i]) = bf16x8_to_f16(w[i], bad);
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) p.v16_ok[((int64_t)b * p.n_kv + g) * gridDim.x + tile] = bad ? 0 : 1;
}

// Paged bf16 V (chunked prefill): one workgroup per (4 logical blocks, KV head,
// sequence) copies the rows below the context length of each block to
// v16[b][block][g][16][D] as f16 and flags it in v16_ok[b][g][block]. Blocks at or
// past the context are never read and get no flag; a block id outside the pool
// gets flag 0 and is not read (the prefill kernel reports that sequence as bad).
// Each thread loads its chunk of all 4 blocks before it stores any.
constexpr int STAGE_BLOCKS = 4;   // logical blocks per staging workgroup
template <int D> __global__ __launch_bounds__(256) void stage_paged_v_f16_kernel(const PrefillArgs p) {
    constexpr int CPR = D * 2 / 16;
    static_assert(16 * CPR <= 256, "one chunk of a block per thread");
    const int g = blockIdx.y, b = blockIdx.z;
    const int ctx = p.context_lens[b];
    if (ctx <= 0 || ctx > p.max_blocks * 16) return;   // uniform
    const int lb0 = blockIdx.x * STAGE_BLOCKS;
    if (lb0 * 16 >= ctx) return;                        // uniform
    const int c = threadIdx.x;
    int rows[STAGE_BLOCKS];
    bool live[STAGE_BLOCKS], ok[STAGE_BLOCKS];
    uint4 w[STAGE_BLOCKS];
#pragma unroll
    for (int i = 0; i < STAGE_BLOCKS; ++i) {   // uniform per block
        const int lb = lb0 + i;
        live[i] = lb * 16 < ctx;               // then lb < max_blocks too
        const int phys = live[i] ? p.block_table[(int64_t)b * p.max_blocks + lb] : -1;
        ok[i] = live[i] && phys >= 0 && phys < p.num_blocks;
        rows[i] = ok[i] ? min(16, ctx - lb * 16) : 0;
        if (c < rows[i] * CPR)
            w[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.v) +
                                                  ((int64_t)phys * p.n_kv + g) * 16 * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < STAGE_BLOCKS; ++i) {
        bool bad = false;
        if (c < rows[i] * CPR) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(p.v16) +
                            (((int64_t)b * p.max_blocks + lb0 + i) * p.n_kv + g) * 16 * D;
            *reinterpret_cast<uint4*>(dst + c * 8) = bf16x8_to_f16(w[i], bad);
        }
        bad = __syncthreads_or(bad);           // every thread, every block: uniform trip count
        if (threadIdx.x == 0 && live[i])
            p.v16_ok[((int64_t)b * p.n_kv + g) * p.max_blocks + lb0 + i] = ok[i] && !bad ? 1 : 0;
    }
}

template <class E, int D, bool PAGED> hipError_t launch_typed(const PrefillArgs& args, hipStream_t s) {
    PrefillArgs a = args;
    a.resident_wgs = device_cus();   // one 8-wave workgroup and its ring per compute unit
    a.hpw = prefill_heads_per_wg(a.group);
    const size_t lds = (size_t)Tile<D>::LDS;
    // Opt in to exactly the dynamic LDS used (static LDS, e.g. the one word
    // __syncthreads_or needs, counts against the same 160 KB).
    static const hipError_t opt_in = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&prefill_kernel<E, D, PAGED>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (opt_in != hipSuccess) return opt_in;
    if constexpr (std::is_same<E, BF16>::value) {
        if (a.v16 != nullptr) {
            if constexpr (PAGED) {
                const dim3 sgrid((a.max_blocks + STAGE_BLOCKS - 1) / STAGE_BLOCKS, a.n_kv, a.batch);
                hipLaunchKernelGGL((stage_paged_v_f16_kernel<D>), sgrid, dim3(256), 0, s, a);
            } else {
                const dim3 sgrid(a.seq_len / BN + (a.seq_len % BN != 0), a.n_kv, a.batch);
                hipLaunchKernelGGL((stage_v_f16_kernel<D>), sgrid, dim3(256), 0, s, a);
            }
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    const int64_t rw = NWAVES * WM / a.hpw;
    const int64_t n_items = ((int64_t)a.seq_len + rw - 1) / rw * (a.n_q / a.hpw) * a.batch;
    if (!prefill_grid_fits(a.seq_len, a.n_q, a.batch, a.group)) return hipErrorInvalidConfiguration;   // checked by the caller
    const dim3 grid((unsigned)n_items);
    hipLaunchKernelGGL((prefill_kernel<E, D, PAGED>), grid, dim3(64 * NWAVES), lds, s, a);
    return hipGetLastError();
}

template <class E, int D> hipError_t launch_kv(const PrefillArgs& a, hipStream_t s) {
    return a.block_table ? launch_typed<E, D, true>(a, s) : launch_typed<E, D, false>(a, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, Elem e, int head_dim, hipStream_t s) {
    if (e == Elem::BF16 && head_dim == 128) return launch_kv<BF16, 128>(a, s);
    if (e == Elem::BF16 && head_dim == 64) return launch_kv<BF16, 64>(a, s);
    if (e == Elem::F16 && head_dim == 128) return launch_kv<F16, 128>(a, s);
    if (e == Elem::F16 && head_dim == 64) return launch_kv<F16, 64>(a, s);
    return hipErrorNotSupported;
}

}  // namespace pa
