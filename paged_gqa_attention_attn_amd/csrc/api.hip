// api.hip -- C-ABI entry points: argument validation, launch planning, error reporting,
// the workspace (decode partials, prefill staging).
//
// By default no entry point reads device memory on the host or synchronises the
// stream: every check uses host-side arguments only, and the kernels bounds-check
// the device-resident metadata themselves. With the PA_OPT_VALIDATE option on,
// the calls also copy that metadata to the host (synchronising the stream) and
// reject what the kernels would only skip or turn into NaN rows. See
// include/pagedattn.h for the contract of each call.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "launch.h"
#include "pagedattn.h"

namespace pa {

int device_cus() {
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace pa

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pa_dtype d) {
    switch (d) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_F16: return 2;
    case PA_FP8_E4M3: return 1;
    case PA_INT8: return 1;
    case PA_FP8_E4M3_PER_CHANNEL: return 1;
    case PA_INT8_PER_CHANNEL: return 1;
    }
    return 0;
}

bool is_quant(pa_dtype d) {
    return d == PA_FP8_E4M3 || d == PA_INT8 || d == PA_FP8_E4M3_PER_CHANNEL || d == PA_INT8_PER_CHANNEL;
}
// One-byte codes with fixed per-channel scales [n_kv][head_dim] instead of per-row ones.
bool is_per_channel(pa_dtype d) { return d == PA_FP8_E4M3_PER_CHANNEL || d == PA_INT8_PER_CHANNEL; }
pa::QuantFmt fmt_of(pa_dtype d) {
    return d == PA_FP8_E4M3 || d == PA_FP8_E4M3_PER_CHANNEL ? pa::QuantFmt::FP8_E4M3 : pa::QuantFmt::INT8;
}

pa::Elem to_elem(pa_dtype d) { return static_cast<pa::Elem>(static_cast<int>(d)); }

constexpr float kLog2e = 1.4426950408889634f;

// The scale multiplying q.k, as the kernels take it: a positive factor |scale| log2(e)
// and a fold of q's words ((word & q_and) ^ q_xor at load). A negative scale flips
// the sign bits of q, which negates every q.k exactly; a zero scale zeroes q, so
// every score is exactly 0 (the product of 0 and a finite q.k) and the factor is
// an arbitrary positive one. Non-finite scales are rejected.
template <class Args> int fold_scale(float scale, pa_dtype q_dtype, Args* a) {
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    const uint32_t sign = q_dtype == PA_F32 ? 0x80000000u : 0x80008000u;
    a->q_and = scale == 0.f ? 0u : ~0u;
    a->q_xor = scale < 0.f ? sign : 0u;
    a->scale_log2 = scale == 0.f ? kLog2e : std::fabs(scale) * kLog2e;
    return PA_OK;
}

std::atomic<int32_t> g_partition_tokens{0};

constexpr int kBlockSize = 16;
constexpr int kMaxWaves = 8;
constexpr int kLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950

// Kernel-choice options: each starts from its environment variable, read once
// when an option is first needed (unset, unparsable or out of range: the
// default), and afterwards changes only through pa_set_option.
struct OptionSpec {
    const char* env;
    int32_t dflt, lo, hi;
};
constexpr OptionSpec kOptions[PA_OPT_COUNT] = {
    {"PA_DECODE_MFMA", 1, 0, 1},     {"PA_DECODE_RING", 1, 1, 2}, {"PA_DECODE_WAVES", 0, 0, kMaxWaves},
    {"PA_PREFILL_STAGE_V", 1, 0, 1}, {"PA_VALIDATE", 0, 0, 1},
};

std::atomic<int32_t>* option_values() {
    static std::atomic<int32_t> v[PA_OPT_COUNT];
    static std::once_flag once;
    std::call_once(once, [] {
        for (int i = 0; i < PA_OPT_COUNT; ++i) {
            const OptionSpec& o = kOptions[i];
            int32_t x = o.dflt;
            if (const char* e = std::getenv(o.env); e && *e) {
                char* end = nullptr;
                const long y = std::strtol(e, &end, 10);
                if (end && *end == 0 && y >= o.lo && y <= o.hi) x = (int32_t)y;
            }
            v[i].store(x, std::memory_order_relaxed);
        }
    });
    return v;
}

int32_t option(pa_option o) { return option_values()[o].load(std::memory_order_relaxed); }

// Sizes and types of a cache description. Quantised caches (one-byte codes plus
// per-row scales) are accepted only by the entry points that take the scales.
int check_cache(const pa_cache_desc* c, bool allow_quant = false) {
    if (!c) return fail(PA_ERR_INVALID_ARG, "cache descriptor is NULL");
    if (c->num_blocks <= 0 || c->n_kv <= 0 || c->head_dim <= 0 || c->block_size <= 0)
        return fail(PA_ERR_INVALID_ARG,
                    "cache sizes must be positive (num_blocks=%d n_kv=%d head_dim=%d block_size=%d)",
                    c->num_blocks, c->n_kv, c->head_dim, c->block_size);
    if (elem_bytes(c->dtype) == 0) return fail(PA_ERR_UNSUPPORTED, "unknown cache dtype %d", (int)c->dtype);
    if (is_quant(c->dtype) && !allow_quant)
        return fail(PA_ERR_UNSUPPORTED,
                    "a quantised cache (dtype %d) needs pa_kv_append_quant / pa_paged_attn_decode_quant",
                    (int)c->dtype);
    if (c->block_size != kBlockSize)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d has no kernel (supported: 16)", c->block_size);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d has no kernel (supported: 64, 128)", c->head_dim);
    return PA_OK;
}

// Decode launch plan; a pure function of the host arguments so that
// pa_decode_workspace_bytes and pa_paged_attn_decode always agree.
struct Plan {
    int32_t gw, hs_wg, hsg, waves_tok, blocks_per_wave, nparts_max, ring, mfma;
    size_t ws_floats_m, ws_floats_acc;  // floats in m (== l) and acc arrays
};

// Decode on the matrix cores (decode_mfma.hip) for bf16/f16 caches whose group
// size fills 4, 8 or 16 MFMA columns, unless the option selects the VALU kernel.
bool decode_uses_mfma(int32_t G, const pa_cache_desc* c) {
    if (c->dtype != PA_BF16 && c->dtype != PA_F16) return false;
    if (G % 4 != 0) return false;
    return option(PA_OPT_DECODE_MATRIX_CORES) != 0;
}

// LDS bytes one wave of the matrix-core decode kernel takes: its ring, or the
// merge slot of `hw` heads (acc rows padded by 4 floats, then m and l) if larger.
int32_t mfma_wave_bytes(int32_t ring, int32_t tile, int32_t hw, int32_t head_dim) {
    const int32_t slot = (hw * (head_dim + 4) + 2 * hw) * 4;
    const int32_t r = ring * 2 * tile;
    return ((r > slot ? r : slot) + 15) / 16 * 16;
}

// Matrix-core decode plan: a grid of about 8 waves per compute unit, each
// streaming as long a run of blocks as that allows (4 to 64 blocks), with the
// partitions of a context balanced. Measured on MI355X: larger runs and fewer
// resident waves stream faster (8B-, 70B-shaped, variable-length and
// sliding-window workloads), as long as every compute unit has work.
int64_t target_waves() { return 8 * (int64_t)pa::device_cus(); }

// Runs of blocks per wave and partitions for `w` waves per workgroup.
void mfma_partitions(int64_t units, int32_t span, int32_t w, int32_t* bpw, int32_t* nparts) {
    int32_t tokens = g_partition_tokens.load();
    int32_t b;
    if (tokens > 0) {   // explicit partition size (pa_set_decode_partition_tokens)
        b = tokens / (w * kBlockSize);
    } else {
        const int64_t tw = target_waves();
        const int64_t want = (span * units + tw - 1) / tw;
        b = (int32_t)std::min<int64_t>(64, std::max<int64_t>(4, want));
        const int32_t p = (span + w * b - 1) / (w * b);
        b = (span + p * w - 1) / (p * w);   // balance the partitions
    }
    b = std::max(1, std::min(64, b));
    *bpw = b;
    *nparts = std::max(1, (span + w * b - 1) / (w * b));
}

int make_plan(int32_t batch, int32_t n_q, int32_t max_blocks, const pa_cache_desc* c, Plan* pl) {
    const int32_t G = n_q / c->n_kv;
    const bool quant = is_quant(c->dtype);
    const bool mfma = quant || decode_uses_mfma(G, c);
    // Query heads per wave. VALU kernel: 4 when the group allows it (keeps acc at
    // 64 fp32 registers for head_dim 128), else the largest power of two dividing
    // G. Matrix-core kernels: one workgroup slice of 16, 8 or 4 heads (MFMA
    // columns); the quantised-cache kernel also takes slices of 2 or 1.
    const int32_t gw = mfma ? (G % 16 == 0 ? 16 : G % 8 == 0 ? 8 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1)
                            : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
    const int32_t hs = G / gw;
    // Each wave keeps `ring` blocks of K and V in flight in its own LDS ring
    // (option PA_OPT_DECODE_RING: 1 or 2).
    const int32_t ring = option(PA_OPT_DECODE_RING);
    const int64_t units = (int64_t)batch * c->n_kv * hs;
    const int32_t tile = kBlockSize * c->head_dim * elem_bytes(c->dtype);
    int32_t hs_wg = 1, waves_tok, bpw, nparts_max;
    if (mfma) {
        waves_tok = option(PA_OPT_DECODE_WAVES);
        if (waves_tok == 0) waves_tok = kMaxWaves;
        const int32_t wave_lds = quant ? pa::quant_wave_bytes(c->head_dim, gw, ring)
                                       : mfma_wave_bytes(ring, tile, gw, c->head_dim);
        while (waves_tok > 1 && waves_tok * wave_lds > kLdsBytes) --waves_tok;
        mfma_partitions(units, max_blocks, waves_tok, &bpw, &nparts_max);
    } else {
        // VALU kernel: 8 waves when there are at least as many (sequence, KV head,
        // head slice) units as compute units, else 4 so that long contexts split
        // into more, smaller workgroups (option PA_OPT_DECODE_WAVES overrides);
        // 2048-token partitions unless overridden. The waves may also split over
        // head slices.
        int32_t max_waves = option(PA_OPT_DECODE_WAVES);
        if (max_waves == 0) max_waves = units >= pa::device_cus() ? kMaxWaves : 4;
        while (max_waves > 1 && max_waves * ring * 2 * tile > kLdsBytes) --max_waves;
        for (int32_t d = max_waves; d >= 1; --d)
            if (hs % d == 0) {
                hs_wg = d;
                break;
            }
        waves_tok = max_waves / hs_wg;
        int32_t tokens = g_partition_tokens.load();
        if (tokens <= 0) tokens = 2048;
        bpw = std::max(1, std::min(64, tokens / (waves_tok * kBlockSize)));
        nparts_max = std::max(1, (max_blocks + bpw * waves_tok - 1) / (bpw * waves_tok));
    }

    pl->gw = gw;
    pl->hs_wg = hs_wg;
    pl->hsg = hs / hs_wg;
    pl->waves_tok = waves_tok;
    pl->blocks_per_wave = bpw;
    pl->nparts_max = nparts_max;
    pl->ring = ring;
    pl->mfma = mfma ? 1 : 0;
    if (pl->nparts_max > 1) {
        pl->ws_floats_m = (size_t)batch * n_q * pl->nparts_max;
        pl->ws_floats_acc = pl->ws_floats_m * (size_t)c->head_dim;
    } else {
        pl->ws_floats_m = pl->ws_floats_acc = 0;
    }
    return PA_OK;
}

size_t round16(size_t n) { return (n + 15) & ~(size_t)15; }

// Workspace of a bf16 prefill over contiguous keys: the f16 copy of v, then one
// flag byte per (sequence, KV head, 64-key tile). Option PA_OPT_PREFILL_STAGE_V = 0
// turns the staging off (P V then stays in bf16 hi + lo parts).
bool prefill_stages(pa_dtype dtype) { return dtype == PA_BF16 && option(PA_OPT_PREFILL_STAGE_V) != 0; }
size_t prefill_stage_v_bytes(int32_t batch, int32_t seq_len, int32_t n_kv, int32_t head_dim) {
    return round16((size_t)batch * seq_len * n_kv * head_dim * 2);
}
size_t prefill_stage_bytes(int32_t batch, int32_t seq_len, int32_t n_kv, int32_t head_dim) {
    const size_t tiles = (size_t)batch * n_kv * (((size_t)seq_len + 63) / 64);
    return prefill_stage_v_bytes(batch, seq_len, n_kv, head_dim) + round16(tiles);
}
// The staging kernels take the sequence as grid z and the KV head as grid y.
bool stage_grid_fits(int32_t batch, int32_t n_kv) { return batch <= 65535 && n_kv <= 65535; }
// Chunked prefill over a bf16 cache: an f16 copy of the V blocks the call reads,
// [batch][max_blocks][n_kv][16][head_dim], then one flag byte per block. Staged only
// up to this size; beyond it P V keeps the bf16 hi + lo form.
constexpr size_t kChunkStageCap = (size_t)256 << 20;
size_t chunked_stage_v_bytes(int32_t batch, int32_t max_blocks, int32_t n_kv, int32_t head_dim) {
    return round16((size_t)batch * max_blocks * n_kv * 16 * head_dim * 2);
}
size_t chunked_stage_bytes(int32_t batch, int32_t max_blocks, int32_t n_kv, int32_t head_dim) {
    return chunked_stage_v_bytes(batch, max_blocks, n_kv, head_dim) + round16((size_t)batch * n_kv * max_blocks);
}

// Blocks one sequence's call can read: all of max_blocks without a window; with
// window W and `rows` query rows, the W + rows - 1 positions from the first
// row's window start to the last row, which touch at most (W + rows + 29) / 16
// blocks of 16 wherever they start. Partition counts and workspaces follow it.
int32_t span_blocks(int32_t max_blocks, int32_t rows, int32_t window) {
    if (window <= 0) return max_blocks;
    const int64_t span = ((int64_t)window + rows - 1 + 2 * (kBlockSize - 1)) / kBlockSize;
    return (int32_t)std::min<int64_t>(max_blocks, span);
}

size_t plan_bytes(const Plan& pl) {
    if (pl.ws_floats_m == 0) return 0;
    return 2 * round16(pl.ws_floats_m * sizeof(float)) + pl.ws_floats_acc * sizeof(float);
}

int check_decode_args(int32_t batch, int32_t n_q, const pa_cache_desc* cache,
                      int32_t max_blocks_per_seq, bool allow_quant = false) {
    int rc = check_cache(cache, allow_quant);
    if (rc) return rc;
    if (batch < 0) return fail(PA_ERR_INVALID_ARG, "batch %d < 0", batch);
    if (n_q <= 0) return fail(PA_ERR_INVALID_ARG, "n_q %d must be positive", n_q);
    if (n_q % cache->n_kv != 0)
        return fail(PA_ERR_INVALID_ARG, "n_q (%d) is not a multiple of n_kv (%d)", n_q, cache->n_kv);
    if (max_blocks_per_seq <= 0)
        return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d must be positive", max_blocks_per_seq);
    if ((int64_t)max_blocks_per_seq * kBlockSize > INT32_MAX / 2)
        return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d too large", max_blocks_per_seq);
    return PA_OK;
}

// Quantised-cache decode of q_rows rows: (query head, row) pairs per KV head in an
// int, and their slices of at most 16 columns within grid y.
bool quant_rows_fit(int32_t batch, int32_t q_rows, int32_t n_q, const pa_cache_desc* c) {
    const int64_t pairs = (int64_t)(n_q / c->n_kv) * q_rows;
    if (pairs > INT32_MAX / 2 || (int64_t)n_q * q_rows > INT32_MAX / 2 || batch > 65535) return false;
    const int64_t gw = pairs % 16 == 0 ? 16 : pairs % 8 == 0 ? 8 : pairs % 4 == 0 ? 4 : pairs % 2 == 0 ? 2 : 1;
    return (pairs / gw) * c->n_kv <= 65535;
}

// Multi-row decode plan: 4 waves per workgroup, each a contiguous run of blocks of
// the partition (2048 tokens unless overridden), groups of 32 (row, head) pairs.
constexpr int kMultiWaves = 4;
constexpr int kMultiRows = 32;

struct MultiPlan {
    int32_t blocks_per_wave, nparts_max, row_groups;
    size_t m_floats, bytes;
    // Matrix-core decode kernel instead (G * q_rows a multiple of 4, at most 16):
    // slices of gw (head, row) pairs as MFMA columns, hsg slices per KV head.
    int32_t mfma, gw, hsg, waves_tok;
};

// (head, row) pairs of one KV head that the matrix-core decode kernel takes as
// MFMA columns: a multiple of 4 up to 16, which one workgroup covers whole (so
// every K/V tile has one reader); larger groups go to the multi-row kernel,
// whose 32-pair tiles read each tile once for up to 32 pairs.
bool multi_uses_mfma(int32_t G, int32_t q_rows, const pa_cache_desc* c) {
    const int64_t pairs = (int64_t)G * q_rows;
    return (c->dtype == PA_BF16 || c->dtype == PA_F16) && pairs % 4 == 0 && pairs <= 16 &&
           option(PA_OPT_DECODE_MATRIX_CORES) != 0;
}

MultiPlan multi_plan(int32_t batch, int32_t q_rows, int32_t n_q, int32_t max_blocks, const pa_cache_desc* c) {
    MultiPlan pl{};
    const int32_t G = n_q / c->n_kv;
    if (multi_uses_mfma(G, q_rows, c)) {
        const int32_t pairs = G * q_rows;
        pl.mfma = 1;
        pl.gw = pairs % 16 == 0 ? 16 : pairs % 8 == 0 ? 8 : 4;
        pl.hsg = pairs / pl.gw;
        int32_t w = option(PA_OPT_DECODE_WAVES);
        if (w == 0) w = kMaxWaves;
        const int32_t tile = kBlockSize * c->head_dim * elem_bytes(c->dtype);
        while (w > 1 && w * mfma_wave_bytes(1, tile, pl.gw, c->head_dim) > kLdsBytes) --w;
        pl.waves_tok = w;
        mfma_partitions((int64_t)batch * c->n_kv * pl.hsg, max_blocks, w, &pl.blocks_per_wave, &pl.nparts_max);
        if (pl.nparts_max > 1) {
            pl.m_floats = (size_t)batch * q_rows * n_q * pl.nparts_max;
            pl.bytes = 2 * round16(pl.m_floats * sizeof(float)) + pl.m_floats * c->head_dim * sizeof(float);
        }
        return pl;
    }
    const int64_t rows_per_kv = (int64_t)(n_q / c->n_kv) * q_rows;
    pl.row_groups = (int32_t)((rows_per_kv + kMultiRows - 1) / kMultiRows);
    int32_t tokens = g_partition_tokens.load();
    if (tokens <= 0) tokens = 2048;
    int32_t bpw = tokens / (kBlockSize * kMultiWaves);
    bpw = std::max(2, std::min(64, bpw & ~1));
    pl.blocks_per_wave = bpw;
    const int32_t bpp = bpw * kMultiWaves;
    pl.nparts_max = std::max(1, (max_blocks + bpp - 1) / bpp);
    if (pl.nparts_max > 1) {
        pl.m_floats = (size_t)batch * q_rows * n_q * pl.nparts_max;
        pl.bytes = 2 * round16(pl.m_floats * sizeof(float)) + pl.m_floats * c->head_dim * sizeof(float);
    }
    return pl;
}

// ---- debug mode (option PA_OPT_VALIDATE): host-side checks of device-resident metadata

bool validate_enabled() { return option(PA_OPT_VALIDATE) != 0; }

template <class T>
int fetch(std::vector<T>& dst, const T* src, size_t n, hipStream_t s, const char* what) {
    dst.resize(n);
    if (n == 0) return PA_OK;
    hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "validate: copying %s: %s", what, hipGetErrorString(e));
    return PA_OK;
}

int validate_slots(const int64_t* slots_dev, int32_t n, const pa_cache_desc* c, hipStream_t s,
                   std::vector<int64_t>& slots) {
    int rc = fetch(slots, slots_dev, (size_t)n, s, "slot_mapping");
    if (rc) return rc;
    const int64_t num_slots = (int64_t)c->num_blocks * c->block_size;
    std::unordered_set<int64_t> seen;
    for (int32_t t = 0; t < n; ++t) {
        const int64_t x = slots[t];
        if (x < 0) continue;
        if (x >= num_slots)
            return fail(PA_ERR_INVALID_ARG, "validate: slot_mapping[%d] = %lld is past the pool (%lld slots)",
                        t, (long long)x, (long long)num_slots);
        if (!seen.insert(x).second)
            return fail(PA_ERR_INVALID_ARG, "validate: slot %lld appears twice in slot_mapping", (long long)x);
    }
    return PA_OK;
}

// Entries checked per sequence: the blocks the kernels read, i.e. those holding
// positions first .. ctx - 1, where first is the earliest of `rows` query rows'
// window start (0 without a window).
int validate_decode(int32_t batch, const pa_cache_desc* c, const int32_t* bt_dev, int32_t max_blocks,
                    const int32_t* ctx_dev, const int64_t* new_slots_dev, hipStream_t s,
                    int32_t rows, int32_t window) {
    std::vector<int32_t> ctx, bt;
    int rc = fetch(ctx, ctx_dev, (size_t)batch, s, "context_lens");
    if (!rc) rc = fetch(bt, bt_dev, (size_t)batch * max_blocks, s, "block_table");
    if (rc) return rc;
    const int64_t cap = (int64_t)max_blocks * c->block_size;
    std::unordered_map<int32_t, int32_t> readers;   // physical block -> sequences attending it
    for (int32_t b = 0; b < batch; ++b) {
        if (ctx[b] < 0 || ctx[b] > cap)
            return fail(PA_ERR_INVALID_ARG, "validate: context_lens[%d] = %d is outside [0, %lld]", b,
                        ctx[b], (long long)cap);
        const int32_t nblk = (ctx[b] + c->block_size - 1) / c->block_size;
        const int32_t first = window > 0 ? std::max(0, ctx[b] - rows + 1 - window) : 0;
        for (int32_t j = first / c->block_size; j < nblk; ++j) {
            const int32_t phys = bt[(size_t)b * max_blocks + j];
            if (phys < 0 || phys >= c->num_blocks)
                return fail(PA_ERR_INVALID_ARG, "validate: block_table[%d][%d] = %d is outside the pool (%d blocks)",
                            b, j, phys, c->num_blocks);
            ++readers[phys];
        }
    }
    if (!new_slots_dev) return PA_OK;
    std::vector<int64_t> slots;
    rc = validate_slots(new_slots_dev, batch, c, s, slots);
    if (rc) return rc;
    for (int32_t b = 0; b < batch; ++b) {
        if (slots[b] < 0) continue;
        if (ctx[b] < 1)
            return fail(PA_ERR_INVALID_ARG, "validate: sequence %d appends a token but its context is empty", b);
        const int32_t pos = ctx[b] - 1;
        const int64_t want = (int64_t)bt[(size_t)b * max_blocks + pos / c->block_size] * c->block_size +
                             pos % c->block_size;
        if (slots[b] != want)
            return fail(PA_ERR_INVALID_ARG,
                        "validate: slot_mapping[%d] = %lld, but position %d of sequence %d is slot %lld",
                        b, (long long)slots[b], pos, b, (long long)want);
        const int32_t phys = (int32_t)(slots[b] / c->block_size);
        if (readers[phys] > 1)
            return fail(PA_ERR_INVALID_ARG,
                        "validate: sequence %d appends into block %d, which another sequence also reads", b, phys);
    }
    return PA_OK;
}

// ---- workspace (decode partials, prefill staging) ---------------------------------

std::mutex g_ws_mu;
void* g_default_ws = nullptr;       // set by pa_set_workspace (caller-owned)
size_t g_default_ws_bytes = 0;
std::unordered_map<int, std::pair<void*, size_t>> g_lib_ws;   // device -> library-owned buffer
std::vector<void*> g_retired_ws;    // superseded library buffers, kept until the process ends

// A workspace of at least `need` bytes when the call passed none: the one set by
// pa_set_workspace if it is large enough, else the library's own for the current
// device, allocated or grown here. A buffer that a larger one replaces is never
// freed: a call on another thread may hold its address and not have enqueued its
// kernels yet, and kernels enqueued earlier may still be running on it. Growth at
// least doubles, so at most log2 of the largest size such buffers exist per device.
// `lock` comes back holding the workspace mutex; the caller keeps it until it has
// enqueued every kernel that uses the buffer, so that calls from several threads
// on one stream cannot interleave their kernels on the shared buffer (a decode
// call's partition kernel and merge kernel, for instance).
int resolve_workspace(size_t need, void** ws, std::unique_lock<std::mutex>* lock) {
    std::unique_lock<std::mutex> l(g_ws_mu);
    if (g_default_ws && g_default_ws_bytes >= need) {
        *ws = g_default_ws;
        *lock = std::move(l);
        return PA_OK;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "workspace: hipGetDevice");
    auto& slot = g_lib_ws[dev];
    if (slot.second < need) {
        const size_t bytes = std::max(need, 2 * slot.second);
        void* p = nullptr;
        e = hipMalloc(&p, bytes);
        if (e != hipSuccess) return hip_fail(e, "workspace: hipMalloc");
        if (slot.first) g_retired_ws.push_back(slot.first);
        slot = {p, bytes};
    }
    *ws = slot.first;
    *lock = std::move(l);
    return PA_OK;
}

}  // namespace

extern "C" {

int32_t pa_version(void) { return 301; }

const char* pa_last_error(void) { return g_err; }

int32_t pa_set_decode_partition_tokens(int32_t tokens) {
    if (tokens < 0 || (tokens % kBlockSize) != 0) return -1;
    return g_partition_tokens.exchange(tokens);
}

int32_t pa_set_option(int32_t o, int32_t value) {
    if (o < 0 || o >= PA_OPT_COUNT || value < kOptions[o].lo || value > kOptions[o].hi) return -1;
    return option_values()[o].exchange(value);
}

int32_t pa_get_option(int32_t o) {
    if (o < 0 || o >= PA_OPT_COUNT) return -1;
    return option(static_cast<pa_option>(o));
}

int pa_set_workspace(void* workspace, size_t bytes) {
    if (!workspace && bytes != 0) return fail(PA_ERR_INVALID_ARG, "pa_set_workspace: NULL with a nonzero size");
    if (workspace && !aligned16(workspace))
        return fail(PA_ERR_INVALID_ARG, "pa_set_workspace: workspace must be 16-byte aligned");
    std::lock_guard<std::mutex> lock(g_ws_mu);
    g_default_ws = workspace;
    g_default_ws_bytes = workspace ? bytes : 0;
    return PA_OK;
}

int pa_kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                 void* k_cache, void* v_cache, const pa_cache_desc* cache, void* stream) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache)
        return fail(PA_ERR_INVALID_ARG, "kv_append: a pointer argument is NULL");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_INVALID_ARG, "kv_append: k, v and the caches must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0)
        return fail(PA_ERR_INVALID_ARG, "kv_append: slot_mapping must be 8-byte aligned");
    if (validate_enabled()) {
        std::vector<int64_t> slots;
        rc = validate_slots(slot_mapping, num_tokens, cache, static_cast<hipStream_t>(stream), slots);
        if (rc) return rc;
    }
    const int32_t row = cache->head_dim * elem_bytes(cache->dtype);
    const hipError_t e = pa::launch_kv_append(k, v, slot_mapping, num_tokens, cache->n_kv, row,
                                              cache->block_size,
                                              (int64_t)cache->num_blocks * cache->block_size,
                                              k_cache, v_cache, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    return PA_OK;
}

}  // extern "C"

namespace {

// Partitions a matrix-core plan can take for any span up to max_blocks (a
// windowed call plans for a shorter span). With fixed runs of blocks per wave
// (an explicit partition size) the partition count grows with the span, so
// max_blocks bounds it. Otherwise each wave gets at least span * units /
// target_waves() blocks and at least 4, so below the 64-block cap a span takes at
// most min(ceil(target_waves() / (waves * units)), ceil(max_blocks / (4 * waves)))
// partitions, and at the cap the count again grows with the span.
int32_t mfma_parts_bound(int32_t nparts_at_max, int64_t units, int32_t waves, int32_t max_blocks) {
    if (g_partition_tokens.load() > 0) return nparts_at_max;
    const int64_t w = waves;
    const int64_t by_waves = (target_waves() + w * units - 1) / (w * units);
    const int64_t by_min_run = (max_blocks + 4 * w - 1) / (4 * w);
    return (int32_t)std::max<int64_t>(nparts_at_max, std::min(by_waves, by_min_run));
}

size_t partials_bytes(int64_t rows, int32_t nparts, int32_t head_dim) {
    if (nparts <= 1) return 0;
    const size_t m_floats = (size_t)rows * nparts;
    return 2 * round16(m_floats * sizeof(float)) + m_floats * head_dim * sizeof(float);
}

}  // namespace

extern "C" {

size_t pa_decode_workspace_bytes(int32_t batch, int32_t n_q, int32_t max_blocks_per_seq,
                                 const pa_cache_desc* cache) {
    if (check_decode_args(batch, n_q, cache, max_blocks_per_seq, true) != PA_OK) return 0;
    Plan pl;
    make_plan(batch, n_q, max_blocks_per_seq, cache, &pl);
    int32_t np = pl.nparts_max;
    if (pl.mfma)
        np = mfma_parts_bound(np, (int64_t)batch * cache->n_kv * pl.hsg, pl.waves_tok, max_blocks_per_seq);
    return partials_bytes((int64_t)batch * n_q, np, cache->head_dim);
}

}  // extern "C"

namespace {

// ---- the no-allocation decode's scratch ---------------------------------------------
// Split-context partials of pa_paged_attn_decode_noalloc live in this file-scope
// device array instead of an allocated workspace. Each GPU the library runs on
// holds its own copy from the moment the code object is loaded there until the
// process ends. In host code `scratch` names a host-side stand-in, never the
// device memory: the device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;                       // guards the map; held while a call enqueues
std::unordered_map<int, void*> g_scratch_ptr;  // device -> its copy of `scratch`

// Device address of the current device's `scratch`; caller holds g_scratch_mu.
int scratch_address(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "decode_noalloc: hipGetDevice");
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *ptr = it->second;
        return PA_OK;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "decode_noalloc: hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(PA_ERR_HIP, "decode_noalloc: no device address for the scratch array");
    g_scratch_ptr.emplace(dev, p);
    *ptr = p;
    return PA_OK;
}

struct FusedAppend {
    const void* k_new;
    const void* v_new;
    const int64_t* slots;
    void* k_cache_w;
    void* v_cache_w;
};

int decode_impl(const void* q, int32_t batch, int32_t n_q, const void* k_cache, const void* v_cache,
                const pa_cache_desc* cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                const int32_t* context_lens, float scale, int32_t window,
                const float* alibi_slopes, void* out,
                pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream,
                const FusedAppend* fa, bool noalloc = false) {
    int rc = check_decode_args(batch, n_q, cache, max_blocks_per_seq);
    if (rc) return rc;
    if (out_dtype != PA_F32 && out_dtype != cache->dtype)
        return fail(PA_ERR_UNSUPPORTED, "out_dtype must be PA_F32 or the cache dtype");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
    if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u)
        return fail(PA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (batch == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out)
        return fail(PA_ERR_INVALID_ARG, "decode: a pointer argument is NULL");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PA_ERR_INVALID_ARG, "decode: q, caches and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return fail(PA_ERR_INVALID_ARG, "decode: block_table and context_lens must be 4-byte aligned");
    if (fa) {
        if (!fa->k_new || !fa->v_new || !fa->slots)
            return fail(PA_ERR_INVALID_ARG, "decode_append: k_new, v_new and slot_mapping must not be NULL");
        if (!aligned16(fa->k_new) || !aligned16(fa->v_new))
            return fail(PA_ERR_INVALID_ARG, "decode_append: k_new and v_new must be 16-byte aligned");
        if (reinterpret_cast<uintptr_t>(fa->slots) & 7u)
            return fail(PA_ERR_INVALID_ARG, "decode_append: slot_mapping must be 8-byte aligned");
    }

    Plan pl;
    make_plan(batch, n_q, span_blocks(max_blocks_per_seq, 1, window), cache, &pl);
    const size_t need = plan_bytes(pl);
    std::unique_lock<std::mutex> ws_lock;   // held until the kernels are enqueued
    if (need > 0 && noalloc) {
        // Partials go to this device's scratch array; nothing is allocated.
        if (need > kNoAllocScratchBytes)
            return fail(PA_ERR_INVALID_ARG,
                        "decode_noalloc: %zu bytes of split-context partials needed, more than the "
                        "%zu-byte scratch (pa_decode_workspace_bytes gives the need)",
                        need, kNoAllocScratchBytes);
        ws_lock = std::unique_lock<std::mutex>(g_scratch_mu);
        rc = scratch_address(&workspace);
        if (rc) return rc;
    } else if (need > 0) {
        if (!workspace) {
            rc = resolve_workspace(need, &workspace, &ws_lock);
            if (rc) return rc;
        } else if (workspace_bytes < need) {
            return fail(PA_ERR_INVALID_ARG, "decode: workspace of %zu bytes required (got %zu)", need,
                        workspace_bytes);
        }
        if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "decode: workspace must be 16-byte aligned");
    }
    if (validate_enabled()) {
        rc = validate_decode(batch, cache, block_table, max_blocks_per_seq, context_lens,
                             fa ? fa->slots : nullptr, static_cast<hipStream_t>(stream), 1, window);
        if (rc) return rc;
    }

    pa::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.out = out;
    if (need > 0) {
        char* w = static_cast<char*>(workspace);
        a.ws_m = reinterpret_cast<float*>(w);
        a.ws_l = reinterpret_cast<float*>(w + round16(pl.ws_floats_m * sizeof(float)));
        a.ws_acc = reinterpret_cast<float*>(w + 2 * round16(pl.ws_floats_m * sizeof(float)));
    }
    a.batch = batch;
    a.n_q = n_q;
    a.n_kv = cache->n_kv;
    a.num_blocks = cache->num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.group = n_q / cache->n_kv;
    a.gw = pl.gw;
    a.hs_wg = pl.hs_wg;
    a.hsg = pl.hsg;
    a.waves_tok = pl.waves_tok;
    a.blocks_per_wave = pl.blocks_per_wave;
    a.nparts_max = pl.nparts_max;
    a.ring = pl.ring;
    a.mfma = pl.mfma;
    fold_scale(scale, cache->dtype, &a);
    a.out_f32 = out_dtype == PA_F32;
    a.q_rows = 1;
    a.window = window;
    a.alibi = alibi_slopes;
    if (fa) {
        a.k_new = fa->k_new;
        a.v_new = fa->v_new;
        a.new_slots = fa->slots;
        a.k_cache_w = fa->k_cache_w;
        a.v_cache_w = fa->v_cache_w;
    }
    const hipError_t e = pa::launch_decode(a, to_elem(cache->dtype), cache->head_dim,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return PA_OK;
}

}  // namespace

namespace {

// Arguments of the fp32 kernel over the paged cache: `rows` query rows per
// sequence at the end of its context (chunked prefill, multi-row decode).
pa::PrefillArgs paged_f32_args(const void* q, int32_t batch, int32_t rows, int32_t n_q, const void* k_cache,
                               const void* v_cache, const pa_cache_desc* cache, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* context_lens, float scale, int32_t window,
                               const float* alibi_slopes, void* out) {
    pa::PrefillArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.batch = batch;
    a.seq_len = rows;
    a.n_q = n_q;
    a.n_kv = cache->n_kv;
    a.group = n_q / cache->n_kv;
    a.causal = 1;
    fold_scale(scale, PA_F32, &a);
    a.out_f32 = 1;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.max_blocks = max_blocks;
    a.num_blocks = cache->num_blocks;
    a.window = window;
    a.alibi = alibi_slopes;
    return a;
}

int launch_f32(const pa::PrefillArgs& a, int32_t head_dim, void* stream, const char* what) {
    const hipError_t e = pa::launch_attn_f32(a, head_dim, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported)
        return fail(PA_ERR_UNSUPPORTED, "%s: f32 rows * group, n_kv or batch past the kernel's grid", what);
    if (e != hipSuccess) return hip_fail(e, "f32 attention launch");
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_paged_attn_decode(const void* q, int32_t batch, int32_t n_q, const void* k_cache,
                         const void* v_cache, const pa_cache_desc* cache,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, float scale, int32_t window,
                         const float* alibi_slopes, void* out,
                         pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(q, batch, n_q, k_cache, v_cache, cache, block_table, max_blocks_per_seq,
                       context_lens, scale, window, alibi_slopes, out, out_dtype, workspace, workspace_bytes,
                       stream, nullptr);
}

int pa_paged_attn_decode_noalloc(const void* q, int32_t batch, int32_t n_q, const void* k_cache,
                                 const void* v_cache, const pa_cache_desc* cache,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, float scale, int32_t window,
                                 const float* alibi_slopes, void* out, pa_dtype out_dtype, void* stream) {
    return decode_impl(q, batch, n_q, k_cache, v_cache, cache, block_table, max_blocks_per_seq,
                       context_lens, scale, window, alibi_slopes, out, out_dtype, nullptr, 0, stream,
                       nullptr, true);
}

int pa_paged_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, int32_t batch, int32_t n_q,
                                void* k_cache, void* v_cache, const pa_cache_desc* cache,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, float scale, int32_t window,
                                const float* alibi_slopes,
                                void* out, pa_dtype out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
    const FusedAppend fa{k_new, v_new, slot_mapping, k_cache, v_cache};
    return decode_impl(q, batch, n_q, k_cache, v_cache, cache, block_table, max_blocks_per_seq,
                       context_lens, scale, window, alibi_slopes, out, out_dtype, workspace, workspace_bytes,
                       stream, &fa);
}

size_t pa_prefill_workspace_bytes(pa_dtype dtype, int32_t batch, int32_t seq_len, int32_t n_kv,
                                  int32_t head_dim) {
    if (!prefill_stages(dtype) || batch <= 0 || seq_len <= 0 || n_kv <= 0 || head_dim <= 0) return 0;
    return prefill_stage_bytes(batch, seq_len, n_kv, head_dim);
}

int pa_paged_attn_prefill(const void* q, const void* k, const void* v, pa_dtype dtype,
                          int32_t batch, int32_t seq_len, int32_t n_q, int32_t n_kv,
                          int32_t head_dim, int32_t causal, float scale, int32_t window,
                          const float* alibi_slopes,
                          void* out, pa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (dtype != PA_BF16 && dtype != PA_F16 && dtype != PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "prefill supports f32, bf16 and f16 inputs");
    if (out_dtype != PA_F32 && out_dtype != dtype)
        return fail(PA_ERR_UNSUPPORTED, "out_dtype must be PA_F32 or the input dtype");
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "prefill head_dim %d has no kernel (supported: 64, 128)", head_dim);
    if (batch < 0 || seq_len < 0) return fail(PA_ERR_INVALID_ARG, "batch and seq_len must be >= 0");
    if (n_q <= 0 || n_kv <= 0) return fail(PA_ERR_INVALID_ARG, "n_q and n_kv must be positive");
    if (n_q % n_kv != 0)
        return fail(PA_ERR_INVALID_ARG, "n_q (%d) is not a multiple of n_kv (%d)", n_q, n_kv);
    if (causal != 0 && causal != 1) return fail(PA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
    if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u)
        return fail(PA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (window > 0 && !causal) return fail(PA_ERR_INVALID_ARG, "a sliding window needs causal == 1");
    if (alibi_slopes && !causal) return fail(PA_ERR_INVALID_ARG, "ALiBi slopes need causal == 1");
    if (batch == 0 || seq_len == 0) return PA_OK;
    if (dtype != PA_F32 && !pa::prefill_grid_fits(seq_len, n_q, batch, n_q / n_kv))
        return fail(PA_ERR_UNSUPPORTED, "prefill: the number of workgroups (ceil(seq_len / rows per workgroup) * n_q / heads per workgroup * batch) exceeds one launch");
    if (!q || !k || !v || !out) return fail(PA_ERR_INVALID_ARG, "prefill: a pointer argument is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(PA_ERR_INVALID_ARG, "prefill: q, k, v and out must be 16-byte aligned");

    pa::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.batch = batch;
    a.seq_len = seq_len;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.group = n_q / n_kv;
    a.causal = causal;
    fold_scale(scale, dtype, &a);
    a.out_f32 = out_dtype == PA_F32;
    a.window = window;
    a.alibi = alibi_slopes;
    if (dtype == PA_F32) return launch_f32(a, head_dim, stream, "prefill");
    std::unique_lock<std::mutex> ws_lock;   // held until the kernels are enqueued
    if (prefill_stages(dtype) && stage_grid_fits(batch, n_kv)) {
        const size_t need = prefill_stage_bytes(batch, seq_len, n_kv, head_dim);
        if (!workspace) {
            const int rc = resolve_workspace(need, &workspace, &ws_lock);
            if (rc != PA_OK) return rc;
        } else if (workspace_bytes < need) {
            return fail(PA_ERR_INVALID_ARG, "prefill: workspace of %zu bytes required (got %zu)", need,
                        workspace_bytes);
        }
        if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "prefill: workspace must be 16-byte aligned");
        a.v16 = workspace;
        a.v16_ok = static_cast<uint8_t*>(workspace) + prefill_stage_v_bytes(batch, seq_len, n_kv, head_dim);
    }
    const hipError_t e = pa::launch_prefill(a, to_elem(dtype), head_dim, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported)
        return fail(PA_ERR_UNSUPPORTED, "prefill: no kernel for these arguments");
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return PA_OK;
}

size_t pa_decode_multi_workspace_bytes(int32_t batch, int32_t q_rows, int32_t n_q,
                                       int32_t max_blocks_per_seq, const pa_cache_desc* cache) {
    if (check_decode_args(batch, n_q, cache, max_blocks_per_seq, true) != PA_OK || q_rows < 1) return 0;
    if (cache->dtype == PA_F32) return 0;   // the fp32 kernel keeps no partials
    if (is_quant(cache->dtype)) {           // the quantised-cache decode kernel, q_rows rows
        if (!quant_rows_fit(batch, q_rows, n_q, cache)) return 0;
        Plan pl;
        make_plan(batch, n_q * q_rows, max_blocks_per_seq, cache, &pl);
        const int32_t np = mfma_parts_bound(pl.nparts_max, (int64_t)batch * cache->n_kv * pl.hsg, pl.waves_tok,
                                            max_blocks_per_seq);
        return partials_bytes((int64_t)batch * q_rows * n_q, np, cache->head_dim);
    }
    const MultiPlan pl = multi_plan(batch, q_rows, n_q, max_blocks_per_seq, cache);
    if (!pl.mfma) return pl.bytes;
    const int32_t np = mfma_parts_bound(pl.nparts_max, (int64_t)batch * cache->n_kv * pl.hsg, pl.waves_tok,
                                        max_blocks_per_seq);
    return partials_bytes((int64_t)batch * q_rows * n_q, np, cache->head_dim);
}

int pa_paged_attn_decode_multi(const void* q, int32_t batch, int32_t q_rows, int32_t n_q,
                               const void* k_cache, const void* v_cache, const pa_cache_desc* cache,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, float scale, int32_t window,
                               const float* alibi_slopes, void* out,
                               pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_decode_args(batch, n_q, cache, max_blocks_per_seq);
    if (rc) return rc;
    if (is_quant(cache->dtype))
        return fail(PA_ERR_UNSUPPORTED, "multi-row decode supports f32, bf16 and f16 caches");
    if (out_dtype != PA_F32 && out_dtype != cache->dtype)
        return fail(PA_ERR_UNSUPPORTED, "out_dtype must be PA_F32 or the cache dtype");
    if (q_rows < 1) return fail(PA_ERR_INVALID_ARG, "q_rows %d must be positive", q_rows);
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
    if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u)
        return fail(PA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (batch == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out)
        return fail(PA_ERR_INVALID_ARG, "multi-row decode: a pointer argument is NULL");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PA_ERR_INVALID_ARG, "multi-row decode: q, caches and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return fail(PA_ERR_INVALID_ARG, "multi-row decode: block_table and context_lens must be 4-byte aligned");
    if (cache->dtype == PA_F32) {   // the fp32 kernel of chunked prefill, q_rows rows per sequence
        if (validate_enabled()) {
            rc = validate_decode(batch, cache, block_table, max_blocks_per_seq, context_lens, nullptr,
                                 static_cast<hipStream_t>(stream), q_rows, window);
            if (rc) return rc;
        }
        pa::PrefillArgs a = paged_f32_args(q, batch, q_rows, n_q, k_cache, v_cache, cache, block_table,
                                           max_blocks_per_seq, context_lens, scale, window, alibi_slopes, out);
        return launch_f32(a, cache->head_dim, stream, "multi-row decode");
    }
    const MultiPlan pl = multi_plan(batch, q_rows, n_q, span_blocks(max_blocks_per_seq, q_rows, window), cache);
    std::unique_lock<std::mutex> ws_lock;   // held until the kernels are enqueued
    if (pl.bytes > 0) {
        if (!workspace) {
            rc = resolve_workspace(pl.bytes, &workspace, &ws_lock);
            if (rc) return rc;
        } else if (workspace_bytes < pl.bytes) {
            return fail(PA_ERR_INVALID_ARG, "multi-row decode: workspace of %zu bytes required (got %zu)",
                        pl.bytes, workspace_bytes);
        }
        if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "multi-row decode: workspace must be 16-byte aligned");
    }
    if (validate_enabled()) {
        rc = validate_decode(batch, cache, block_table, max_blocks_per_seq, context_lens, nullptr,
                             static_cast<hipStream_t>(stream), q_rows, window);
        if (rc) return rc;
    }

    pa::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.out = out;
    if (pl.bytes > 0) {
        char* w = static_cast<char*>(workspace);
        a.ws_m = reinterpret_cast<float*>(w);
        a.ws_l = reinterpret_cast<float*>(w + round16(pl.m_floats * sizeof(float)));
        a.ws_acc = reinterpret_cast<float*>(w + 2 * round16(pl.m_floats * sizeof(float)));
    }
    a.batch = batch;
    a.n_q = n_q;
    a.n_kv = cache->n_kv;
    a.num_blocks = cache->num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.group = n_q / cache->n_kv;
    a.blocks_per_wave = pl.blocks_per_wave;
    a.nparts_max = pl.nparts_max;
    fold_scale(scale, cache->dtype, &a);
    a.out_f32 = out_dtype == PA_F32;
    a.q_rows = q_rows;
    a.window = window;
    a.alibi = alibi_slopes;
    hipError_t e;
    if (pl.mfma) {
        a.gw = pl.gw;
        a.hs_wg = 1;
        a.hsg = pl.hsg;
        a.waves_tok = pl.waves_tok;
        a.ring = 1;
        a.mfma = 1;
        e = pa::launch_decode_mfma(a, to_elem(cache->dtype), cache->head_dim, static_cast<hipStream_t>(stream));
    } else {
        a.waves_tok = kMultiWaves;
        a.row_groups = pl.row_groups;
        e = pa::launch_decode_multi(a, to_elem(cache->dtype), cache->head_dim, static_cast<hipStream_t>(stream));
    }
    if (e == hipErrorNotSupported)
        return fail(PA_ERR_UNSUPPORTED, "multi-row decode: no kernel for these arguments");
    if (e != hipSuccess) return hip_fail(e, "multi-row decode launch");
    return PA_OK;
}

size_t pa_chunked_prefill_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq,
                                          const pa_cache_desc* cache) {
    if (check_cache(cache) != PA_OK || batch <= 0 || max_blocks_per_seq <= 0) return 0;
    if (!prefill_stages(cache->dtype) || !stage_grid_fits(batch, cache->n_kv)) return 0;
    const size_t need = chunked_stage_bytes(batch, max_blocks_per_seq, cache->n_kv, cache->head_dim);
    return need <= kChunkStageCap ? need : 0;
}

int pa_paged_attn_chunked_prefill(const void* q, int32_t batch, int32_t chunk_len, int32_t n_q,
                                  const void* k_cache, const void* v_cache, const pa_cache_desc* cache,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, float scale, int32_t window,
                                  const float* alibi_slopes,
                                  void* out, pa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    int rc = check_decode_args(batch, n_q, cache, max_blocks_per_seq);
    if (rc) return rc;
    if (is_quant(cache->dtype))
        return fail(PA_ERR_UNSUPPORTED, "chunked prefill supports f32, bf16 and f16 caches");
    if (out_dtype != PA_F32 && out_dtype != cache->dtype)
        return fail(PA_ERR_UNSUPPORTED, "out_dtype must be PA_F32 or the cache dtype");
    if (chunk_len < 0) return fail(PA_ERR_INVALID_ARG, "chunk_len %d < 0", chunk_len);
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
    if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u)
        return fail(PA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (batch == 0 || chunk_len == 0) return PA_OK;
    if (cache->dtype != PA_F32 && !pa::prefill_grid_fits(chunk_len, n_q, batch, n_q / cache->n_kv))
        return fail(PA_ERR_UNSUPPORTED, "chunked prefill: the number of workgroups exceeds one launch");
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out)
        return fail(PA_ERR_INVALID_ARG, "chunked prefill: a pointer argument is NULL");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PA_ERR_INVALID_ARG, "chunked prefill: q, caches and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return fail(PA_ERR_INVALID_ARG, "chunked prefill: block_table and context_lens must be 4-byte aligned");
    if (validate_enabled()) {
        rc = validate_decode(batch, cache, block_table, max_blocks_per_seq, context_lens, nullptr,
                             static_cast<hipStream_t>(stream), chunk_len, window);
        if (rc) return rc;
    }
    if (cache->dtype == PA_F32) {
        pa::PrefillArgs a = paged_f32_args(q, batch, chunk_len, n_q, k_cache, v_cache, cache, block_table,
                                           max_blocks_per_seq, context_lens, scale, window, alibi_slopes, out);
        return launch_f32(a, cache->head_dim, stream, "chunked prefill");
    }

    pa::PrefillArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.batch = batch;
    a.seq_len = chunk_len;
    a.n_q = n_q;
    a.n_kv = cache->n_kv;
    a.group = n_q / cache->n_kv;
    a.causal = 1;
    fold_scale(scale, cache->dtype, &a);
    a.out_f32 = out_dtype == PA_F32;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = cache->num_blocks;
    a.window = window;
    a.alibi = alibi_slopes;
    const size_t need = pa_chunked_prefill_workspace_bytes(batch, max_blocks_per_seq, cache);
    std::unique_lock<std::mutex> ws_lock;   // held until the kernels are enqueued
    if (need > 0) {
        if (!workspace) {
            rc = resolve_workspace(need, &workspace, &ws_lock);
            if (rc != PA_OK) return rc;
        } else if (workspace_bytes < need) {
            return fail(PA_ERR_INVALID_ARG, "chunked prefill: workspace of %zu bytes required (got %zu)", need,
                        workspace_bytes);
        }
        if (!aligned16(workspace))
            return fail(PA_ERR_INVALID_ARG, "chunked prefill: workspace must be 16-byte aligned");
        a.v16 = workspace;
        a.v16_ok = static_cast<uint8_t*>(workspace) +
                   chunked_stage_v_bytes(batch, max_blocks_per_seq, cache->n_kv, cache->head_dim);
    }
    const hipError_t e = pa::launch_prefill(a, to_elem(cache->dtype), cache->head_dim,
                                            static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported)
        return fail(PA_ERR_UNSUPPORTED, "chunked prefill: no kernel for these arguments");
    if (e != hipSuccess) return hip_fail(e, "chunked prefill launch");
    return PA_OK;
}


int pa_kv_append_quant(const void* k, const void* v, pa_dtype src_dtype, const int64_t* slot_mapping,
                       int32_t num_tokens, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                       const pa_cache_desc* cache, void* stream) {
    int rc = check_cache(cache, true);
    if (rc) return rc;
    if (!is_quant(cache->dtype))
        return fail(PA_ERR_INVALID_ARG,
                    "kv_append_quant: cache dtype must be PA_FP8_E4M3 or PA_INT8 (or their _PER_CHANNEL forms)");
    if (src_dtype != PA_F32 && src_dtype != PA_BF16 && src_dtype != PA_F16)
        return fail(PA_ERR_UNSUPPORTED, "kv_append_quant: k and v must be f32, bf16 or f16");
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
        return fail(PA_ERR_INVALID_ARG, "kv_append_quant: a pointer argument is NULL");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(k_scale) || !aligned16(v_scale))
        return fail(PA_ERR_INVALID_ARG, "kv_append_quant: k, v, the caches and the scales must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0)
        return fail(PA_ERR_INVALID_ARG, "kv_append_quant: slot_mapping must be 8-byte aligned");
    if (validate_enabled()) {
        std::vector<int64_t> slots;
        rc = validate_slots(slot_mapping, num_tokens, cache, static_cast<hipStream_t>(stream), slots);
        if (rc) return rc;
    }
    const hipError_t e = pa::launch_kv_append_quant(
        k, v, to_elem(src_dtype), fmt_of(cache->dtype), is_per_channel(cache->dtype), slot_mapping,
        num_tokens, cache->n_kv, cache->head_dim, (int64_t)cache->num_blocks * cache->block_size, k_cache,
        v_cache, k_scale, v_scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_append_quant launch");
    return PA_OK;
}

}  // extern "C"

namespace {

// The new rows of a fused quantising append, with the pools and scales it writes.
struct FusedQuantAppend {
    const void* k_new;
    const void* v_new;
    const int64_t* slots;
    void* k_cache_w;
    void* v_cache_w;
    float* k_scale_w;
    float* v_scale_w;
};

// Decode of q_rows query rows per sequence (1: single-row decode, which may carry
// a fused append) over a quantised cache; `what` names the entry point in errors.
int decode_quant_impl(const void* q, pa_dtype q_dtype, int32_t batch, int32_t q_rows, int32_t n_q,
                      const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, const pa_cache_desc* cache,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, float scale, int32_t window,
                      const float* alibi_slopes, void* out,
                      pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream,
                      const FusedQuantAppend* fa) {
    int rc = check_decode_args(batch, n_q, cache, max_blocks_per_seq, true);
    if (rc) return rc;
    if (q_rows < 1) return fail(PA_ERR_INVALID_ARG, "q_rows %d must be positive", q_rows);
    if (!quant_rows_fit(batch, q_rows, n_q, cache))
        return fail(PA_ERR_UNSUPPORTED, "decode_quant: (query head, row) pairs per KV head past the grid");
    if (!is_quant(cache->dtype))
        return fail(PA_ERR_INVALID_ARG,
                    "decode_quant: cache dtype must be PA_FP8_E4M3 or PA_INT8 (or their _PER_CHANNEL forms)");
    if (q_dtype != PA_BF16 && q_dtype != PA_F16)
        return fail(PA_ERR_UNSUPPORTED, "decode_quant: q must be bf16 or f16");
    if (out_dtype != PA_F32 && out_dtype != q_dtype)
        return fail(PA_ERR_UNSUPPORTED, "out_dtype must be PA_F32 or q_dtype");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    if (window < 0) return fail(PA_ERR_INVALID_ARG, "window %d < 0", window);
    if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u)
        return fail(PA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (batch == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !context_lens || !out)
        return fail(PA_ERR_INVALID_ARG, "decode_quant: a pointer argument is NULL");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_scale) ||
        !aligned16(v_scale) || !aligned16(out))
        return fail(PA_ERR_INVALID_ARG, "decode_quant: q, caches, scales and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return fail(PA_ERR_INVALID_ARG, "decode_quant: block_table and context_lens must be 4-byte aligned");
    if (fa) {
        if (!fa->k_new || !fa->v_new || !fa->slots)
            return fail(PA_ERR_INVALID_ARG, "decode_quant_append: k_new, v_new and slot_mapping must not be NULL");
        if (!aligned16(fa->k_new) || !aligned16(fa->v_new))
            return fail(PA_ERR_INVALID_ARG, "decode_quant_append: k_new and v_new must be 16-byte aligned");
        if (reinterpret_cast<uintptr_t>(fa->slots) & 7u)
            return fail(PA_ERR_INVALID_ARG, "decode_quant_append: slot_mapping must be 8-byte aligned");
    }

    // The (query head, row) pairs of a KV head are the columns, as query heads are
    // for one row: plan as for n_q * q_rows heads.
    Plan pl;
    make_plan(batch, n_q * q_rows, span_blocks(max_blocks_per_seq, q_rows, window), cache, &pl);
    const size_t need = plan_bytes(pl);
    std::unique_lock<std::mutex> ws_lock;   // held until the kernels are enqueued
    if (need > 0) {
        if (!workspace) {
            rc = resolve_workspace(need, &workspace, &ws_lock);
            if (rc) return rc;
        } else if (workspace_bytes < need) {
            return fail(PA_ERR_INVALID_ARG, "decode_quant: workspace of %zu bytes required (got %zu)", need,
                        workspace_bytes);
        }
        if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "decode_quant: workspace must be 16-byte aligned");
    }
    if (validate_enabled()) {
        rc = validate_decode(batch, cache, block_table, max_blocks_per_seq, context_lens,
                             fa ? fa->slots : nullptr, static_cast<hipStream_t>(stream), q_rows, window);
        if (rc) return rc;
    }

    pa::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.chan_scales = is_per_channel(cache->dtype) ? 1 : 0;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.out = out;
    if (need > 0) {
        char* w = static_cast<char*>(workspace);
        a.ws_m = reinterpret_cast<float*>(w);
        a.ws_l = reinterpret_cast<float*>(w + round16(pl.ws_floats_m * sizeof(float)));
        a.ws_acc = reinterpret_cast<float*>(w + 2 * round16(pl.ws_floats_m * sizeof(float)));
    }
    a.batch = batch;
    a.n_q = n_q;
    a.n_kv = cache->n_kv;
    a.num_blocks = cache->num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.group = n_q / cache->n_kv;
    a.gw = pl.gw;
    a.hs_wg = pl.hs_wg;
    a.hsg = pl.hsg;
    a.waves_tok = pl.waves_tok;
    a.blocks_per_wave = pl.blocks_per_wave;
    a.nparts_max = pl.nparts_max;
    a.ring = pl.ring;
    a.mfma = 1;
    fold_scale(scale, q_dtype, &a);
    a.out_f32 = out_dtype == PA_F32;
    a.q_rows = q_rows;
    a.window = window;
    a.alibi = alibi_slopes;
    if (fa) {
        a.k_new = fa->k_new;
        a.v_new = fa->v_new;
        a.new_slots = fa->slots;
        a.k_cache_w = fa->k_cache_w;
        a.v_cache_w = fa->v_cache_w;
        a.k_scale_w = fa->k_scale_w;
        a.v_scale_w = fa->v_scale_w;
    }
    const hipError_t e = pa::launch_decode_quant(a, to_elem(q_dtype),
                                                 fmt_of(cache->dtype),
                                                 cache->head_dim, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode_quant launch");
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_paged_attn_decode_quant(const void* q, pa_dtype q_dtype, int32_t batch, int32_t n_q,
                               const void* k_cache, const void* v_cache, const float* k_scale,
                               const float* v_scale, const pa_cache_desc* cache,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, float scale, int32_t window,
                               const float* alibi_slopes, void* out,
                               pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_quant_impl(q, q_dtype, batch, 1, n_q, k_cache, v_cache, k_scale, v_scale, cache, block_table,
                             max_blocks_per_seq, context_lens, scale, window, alibi_slopes, out, out_dtype, workspace,
                             workspace_bytes, stream, nullptr);
}

int pa_paged_attn_decode_multi_quant(const void* q, pa_dtype q_dtype, int32_t batch, int32_t q_rows, int32_t n_q,
                                     const void* k_cache, const void* v_cache, const float* k_scale,
                                     const float* v_scale, const pa_cache_desc* cache,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, float scale, int32_t window,
                                     const float* alibi_slopes, void* out, pa_dtype out_dtype, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    return decode_quant_impl(q, q_dtype, batch, q_rows, n_q, k_cache, v_cache, k_scale, v_scale, cache,
                             block_table, max_blocks_per_seq, context_lens, scale, window, alibi_slopes, out,
                             out_dtype, workspace, workspace_bytes, stream, nullptr);
}

int pa_paged_attn_chunked_prefill_quant(const void* q, pa_dtype q_dtype, int32_t batch, int32_t chunk_len,
                                        int32_t n_q, const void* k_cache, const void* v_cache, const float* k_scale,
                                        const float* v_scale, const pa_cache_desc* cache,
                                        const int32_t* block_table, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, float scale, int32_t window,
                                        const float* alibi_slopes, void* out, pa_dtype out_dtype, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    if (chunk_len < 0) return fail(PA_ERR_INVALID_ARG, "chunk_len %d < 0", chunk_len);
    if (chunk_len == 0) {
        const int rc = check_decode_args(batch, n_q, cache, max_blocks_per_seq, true);
        return rc ? rc : PA_OK;
    }
    return decode_quant_impl(q, q_dtype, batch, chunk_len, n_q, k_cache, v_cache, k_scale, v_scale, cache,
                             block_table, max_blocks_per_seq, context_lens, scale, window, alibi_slopes, out,
                             out_dtype, workspace, workspace_bytes, stream, nullptr);
}

int pa_paged_attn_decode_quant_append(const void* q, const void* k_new, const void* v_new, pa_dtype q_dtype,
                                      const int64_t* slot_mapping, int32_t batch, int32_t n_q, void* k_cache,
                                      void* v_cache, float* k_scale, float* v_scale, const pa_cache_desc* cache,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, float scale, int32_t window,
                                      const float* alibi_slopes, void* out,
                                      pa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                      void* stream) {
    const FusedQuantAppend fa{k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale};
    return decode_quant_impl(q, q_dtype, batch, 1, n_q, k_cache, v_cache, k_scale, v_scale, cache, block_table,
                             max_blocks_per_seq, context_lens, scale, window, alibi_slopes, out, out_dtype, workspace,
                             workspace_bytes, stream, &fa);
}

}  // extern "C"
