"""GPU parity of sliding-window attention, in every kernel, against the fp64 oracle.

With window W > 0 the query at position p attends to positions p - W + 1 .. p
only. Decode, fused decode + append, multi-row decode, chunked prefill and
contiguous prefill are each compared with the oracle's windowed definition on
the same seeded inputs (max-abs 2e-3 and norm-wise relative 1e-2 for bf16/f16,
1e-5 for fp32). Block-table entries of blocks wholly before the window are
then overwritten with -1: the kernels never read them, so every output bit
must stay the same.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, oracle_pools, same_bits, say, stored_np
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["default", "valu"])
def decode_kernel(request, option):
    """Single-row decode tests run with the default kernel choice (matrix cores for
    bf16/f16 groups of 4, 8 or 16) and with the VALU kernel forced."""
    option("decode_matrix_cores", 0 if request.param == "valu" else 1)
    return request.param


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_gqa_attention_attn_amd as pa
    pa._lib.load()  # raises if the HIP library is missing: no fallback
    return pa


def _poison_before(block_table, context_lens, rows, window):
    """Copy of the table with every entry wholly before the earliest row's window set to -1."""
    bt = block_table.clone()
    for b, ctx in enumerate(context_lens.tolist()):
        first = max(0, ctx - rows + 1 - window)
        bt[b, : first // 16] = -1
    return bt


# ---- single-row decode --------------------------------------------------------------------

DECODE = {
    # name: (n_q, n_kv, head_dim, context lengths, dtype)
    "gqa4_bf16_d128": (32, 8, 128, [1, 15, 16, 17, 100, 257, 1000, 5000, 9000], "bf16"),
    "gqa4_f16_d64": (8, 2, 64, [3, 64, 130, 2100], "f16"),
    "gqa2_f32_d128": (4, 2, 128, [9, 77, 600], "f32"),
    "mqa_bf16": (16, 1, 128, [40, 700, 3000], "bf16"),
}


def _decode_case(name, seed_extra=0):
    n_q, n_kv, d, ctx, dt = DECODE[name]
    return wl.make_decode_case(batch=len(ctx), n_q=n_q, n_kv=n_kv, head_dim=d, context_lens=ctx,
                               dtype=dt, free_fraction=0.2, seed=len(name) * 13 + seed_extra,
                               device="cuda", name=name)


def _appended(pa, c):
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.new_k, c.new_v, c.slot_mapping, kp, vp)
    return kp, vp


@pytest.mark.parametrize("window", [1, 16, 100, 4096])
@pytest.mark.parametrize("name", sorted(DECODE))
def test_decode_window_matches_oracle(pa, decode_kernel, name, window):
    c = _decode_case(name)
    say(f"[window] decode {name} W={window} ctx={c.context_lens.tolist()}")
    kp, vp = _appended(pa, c)
    got = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale, window=window)
    torch.cuda.synchronize()
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), c.dtype,
                         c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                         window=window)
    stats = assert_parity(got.cpu().numpy(), want, c.dtype, f"decode {name} W={window}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
    # Entries before the window are never read.
    bt = _poison_before(c.block_table, c.context_lens, 1, window)
    again = pa.paged_attn_decode(c.q, kp, vp, bt, c.context_lens, c.scale, window=window)
    torch.cuda.synchronize()
    assert same_bits(got, again)


@pytest.mark.parametrize("tokens", [256, 1024])
def test_decode_window_partition_sizes(pa, decode_kernel, tokens):
    c = _decode_case("gqa4_bf16_d128", seed_extra=1)
    say(f"[window] decode partitions of {tokens} tokens, W=3000")
    kp, vp = _appended(pa, c)
    prev = pa.set_decode_partition_tokens(tokens)
    try:
        got = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale, window=3000)
        torch.cuda.synchronize()
    finally:
        pa.set_decode_partition_tokens(prev)
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), c.dtype,
                         c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                         window=3000)
    assert_parity(got.cpu().numpy(), want, c.dtype, f"partition {tokens}")


def test_decode_append_window_equals_two_calls_bitwise(pa, decode_kernel):
    c = _decode_case("gqa4_bf16_d128", seed_extra=2)
    say("[window] fused decode + append vs kv_append + decode, W=500")
    kp, vp = _appended(pa, c)
    two = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale, window=500)
    kf, vf = c.k_pool.clone(), c.v_pool.clone()
    one = pa.paged_attn_decode_append(c.q, c.new_k, c.new_v, c.slot_mapping, kf, vf, c.block_table,
                                      c.context_lens, c.scale, window=500)
    torch.cuda.synchronize()
    assert same_bits(one, two)
    assert same_bits(kf, kp) and same_bits(vf, vp)


def test_decode_window_covering_the_context_is_the_plain_decode(pa, decode_kernel):
    c = _decode_case("gqa4_f16_d64", seed_extra=3)
    say("[window] W >= every context gives the unwindowed bits")
    kp, vp = _appended(pa, c)
    full = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale)
    wide = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale,
                                window=int(c.context_lens.max()))
    torch.cuda.synchronize()
    assert same_bits(full, wide)


# ---- multi-row decode ---------------------------------------------------------------------

MULTI = [
    # (q_rows, prefix lengths, n_q, n_kv, head_dim, dtype, window)
    (4, [100, 2047, 9000], 32, 8, 128, "bf16", 64),
    (4, [100, 2047, 9000], 32, 8, 128, "bf16", 4096),
    (8, [300, 4000], 64, 8, 128, "bf16", 3),        # window shorter than the rows
    (2, [0, 17, 33], 8, 2, 64, "f16", 20),
    (5, [700], 4, 4, 128, "bf16", 1),               # each row sees only itself
]


@pytest.mark.parametrize("shape", MULTI, ids=[f"R{s[0]}_P{'-'.join(map(str, s[1]))}_{s[2]}x{s[3]}_d{s[4]}_{s[5]}_W{s[6]}"
                                              for s in MULTI])
def test_decode_multi_window_matches_oracle(pa, shape):
    R, pre, n_q, n_kv, d, dt, W = shape
    c = wl.make_chunk_case(batch=len(pre), chunk_len=R, prefix_lens=pre, n_q=n_q, n_kv=n_kv,
                           head_dim=d, dtype=dt, free_fraction=0.2, seed=sum(pre) + W, device="cuda")
    say(f"[window] multi-row decode R={R} prefix={pre} {n_q}x{n_kv} d={d} {dt} W={W}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    got = pa.paged_attn_decode_multi(c.q, kp, vp, c.block_table, c.context_lens, c.scale, window=W)
    bt = _poison_before(c.block_table, c.context_lens, R, W)
    again = pa.paged_attn_decode_multi(c.q, kp, vp, bt, c.context_lens, c.scale, window=W)
    torch.cuda.synchronize()
    want = oracle.chunked_prefill(stored_np(c.q), *oracle_pools(c), dt,
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                                  window=W)
    stats = assert_parity(got.cpu().numpy(), want, dt, f"multi W={W}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
    assert same_bits(got, again)


# ---- chunked and contiguous prefill -------------------------------------------------------

CHUNKED = [
    # (chunk_len, prefix lengths, n_q, n_kv, head_dim, dtype, window)
    (300, [1000, 17], 16, 4, 128, "f16", 128),
    (64, [0, 0], 8, 2, 128, "bf16", 16),
    (130, [64, 500], 8, 2, 64, "bf16", 1),
    (17, [5, 400], 8, 2, 128, "bf16", 70),
    (200, [700], 4, 4, 128, "bf16", 1000),
]


@pytest.mark.parametrize("shape", CHUNKED, ids=[f"C{s[0]}_P{'-'.join(map(str, s[1]))}_{s[2]}x{s[3]}_d{s[4]}_{s[5]}_W{s[6]}"
                                                for s in CHUNKED])
def test_chunked_prefill_window_matches_oracle(pa, shape):
    C, pre, n_q, n_kv, d, dt, W = shape
    c = wl.make_chunk_case(batch=len(pre), chunk_len=C, prefix_lens=pre, n_q=n_q, n_kv=n_kv,
                           head_dim=d, dtype=dt, free_fraction=0.2, seed=sum(pre) + 3 * W + C,
                           device="cuda")
    say(f"[window] chunked prefill C={C} prefix={pre} {n_q}x{n_kv} d={d} {dt} W={W}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    got = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, c.scale,
                                        window=W)
    bt = _poison_before(c.block_table, c.context_lens, C, W)
    again = pa.paged_attn_chunked_prefill(c.q, kp, vp, bt, c.context_lens, c.scale, window=W)
    torch.cuda.synchronize()
    want = oracle.chunked_prefill(stored_np(c.q), *oracle_pools(c), dt,
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                                  window=W)
    stats = assert_parity(got.cpu().numpy(), want, dt, f"chunked W={W}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
    assert same_bits(got, again)


@pytest.mark.parametrize("window", [1, 64, 100, 129, 4096])
def test_prefill_window_matches_oracle(pa, window):
    B, S, n_q, n_kv, d, dt = 2, 300, 8, 2, 128, "bf16"
    g = torch.Generator(device="cuda").manual_seed(window)
    t = wl.TORCH_DTYPES[dt]
    q = torch.randn(B, S, n_q, d, generator=g, device="cuda").to(t)
    k = torch.randn(B, S, n_kv, d, generator=g, device="cuda").to(t)
    v = torch.randn(B, S, n_kv, d, generator=g, device="cuda").to(t)
    say(f"[window] prefill B={B} S={S} {n_q}x{n_kv} d={d} W={window}")
    out = pa.paged_attn_prefill(q, k, v, True, d ** -0.5, window=window)
    torch.cuda.synchronize()
    want = oracle.prefill(stored_np(q), stored_np(k), stored_np(v), dt, True, d ** -0.5,
                          window=window)
    stats = assert_parity(out.cpu().numpy(), want, dt, f"prefill W={window}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


@pytest.mark.parametrize("stage", ["1", "0"], ids=["staged", "unstaged"])
def test_whole_prompt_chunk_equals_contiguous_prefill_with_window_bitwise(pa, option, stage):
    option("prefill_stage_v", int(stage))
    c = wl.make_prefill_case(batch=2, seq_len=300, n_q=8, n_kv=2, head_dim=128, dtype="bf16",
                             seed=78, device="cuda")
    say(f"[window] whole-prompt chunk vs contiguous prefill, W=90, bitwise, PA_PREFILL_STAGE_V={stage}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.k.reshape(-1, c.n_kv, c.head_dim), c.v.reshape(-1, c.n_kv, c.head_dim),
                 c.prompt_slots, kp, vp)
    ctx = torch.full((c.batch,), c.seq_len, dtype=torch.int32, device="cuda")
    paged = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, ctx, c.scale, window=90)
    contig = pa.paged_attn_prefill(c.q, c.k, c.v, True, c.scale, window=90)
    torch.cuda.synchronize()
    assert same_bits(paged, contig)


def test_window_rejections_reach_python(pa):
    c = _decode_case("gqa2_f32_d128")
    with pytest.raises(pa.PagedAttnError, match="window"):
        pa.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                             window=-1)
    q = torch.zeros(1, 8, 4, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pa.PagedAttnError, match="causal"):
        pa.paged_attn_prefill(q, kv, kv, False, 0.1, window=4)


def test_window_bench_shape_all_rows(pa):
    """The bench's sliding-window step at full size (B=32, 32/8 heads, d=128, bf16, contexts of
    16384, W=4096, the new token appended in the same launch): every row against the oracle,
    into a NaN-filled output, and every row again after poisoning the entries before the window."""
    from gpu_helpers import nan_out
    c = wl.make_window_decode_case(device="cuda")
    W = wl.WINDOW_TOKENS
    say(f"[window] 8B shape, ctx 16384, W={W}, fused step, full size, all rows")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    out = nan_out((c.batch, c.n_q, c.head_dim))
    pa.paged_attn_decode_append(c.q, c.new_k, c.new_v, c.slot_mapping, kp, vp, c.block_table,
                                c.context_lens, c.scale, out=out, window=W)
    torch.cuda.synchronize()
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), c.dtype,
                         c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale, window=W)
    stats = assert_parity(out.cpu().numpy(), want, c.dtype, "window 8B shape, all 1024 rows")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
    bt = _poison_before(c.block_table, c.context_lens, 1, W)
    again = pa.paged_attn_decode(c.q, kp, vp, bt, c.context_lens, c.scale, window=W)
    torch.cuda.synchronize()
    assert same_bits(out, again), "the fused step and the plain decode after it must agree bit for bit"
