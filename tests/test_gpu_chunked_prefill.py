"""GPU parity of chunked prefill over a paged prefix against the fp64 oracle.

Each case appends the chunk's K/V into the paged pools (kv_append), then runs
pa_paged_attn_chunked_prefill; the oracle does the same with its own append
and its chunked-prefill definition. Every output row is compared.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, oracle_pools, same_bits, say, stored_np
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_gqa_attention_attn_amd as pa
    pa._lib.load()  # raises if the HIP library is missing: no fallback
    return pa


def gpu_chunk(pa, c, out_dtype=torch.float32):
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    out = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, c.scale,
                                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_chunk(c, sel=None):
    kp, vp = stored_np(c.k_pool).copy(), stored_np(c.v_pool).copy()
    oracle.kv_append(stored_np(c.chunk_k), stored_np(c.chunk_v), c.chunk_slots.cpu().numpy(), kp, vp)
    return oracle.chunked_prefill(stored_np(c.q), kp, vp, c.dtype, c.block_table.cpu().numpy(),
                                  c.context_lens.cpu().numpy(), c.scale, sel=sel)


SHAPES = [
    # (batch, chunk_len, prefix lengths, n_q, n_kv, head_dim, dtype)
    (2, 64, [0, 0], 8, 2, 128, "bf16"),
    (2, 17, [5, 40], 8, 2, 128, "bf16"),
    (3, 128, [100, 333, 0], 32, 8, 128, "bf16"),
    (1, 200, [700], 4, 4, 64, "f16"),
    (2, 1, [50, 3], 8, 1, 128, "bf16"),
    (2, 300, [1000, 17], 16, 4, 128, "f16"),
    (1, 130, [64], 8, 2, 64, "bf16"),
    (3, 150, [10, 400, 77], 6, 2, 128, "bf16"),   # 36 work items: not a multiple of 8 XCDs
    (1, 257, [33], 3, 1, 64, "f16"),              # 9 work items
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}_C{s[1]}_P{'-'.join(map(str, s[2]))}_{s[3]}x{s[4]}_d{s[5]}_{s[6]}"
                                               for s in SHAPES])
def test_chunked_prefill_matches_oracle(pa, shape):
    B, C, pre, n_q, n_kv, d, dt = shape
    c = wl.make_chunk_case(batch=B, chunk_len=C, prefix_lens=pre, n_q=n_q, n_kv=n_kv, head_dim=d,
                           dtype=dt, free_fraction=0.2, seed=sum(pre) + 31 * C + d, device="cuda")
    say(f"[chunk] B={B} C={C} prefix={pre} n_q={n_q} n_kv={n_kv} d={d} {dt}")
    got = gpu_chunk(pa, c)
    want = oracle_chunk(c)
    stats = assert_parity(got.cpu().numpy(), want, dt, "chunked prefill")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


@pytest.mark.parametrize("stage", ["1", "0"], ids=["staged", "unstaged"])
def test_whole_prompt_chunk_equals_contiguous_prefill_bitwise(pa, option, stage):
    # A chunk that is the whole prompt runs the same tile arithmetic as the
    # contiguous prefill kernel (both with V copied to f16, or both without):
    # every output bit must agree.
    option("prefill_stage_v", int(stage))
    c = wl.make_prefill_case(batch=2, seq_len=300, n_q=8, n_kv=2, head_dim=128, dtype="bf16",
                             seed=77, device="cuda")
    say(f"[chunk] whole-prompt chunk vs contiguous prefill, bitwise, PA_PREFILL_STAGE_V={stage}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.k.reshape(-1, c.n_kv, c.head_dim), c.v.reshape(-1, c.n_kv, c.head_dim),
                 c.prompt_slots, kp, vp)
    ctx = torch.full((c.batch,), c.seq_len, dtype=torch.int32, device="cuda")
    paged = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, ctx, c.scale)
    contig = pa.paged_attn_prefill(c.q, c.k, c.v, True, c.scale)
    torch.cuda.synchronize()
    assert same_bits(paged, contig)


@pytest.mark.parametrize("where", ["prefix", "chunk"])
def test_chunked_prefill_v_beyond_f16_matches_oracle(pa, where):
    """A finite V value past f16's range (70144) in one block: workgroups whose rows
    read that block keep the bf16 hi + lo product, the others use the f16 copy. The
    dimension holding it scales with the value, so it is checked norm-wise relative;
    every other dimension against the usual bound."""
    c = wl.make_chunk_case(batch=2, chunk_len=200, prefix_lens=[300, 60], n_q=8, n_kv=2,
                           head_dim=128, dtype="bf16", free_fraction=0.2, seed=401, device="cuda")
    say(f"[chunk] one V value of 70144 in the {where}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    cv = c.chunk_v.clone()
    if where == "chunk":                    # sequence 0, chunk row 150 = position 450, KV head 1
        cv[150, 1, 7] = 70144.0
        e, h0 = 7, 4
    pa.kv_append(c.chunk_k, cv, c.chunk_slots, kp, vp)
    if where == "prefix":                   # sequence 0, position 83, KV head 0
        vp[int(c.block_table[0, 5]), 0, 3, 11] = 70144.0
        e, h0 = 11, 0
    got = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, c.scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    okp, ovp = oracle_pools(c, v_new=cv)      # the same edits on the oracle's own pools
    if where == "prefix":
        ovp[int(c.block_table[0, 5]), 0, 3, 11] = stored_np(torch.tensor([70144.0], dtype=torch.bfloat16))[0]
    want = oracle.chunked_prefill(stored_np(c.q), okp, ovp, "bf16",
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale)
    assert np.isfinite(got).all()
    big = np.zeros(got.shape, bool)
    big[0, :, h0:h0 + 4, e] = True
    assert_parity(got[~big], want[~big], "bf16", "dimensions without the large value")
    g_, w_ = got[0, :, h0:h0 + 4, e], want[0, :, h0:h0 + 4, e]
    rel = np.abs(g_ - w_).max() / np.abs(w_).max()
    say(f"    heads {h0}..{h0 + 3} dim {e}: norm-wise rel {rel:.2e}")
    assert rel <= 1e-3, rel


def test_relabelled_blocks_give_identical_bits(pa):
    c = wl.make_chunk_case(batch=2, chunk_len=70, prefix_lens=[90, 250], n_q=8, n_kv=2,
                           head_dim=128, dtype="bf16", free_fraction=0.25, seed=5, device="cuda")
    say("[chunk] physical relabelling")
    first = gpu_chunk(pa, c)
    perm = torch.as_tensor(np.random.default_rng(9).permutation(c.num_blocks), device="cuda")
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(c.num_blocks, device="cuda")
    c2 = wl.ChunkCase(**{k: getattr(c, k) for k in c.__dataclass_fields__})
    c2.k_pool = c.k_pool[inv]            # new block i holds old block inv[i]; old b -> new perm[b]
    c2.v_pool = c.v_pool[inv]
    c2.block_table = perm[c.block_table.long()].int()
    bs = c.block_size
    c2.chunk_slots = perm[(c.chunk_slots // bs)] * bs + c.chunk_slots % bs
    second = gpu_chunk(pa, c2)
    assert same_bits(first, second)


def test_short_context_and_bad_metadata(pa):
    c = wl.make_chunk_case(batch=4, chunk_len=20, prefix_lens=[30, 30, 30, 30], n_q=8, n_kv=2,
                           head_dim=128, dtype="bf16", free_fraction=0.3, seed=12, device="cuda")
    say("[chunk] context shorter than the chunk, over-long context, out-of-pool block id")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    ctx = c.context_lens.clone()
    ctx[0] = 7                                   # rows 0..12 sit before the sequence start
    ctx[2] = c.max_blocks_per_seq * 16 + 1       # past the block table's reach
    bt = c.block_table.clone()
    bt[3, 1] = c.num_blocks + 3                  # a block the rows read, outside the pool
    out = pa.paged_attn_chunked_prefill(c.q, kp, vp, bt, ctx, c.scale)
    torch.cuda.synchronize()
    out = out.cpu()
    assert (out[0, :13] == 0).all(), "rows at negative positions must be zero"
    assert torch.isnan(out[2]).all() and torch.isnan(out[3]).all()
    want = oracle.chunked_prefill(stored_np(c.q[:2]), *oracle_pools(c), "bf16",
                                  c.block_table[:2].cpu().numpy(), ctx[:2].cpu().numpy(), c.scale)
    assert_parity(out[0, 13:].numpy(), want[0, 13:], "bf16", "rows of the short sequence")
    assert_parity(out[1].numpy(), want[1], "bf16", "sequence next to bad metadata")


def test_bf16_output(pa):
    c = wl.make_chunk_case(batch=2, chunk_len=96, prefix_lens=[64, 200], n_q=8, n_kv=2,
                           head_dim=128, dtype="bf16", seed=21, device="cuda")
    say("[chunk] bf16 output")
    got = gpu_chunk(pa, c, out_dtype=torch.bfloat16).float().cpu().numpy()
    want = oracle_chunk(c)
    assert (np.abs(got - want) <= 2e-3 + 2.0**-8 * np.abs(want)).all()


def test_chunked_prefill_past_the_copy_cap_keeps_the_bf16_product(pa, option):
    """A block table 9000 blocks wide over 8 KV heads would need a 295 MB f16 copy of V,
    past the 256 MiB a call stages: P V then keeps the bf16 hi + lo product. The result
    matches the oracle and, bit for bit, the same call on the narrow table with the copy
    switched off."""
    c = wl.make_chunk_case(batch=2, chunk_len=130, prefix_lens=[400, 33], n_q=16, n_kv=8,
                           head_dim=128, dtype="bf16", free_fraction=0.2, seed=902, device="cuda")
    say("[chunk] 9000-block table: past the f16 copy's size cap")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    wide = torch.full((c.batch, 9000), -1, dtype=torch.int32, device="cuda")   # unused entries
    wide[:, :c.max_blocks_per_seq] = c.block_table
    got = pa.paged_attn_chunked_prefill(c.q, kp, vp, wide, c.context_lens, c.scale)
    option("prefill_stage_v", 0)
    unstaged = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, c.scale)
    torch.cuda.synchronize()
    want = oracle.chunked_prefill(stored_np(c.q), *oracle_pools(c), "bf16",
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale)
    stats = assert_parity(got.cpu().numpy(), want, "bf16", "chunked prefill, 9000-block table")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
    assert same_bits(got, unstaged)


def test_chunked_prefill_bench_shape_all_rows(pa):
    """The bench's chunked prefill at full size: 2 sequences, a 1024-token chunk over a
    3072-token paged prefix, 32/8 heads, d=128, bf16 (f16 copy of V); all 65536 (row, head)
    outputs against the oracle, into a NaN-filled output."""
    from gpu_helpers import nan_out
    c = wl.make_chunk_case(batch=2, chunk_len=1024, prefix_lens=[3072, 3072], n_q=32, n_kv=8, head_dim=128,
                           dtype="bf16", free_fraction=0.2, seed=3, device="cuda")
    say("[chunk] bench shape 2 x 1024 over 3072, full size, all rows")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    out = nan_out(tuple(c.q.shape))
    pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, c.scale, out=out)
    torch.cuda.synchronize()
    stats = assert_parity(out.cpu().numpy(), oracle_chunk(c), "bf16", "chunked prefill 2 x 1024 over 3072, all rows")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
