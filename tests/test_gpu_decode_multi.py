"""GPU parity of multi-row decode (several new tokens per sequence) against the oracle.

The q_rows new tokens of each sequence are appended into the paged pools
(kv_append), then pa_paged_attn_decode_multi attends. Row r is position
ctx - q_rows + r, so the oracle is the chunked-prefill definition with
chunk_len = q_rows. Every output row is compared.
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


def appended(pa, c):
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    return kp, vp


def gpu_multi(pa, c, out_dtype=torch.float32):
    kp, vp = appended(pa, c)
    out = pa.paged_attn_decode_multi(c.q, kp, vp, c.block_table, c.context_lens, c.scale,
                                     out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_multi(c):
    kp, vp = stored_np(c.k_pool).copy(), stored_np(c.v_pool).copy()
    oracle.kv_append(stored_np(c.chunk_k), stored_np(c.chunk_v), c.chunk_slots.cpu().numpy(), kp, vp)
    return oracle.chunked_prefill(stored_np(c.q), kp, vp, c.dtype, c.block_table.cpu().numpy(),
                                  c.context_lens.cpu().numpy(), c.scale)


SHAPES = [
    # (batch, q_rows, prefix lengths, n_q, n_kv, head_dim, dtype)
    (4, 4, [100, 2047, 5, 600], 32, 8, 128, "bf16"),
    (2, 8, [300, 4000], 64, 8, 128, "bf16"),       # 64 (row, head) pairs: 2 row groups; split contexts
    (3, 2, [0, 17, 33], 8, 2, 64, "f16"),
    (2, 1, [200, 31], 8, 1, 128, "bf16"),          # MQA, a single row
    (1, 5, [3], 4, 4, 128, "bf16"),                # MHA, short context
    (2, 3, [9000, 20], 16, 4, 128, "bf16"),        # 5 partitions for the long one
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}_R{s[1]}_P{'-'.join(map(str, s[2]))}_{s[3]}x{s[4]}_d{s[5]}_{s[6]}"
                                               for s in SHAPES])
def test_decode_multi_matches_oracle(pa, shape):
    B, R, pre, n_q, n_kv, d, dt = shape
    c = wl.make_chunk_case(batch=B, chunk_len=R, prefix_lens=pre, n_q=n_q, n_kv=n_kv, head_dim=d,
                           dtype=dt, free_fraction=0.2, seed=sum(pre) + 7 * R + d, device="cuda")
    say(f"[multi] B={B} rows={R} prefix={pre} n_q={n_q} n_kv={n_kv} d={d} {dt}")
    got = gpu_multi(pa, c)
    stats = assert_parity(got.cpu().numpy(), oracle_multi(c), dt, "multi-row decode")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


@pytest.mark.parametrize("tokens", [256, 1024])
def test_partition_sizes_agree(pa, tokens):
    c = wl.make_chunk_case(batch=2, chunk_len=4, prefix_lens=[3000, 700], n_q=16, n_kv=4,
                           head_dim=128, dtype="bf16", seed=61, device="cuda")
    say(f"[multi] partitions of {tokens} tokens")
    prev = pa.set_decode_partition_tokens(tokens)
    try:
        got = gpu_multi(pa, c)
    finally:
        pa.set_decode_partition_tokens(prev)
    assert_parity(got.cpu().numpy(), oracle_multi(c), "bf16", f"partition {tokens}")


@pytest.mark.parametrize("kernel", ["mfma", "multi"])
def test_blocks_past_the_first_rows_position(pa, option, kernel):
    """One block per wave: a wave whose only block lies past row 0's position (or
    wholly before a later row's window) attends nothing for that row's columns,
    which must give weights of 0, not NaN."""
    if kernel == "multi":
        option("decode_matrix_cores", 0)
    c = wl.make_chunk_case(batch=4, chunk_len=4, prefix_lens=[93, 77, 12, 2000], n_q=32, n_kv=8,
                           head_dim=128, dtype="bf16", seed=64, device="cuda")
    say(f"[multi] {kernel}: contexts {[p + 4 for p in (93, 77, 12, 2000)]}, one block per wave")
    prev = pa.set_decode_partition_tokens(128 if kernel == "mfma" else 256)
    try:
        got = gpu_multi(pa, c)
    finally:
        pa.set_decode_partition_tokens(prev)
    assert_parity(got.cpu().numpy(), oracle_multi(c), "bf16", f"{kernel}: short runs")


def test_agrees_with_chunked_prefill_and_is_reproducible(pa):
    c = wl.make_chunk_case(batch=3, chunk_len=6, prefix_lens=[50, 1500, 2600], n_q=32, n_kv=8,
                           head_dim=128, dtype="bf16", free_fraction=0.2, seed=62, device="cuda")
    say("[multi] vs chunked prefill; run twice")
    kp, vp = appended(pa, c)
    a = pa.paged_attn_decode_multi(c.q, kp, vp, c.block_table, c.context_lens, c.scale)
    b = pa.paged_attn_decode_multi(c.q, kp, vp, c.block_table, c.context_lens, c.scale)
    ch = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, c.scale)
    torch.cuda.synchronize()
    assert same_bits(a, b)
    assert float((a - ch).abs().max()) <= 2e-3


def test_relabelled_blocks_give_identical_bits(pa):
    c = wl.make_chunk_case(batch=2, chunk_len=4, prefix_lens=[2500, 90], n_q=16, n_kv=4,
                           head_dim=128, dtype="bf16", free_fraction=0.25, seed=63, device="cuda")
    say("[multi] physical relabelling")
    first = gpu_multi(pa, c)
    perm = torch.as_tensor(np.random.default_rng(3).permutation(c.num_blocks), device="cuda")
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(c.num_blocks, device="cuda")
    c2 = wl.ChunkCase(**{k: getattr(c, k) for k in c.__dataclass_fields__})
    c2.k_pool, c2.v_pool = c.k_pool[inv], c.v_pool[inv]
    c2.block_table = perm[c.block_table.long()].int()
    c2.chunk_slots = perm[c.chunk_slots // 16] * 16 + c.chunk_slots % 16
    assert same_bits(first, gpu_multi(pa, c2))


def test_short_context_and_bad_metadata(pa):
    c = wl.make_chunk_case(batch=4, chunk_len=4, prefix_lens=[40, 40, 40, 40], n_q=8, n_kv=2,
                           head_dim=128, dtype="bf16", free_fraction=0.3, seed=64, device="cuda")
    say("[multi] context shorter than the rows, over-long context, out-of-pool block id")
    kp, vp = appended(pa, c)
    ctx = c.context_lens.clone()
    ctx[0] = 2                                   # rows 0 and 1 sit before the sequence start
    ctx[2] = c.max_blocks_per_seq * 16 + 1
    bt = c.block_table.clone()
    bt[3, 0] = c.num_blocks + 9
    out = pa.paged_attn_decode_multi(c.q, kp, vp, bt, ctx, c.scale)
    torch.cuda.synchronize()
    out = out.cpu()
    assert (out[0, :2] == 0).all()
    assert torch.isnan(out[2]).all() and torch.isnan(out[3]).all()
    want = oracle.chunked_prefill(stored_np(c.q[:2]), *oracle_pools(c), "bf16",
                                  c.block_table[:2].cpu().numpy(), ctx[:2].cpu().numpy(), c.scale)
    assert_parity(out[0, 2:].numpy(), want[0, 2:], "bf16", "rows of the short sequence")
    assert_parity(out[1].numpy(), want[1], "bf16", "sequence next to bad metadata")


def test_bf16_output(pa):
    c = wl.make_chunk_case(batch=2, chunk_len=4, prefix_lens=[700, 2100], n_q=32, n_kv=8,
                           head_dim=128, dtype="bf16", seed=65, device="cuda")
    say("[multi] bf16 output")
    got = gpu_multi(pa, c, out_dtype=torch.bfloat16).float().cpu().numpy()
    want = oracle_multi(c)
    assert (np.abs(got - want) <= 2e-3 + 2.0**-8 * np.abs(want)).all()


def test_full_size_4_rows_on_the_8b_shape_all_rows(pa):
    """The bench's speculative-verification shape: B=32, 4 new rows per sequence, 32/8 heads,
    d=128, contexts of 2048 including the new rows, bf16; every one of the 4096 output rows
    against the oracle, into a NaN-filled output."""
    from gpu_helpers import nan_out
    c = wl.make_chunk_case(batch=32, chunk_len=4, prefix_lens=[2044] * 32, n_q=32, n_kv=8, head_dim=128,
                           dtype="bf16", seed=1007, device="cuda")
    say("[multi] 8B shape, 4 rows per sequence, full size, all rows")
    kp, vp = appended(pa, c)
    out = nan_out(tuple(c.q.shape))
    pa.paged_attn_decode_multi(c.q, kp, vp, c.block_table, c.context_lens, c.scale, out=out)
    torch.cuda.synchronize()
    stats = assert_parity(out.cpu().numpy(), oracle_multi(c), "bf16", "multi-row 8B, all 4096 rows")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
