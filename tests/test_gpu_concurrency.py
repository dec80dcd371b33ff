"""The library's shared workspace under concurrent host threads, and calls on a
side stream, through the C ABI on the GPU.

Two host threads issue decode calls with growing context lengths on one stream,
each passing no workspace, so both use the library's own buffer while it grows.
A buffer that a larger one replaces must stay valid for calls that already hold
it, and one call's partition and merge kernels must not interleave with the
other thread's on the shared buffer. Every output must equal, bit for bit, the
same call made alone with an explicit workspace. The binding's side-stream
calls must match the oracle with outputs and scratch it allocated itself.
"""
import ctypes
import threading

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, nan_out, oracle_pools, same_bits, say, stored_np
from paged_gqa_attention_attn_amd import _lib
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_gqa_attention_attn_amd as pa
    pa._lib.load()  # raises if the HIP library is missing: no fallback
    return pa


def _case(ctx, seed):
    return wl.make_decode_case(batch=2, n_q=16, n_kv=2, head_dim=128, context_lens=[ctx, ctx // 3 + 1],
                               dtype="bf16", free_fraction=0.1, seed=seed, device="cuda", name="grow")


def _raw_decode(case, out, stream):
    L = _lib.load()
    desc = _lib.CacheDesc(case.num_blocks, 16, case.n_kv, case.head_dim, _lib.PA_BF16)
    return L.pa_paged_attn_decode(
        case.q.data_ptr(), case.batch, case.n_q, case.k_pool.data_ptr(), case.v_pool.data_ptr(),
        ctypes.byref(desc), case.block_table.data_ptr(), case.max_blocks_per_seq,
        case.context_lens.data_ptr(), case.scale, 0, None, out.data_ptr(), _lib.PA_F32, None, 0,
        ctypes.c_void_p(stream.cuda_stream))


def test_two_threads_grow_the_library_workspace(pa):
    # 256-token partitions: each longer context needs a larger partial-result buffer.
    prev = pa.set_decode_partition_tokens(256)
    try:
        sizes = [300, 900, 2000, 4100, 7000, 12000]
        cases = {(t, i): _case(n, 100 * t + i) for t in range(2) for i, n in enumerate(sizes)}
        want = {}
        for key, c in cases.items():
            want[key] = pa.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        outs = {key: nan_out((c.batch, c.n_q, c.head_dim)) for key, c in cases.items()}
        errors = []
        barrier = threading.Barrier(2)

        def worker(t):
            barrier.wait()
            for rep in range(3):
                for i in range(len(sizes)):
                    rc = _raw_decode(cases[(t, i)], outs[(t, i)], stream)
                    if rc != 0:
                        errors.append((t, i, rc, _lib.last_error()))

        say(f"[concurrency] two threads, growing library workspace, sizes {sizes}")
        threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        torch.cuda.synchronize()
    finally:
        pa.set_decode_partition_tokens(prev)
    assert not errors, errors
    for key in cases:
        assert same_bits(outs[key], want[key]), f"thread {key[0]}, size {sizes[key[1]]}: output differs"


def test_side_stream_calls_match_the_oracle(pa):
    """Outputs and scratch the binding allocates belong to the stream the kernels run on."""
    c = _case(5000, 7)
    side = torch.cuda.Stream()
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    torch.cuda.synchronize()
    say("[concurrency] decode, prefill and chunked prefill on a side stream")
    prev = pa.set_decode_partition_tokens(512)
    try:
        pa.kv_append(c.new_k, c.new_v, c.slot_mapping, kp, vp, stream=side)
        outs = [pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale, stream=side)
                for _ in range(3)]
        # Churn the default stream's allocator while the side stream runs.
        junk = [torch.full((1 << 20,), 3.0, device="cuda") for _ in range(8)]
        del junk
    finally:
        pa.set_decode_partition_tokens(prev)
    g = torch.Generator(device="cuda").manual_seed(3)
    q = torch.randn(1, 300, 8, 128, generator=g, device="cuda").bfloat16()
    k = torch.randn(1, 300, 2, 128, generator=g, device="cuda").bfloat16()
    v = torch.randn(1, 300, 2, 128, generator=g, device="cuda").bfloat16()
    side.wait_stream(torch.cuda.current_stream())
    pre = pa.paged_attn_prefill(q, k, v, True, 0.1, stream=side)
    ch = wl.make_chunk_case(batch=2, chunk_len=64, prefix_lens=[100, 500], n_q=8, n_kv=2, head_dim=128,
                            dtype="bf16", free_fraction=0.1, seed=5, device="cuda", name="side")
    ckp, cvp = ch.k_pool.clone(), ch.v_pool.clone()
    side.wait_stream(torch.cuda.current_stream())
    pa.kv_append(ch.chunk_k, ch.chunk_v, ch.chunk_slots, ckp, cvp, stream=side)
    chunk = pa.paged_attn_chunked_prefill(ch.q, ckp, cvp, ch.block_table, ch.context_lens, ch.scale, stream=side)
    side.synchronize()
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), "bf16", c.block_table.cpu().numpy(),
                         c.context_lens.cpu().numpy(), c.scale)
    for o in outs:
        assert_parity(o.cpu().numpy(), want, "bf16", "side-stream decode")
    assert_parity(pre.cpu().numpy(), oracle.prefill(stored_np(q), stored_np(k), stored_np(v), "bf16", True, 0.1),
                  "bf16", "side-stream prefill")
    wc = oracle.chunked_prefill(stored_np(ch.q), *oracle_pools(ch), "bf16",
                                ch.block_table.cpu().numpy(), ch.context_lens.cpu().numpy(), ch.scale)
    assert_parity(chunk.cpu().numpy(), wc, "bf16", "side-stream chunked prefill")
    assert np.isfinite(chunk.cpu().numpy()).all()
