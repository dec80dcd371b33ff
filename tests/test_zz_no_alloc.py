"""pa_paged_attn_decode_noalloc through the C ABI on the GPU.

The entry point for callers that cannot allocate must give, bit for bit, the
output of pa_paged_attn_decode (called with an explicit workspace) on the same
arguments: here with contexts split into partitions, so that its partials go to
the library's fixed scratch array, on two calls in a row, the second with a
smaller input, and once more without a split. A request whose partials exceed
the array is refused before anything is enqueued.
"""
import ctypes

import pytest
import torch

import oracle
from gpu_helpers import assert_parity, nan_out, same_bits, say, stored_np
from paged_gqa_attention_attn_amd import _lib
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20     # PA_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _lib.load()   # raises if the HIP library is missing: no fallback


def _desc(c):
    return _lib.CacheDesc(c.num_blocks, 16, c.n_kv, c.head_dim, _lib.PA_BF16)


def _args(c, out):
    return (c.q.data_ptr(), c.batch, c.n_q, c.k_pool.data_ptr(), c.v_pool.data_ptr(), ctypes.byref(_desc(c)),
            c.block_table.data_ptr(), c.max_blocks_per_seq, c.context_lens.data_ptr(), c.scale, 0, None,
            out.data_ptr(), _lib.PA_F32)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _appended(c):
    """The case with each sequence's new token written at its last position (the
    generator leaves that slot NaN until then)."""
    import paged_gqa_attention_attn_amd as pa
    pa.kv_append(c.new_k, c.new_v, c.slot_mapping, c.k_pool, c.v_pool)
    return c


def _both(L, c):
    """(reference, noalloc) outputs of the same decode, each into a NaN-filled buffer."""
    need = L.pa_decode_workspace_bytes(c.batch, c.n_q, c.max_blocks_per_seq, ctypes.byref(_desc(c)))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    ref = nan_out((c.batch, c.n_q, c.head_dim))
    got = nan_out((c.batch, c.n_q, c.head_dim))
    assert L.pa_paged_attn_decode(*_args(c, ref), ws.data_ptr(), ws.numel(), _stream()) == 0, _lib.last_error()
    assert L.pa_paged_attn_decode_noalloc(*_args(c, got), _stream()) == 0, _lib.last_error()
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    return need, ref, got


def test_noalloc_equals_decode_twice_then_smaller(L):
    prev = L.pa_set_decode_partition_tokens(256)    # split every context longer than 256 tokens
    try:
        big = wl.make_decode_case(batch=6, n_q=32, n_kv=8, head_dim=128, context_lens=[4000, 1, 700, 2500, 33, 3100],
                                  dtype="bf16", free_fraction=0.1, seed=61, device="cuda", name="noalloc_big")
        big = _appended(big)
        small = wl.make_decode_case(batch=2, n_q=8, n_kv=2, head_dim=128, context_lens=[600, 290],
                                    dtype="bf16", free_fraction=0.1, seed=62, device="cuda", name="noalloc_small")
        small = _appended(small)
        for what, c in (("first call", big), ("second call, smaller", small)):
            need, ref, got = _both(L, c)
            say(f"[noalloc] {what}: B={c.batch} n_q={c.n_q} ctx={c.context_lens.tolist()} partials {need} bytes")
            assert 0 < need <= SCRATCH_BYTES
            assert same_bits(got, ref), f"{what}: output differs from pa_paged_attn_decode"
            want = oracle.decode(stored_np(c.q), stored_np(c.k_pool), stored_np(c.v_pool), "bf16",
                                 c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale)
            assert_parity(got.cpu().numpy(), want, "bf16", f"noalloc {what}")
    finally:
        L.pa_set_decode_partition_tokens(prev)
    # Contexts within one block: no partials at all.
    tiny = wl.make_decode_case(batch=3, n_q=8, n_kv=2, head_dim=128, context_lens=[5, 16, 1], dtype="bf16",
                               free_fraction=0.2, seed=64, device="cuda", name="noalloc_tiny")
    tiny = _appended(tiny)
    need, ref, got = _both(L, tiny)
    assert need == 0 and same_bits(got, ref)


def test_noalloc_refuses_partials_beyond_the_scratch(L):
    prev = L.pa_set_decode_partition_tokens(16)     # one partition per block: a large need
    try:
        c = wl.make_decode_case(batch=4, n_q=64, n_kv=1, head_dim=128, context_lens=[33000, 20, 33000, 9000],
                                dtype="bf16", free_fraction=0.0, seed=63, device="cuda", name="noalloc_huge")
        need = L.pa_decode_workspace_bytes(c.batch, c.n_q, c.max_blocks_per_seq, ctypes.byref(_desc(c)))
        assert need > SCRATCH_BYTES
        out = torch.full((c.batch, c.n_q, c.head_dim), 7.0, device="cuda")
        say(f"[noalloc] refusal: partials {need} bytes > {SCRATCH_BYTES}")
        assert L.pa_paged_attn_decode_noalloc(*_args(c, out), _stream()) == _lib.PA_ERR_INVALID_ARG
        assert "scratch" in _lib.last_error()
        torch.cuda.synchronize()
        assert (out == 7.0).all(), "a refused call must enqueue nothing"
    finally:
        L.pa_set_decode_partition_tokens(prev)
