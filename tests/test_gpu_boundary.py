"""The C ABI's workspace options and its validate debug mode, on the GPU.

Every call here goes through the C ABI with real device buffers. The results
with a library-owned or a default workspace must equal, bit for bit, those with
an explicit one; the validate option must reject bad device metadata before anything
is enqueued, and leave valid calls' results unchanged.
"""
import ctypes

import pytest
import torch

from gpu_helpers import same_bits, say
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


@pytest.fixture
def validate(option):
    option("validate", 1)
    return option


def _split_case():
    # 2048-token partitions: contexts of 5000 tokens need a workspace.
    return wl.make_decode_case(batch=3, n_q=16, n_kv=2, head_dim=128, context_lens=[5000, 4097, 700],
                               dtype="bf16", free_fraction=0.1, seed=71, device="cuda", name="split")


def _desc(case):
    return _lib.CacheDesc(case.num_blocks, 16, case.n_kv, case.head_dim, _lib.PA_BF16)


def _raw_decode(case, bt, ctx, out, ws, ws_bytes):
    L = _lib.load()
    desc = _desc(case)
    return L.pa_paged_attn_decode(
        case.q.data_ptr(), case.batch, case.n_q, case.k_pool.data_ptr(), case.v_pool.data_ptr(),
        ctypes.byref(desc), bt.data_ptr(), case.max_blocks_per_seq, ctx.data_ptr(), case.scale,
        0, None, out.data_ptr(), _lib.PA_F32, ws, ws_bytes, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_null_workspace_uses_the_librarys_own(pa):
    case = _split_case()
    need = pa.decode_workspace_bytes(case.batch, case.n_q, case.max_blocks_per_seq, case.k_pool)
    assert need > 0
    say(f"[boundary] library-owned workspace ({need} bytes needed)")
    want = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                                case.scale)
    got = torch.full_like(want, float("nan"))
    assert _raw_decode(case, case.block_table, case.context_lens, got, None, 0) == 0, _lib.last_error()
    again = torch.full_like(want, float("nan"))
    assert _raw_decode(case, case.block_table, case.context_lens, again, None, 0) == 0, _lib.last_error()
    torch.cuda.synchronize()
    assert same_bits(got, want) and same_bits(again, want)


def test_default_workspace(pa):
    case = _split_case()
    need = pa.decode_workspace_bytes(case.batch, case.n_q, case.max_blocks_per_seq, case.k_pool)
    say("[boundary] pa_set_workspace")
    want = pa.paged_attn_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.context_lens,
                                case.scale)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    pa.set_workspace(ws)
    try:
        got = torch.full_like(want, float("nan"))
        assert _raw_decode(case, case.block_table, case.context_lens, got, None, 0) == 0, _lib.last_error()
        torch.cuda.synchronize()
        assert ws.any(), "the default workspace was not used"
    finally:
        pa.set_workspace(None)
    assert same_bits(got, want)


def test_validate_passes_good_calls_unchanged(pa, validate):
    case = _split_case()
    say("[boundary] the validate option on valid metadata")
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    pa.kv_append(case.new_k, case.new_v, case.slot_mapping, kp, vp)
    got = pa.paged_attn_decode(case.q, kp, vp, case.block_table, case.context_lens, case.scale)
    validate("validate", 0)
    kp2, vp2 = case.k_pool.clone(), case.v_pool.clone()
    pa.kv_append(case.new_k, case.new_v, case.slot_mapping, kp2, vp2)
    want = pa.paged_attn_decode(case.q, kp2, vp2, case.block_table, case.context_lens, case.scale)
    torch.cuda.synchronize()
    assert same_bits(kp, kp2) and same_bits(vp, vp2) and same_bits(got, want)


def test_validate_rejects_bad_decode_metadata(pa, validate):
    case = _split_case()
    out = torch.full((case.batch, case.n_q, case.head_dim), 7.0, device="cuda")
    ws = torch.empty(pa.decode_workspace_bytes(case.batch, case.n_q, case.max_blocks_per_seq, case.k_pool),
                     dtype=torch.uint8, device="cuda")
    bt = case.block_table.clone()
    bt[1, 3] = case.num_blocks          # inside sequence 1's context, outside the pool
    say("[boundary] validate rejects an out-of-pool block id")
    assert _raw_decode(case, bt, case.context_lens, out, ws.data_ptr(), ws.numel()) == _lib.PA_ERR_INVALID_ARG
    assert "block_table[1][3]" in _lib.last_error()
    ctx = case.context_lens.clone()
    ctx[2] = case.max_blocks_per_seq * 16 + 1
    say("[boundary] validate rejects a context past the block table")
    assert _raw_decode(case, case.block_table, ctx, out, ws.data_ptr(), ws.numel()) == _lib.PA_ERR_INVALID_ARG
    assert "context_lens[2]" in _lib.last_error()
    torch.cuda.synchronize()
    assert (out == 7.0).all(), "a rejected call must not enqueue work"


def test_validate_rejects_bad_slots(pa, validate):
    case = wl.make_config(1, device="cuda")
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    say("[boundary] validate rejects repeated and out-of-pool slots")
    dup = torch.tensor([5, 5], dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PagedAttnError, match="twice"):
        pa.kv_append(case.new_k, case.new_v, dup, kp, vp)
    past = torch.tensor([-1, case.num_blocks * 16], dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PagedAttnError, match="past the pool"):
        pa.kv_append(case.new_k, case.new_v, past, kp, vp)
    torch.cuda.synchronize()
    assert same_bits(kp, case.k_pool) and same_bits(vp, case.v_pool)


def test_validate_rejects_misplaced_fused_append(pa, validate):
    case = wl.make_config(1, device="cuda")
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    slots = case.slot_mapping.clone()
    slots[0] += 1                          # not position ctx - 1 of sequence 0
    say("[boundary] validate rejects a fused append at the wrong slot")
    with pytest.raises(pa.PagedAttnError, match="position"):
        pa.paged_attn_decode_append(case.q, case.new_k, case.new_v, slots, kp, vp, case.block_table,
                                    case.context_lens, case.scale)
    out = pa.paged_attn_decode_append(case.q, case.new_k, case.new_v, case.slot_mapping, kp, vp,
                                      case.block_table, case.context_lens, case.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
