"""GPU parity of kv_append + paged decode against the fp64 CPU oracle.

Every case runs the library's HIP kernels through the C ABI and compares with
the oracle on the same seeded inputs: kv_append bit-exact, decode within
max-abs 2e-3 and norm-wise relative 1e-2 for bf16/fp16 (1e-5 for fp32).

Each test runs twice: with the default kernel choice (the matrix-core decode for
bf16/f16 caches whose group size is a multiple of 4, the VALU kernel otherwise)
and with PA_DECODE_MFMA=0, which forces the VALU kernel everywhere.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, gpu_step, nan_out, oracle_step, same_bits, say, stored_np
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["default", "valu"], autouse=True)
def decode_kernel(request, option):
    option("decode_matrix_cores", 0 if request.param == "valu" else 1)
    return request.param


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_gqa_attention_attn_amd as pa
    pa._lib.load()  # raises if the HIP library is missing: no fallback
    return pa


def check_full(pa, case, what):
    say(f"[decode] {what}: B={case.batch} n_q={case.n_q} n_kv={case.n_kv} d={case.head_dim} "
        f"dtype={case.dtype} ctx={case.context_lens.tolist()[:8]}")
    kp, vp, out = gpu_step(pa, case)
    okp, ovp, oout = oracle_step(case)
    assert same_bits(kp.cpu(), torch.from_numpy(okp).view(kp.dtype)), \
        f"{what}: K pool after kv_append differs from the oracle"
    assert same_bits(vp.cpu(), torch.from_numpy(ovp).view(vp.dtype)), \
        f"{what}: V pool after kv_append differs from the oracle"
    stats = assert_parity(out.cpu().numpy(), oout, case.dtype, what)
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
    return out


def test_config1_tiny_fp32(pa):
    check_full(pa, wl.make_config(1, device="cuda"), "config1")


SMALL = {
    # name: (n_q, n_kv, head_dim, context_lens, dtype)
    "gqa4_bf16_d128_ragged": (8, 2, 128, [1, 15, 16, 17, 33, 300, 1000], "bf16"),
    "gqa4_bf16_d64": (8, 2, 64, [5, 64, 130], "bf16"),
    "gqa2_f16_d128": (4, 2, 128, [7, 200, 513], "f16"),
    "gqa4_f16_d128": (8, 2, 128, [2, 19, 250, 1100], "f16"),
    "gqa8_f16_d64": (16, 2, 64, [1, 47, 600], "f16"),
    "gqa8_bf16_d64": (32, 4, 64, [16, 31, 800], "bf16"),
    "gqa16_bf16": (32, 2, 128, [5, 900], "bf16"),
    "gqa2_f32_d128": (4, 2, 128, [9, 77], "f32"),
    "gqa4_f32_d64": (8, 2, 64, [31, 1], "f32"),
    "mqa16_bf16": (16, 1, 128, [40, 700], "bf16"),
    "mqa32_bf16": (32, 1, 128, [260], "bf16"),
    "mqa64_bf16": (64, 1, 128, [100, 17], "bf16"),
    "mha_bf16": (4, 4, 128, [3, 90], "bf16"),
    "gqa8_bf16": (64, 8, 128, [1500, 2100], "bf16"),
    "gqa3_bf16": (6, 2, 128, [50, 129], "bf16"),
    "gqa6_bf16": (12, 2, 128, [333], "bf16"),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_shapes(pa, name):
    n_q, n_kv, d, ctx, dt = SMALL[name]
    case = wl.make_decode_case(batch=len(ctx), n_q=n_q, n_kv=n_kv, head_dim=d, context_lens=ctx,
                               dtype=dt, free_fraction=0.25, seed=zlib.crc32(name.encode()) % 10000,
                               device="cuda", name=name)
    check_full(pa, case, name)


def _sweep_case():
    return wl.make_decode_case(batch=4, n_q=16, n_kv=4, head_dim=128,
                               context_lens=[3000, 1, 700, 2048], dtype="bf16", free_fraction=0.1,
                               seed=5, device="cuda", name="sweep")


@pytest.mark.parametrize("tokens", [128, 256, 512, 1024, 2048, 8192, 0])
def test_partition_sweep(pa, tokens):
    prev = pa.set_decode_partition_tokens(tokens)
    try:
        check_full(pa, _sweep_case(), f"partition={tokens}")
    finally:
        pa.set_decode_partition_tokens(prev)


def test_block_relabelling_is_bitwise_invariant(pa):
    case = _sweep_case()
    _, _, base = gpu_step(pa, case)
    nb = case.num_blocks
    relabel = torch.as_tensor(np.random.default_rng(7).permutation(nb), device="cuda")
    moved = wl.DecodeCase(**{k: getattr(case, k) for k in case.__dataclass_fields__})
    moved.k_pool = torch.empty_like(case.k_pool)
    moved.v_pool = torch.empty_like(case.v_pool)
    moved.k_pool[relabel] = case.k_pool
    moved.v_pool[relabel] = case.v_pool
    moved.block_table = relabel[case.block_table.long()].to(torch.int32)
    slot = case.slot_mapping
    moved.slot_mapping = relabel[slot // 16] * 16 + slot % 16
    say("[decode] block relabelling")
    _, _, got = gpu_step(pa, moved)
    assert same_bits(got, base), "relabelling physical blocks changed output bits"


def test_run_twice_is_bitwise_identical(pa):
    case = _sweep_case()
    say("[decode] run twice")
    _, _, a = gpu_step(pa, case)
    _, _, b = gpu_step(pa, case)
    assert same_bits(a, b)


def test_unread_bytes_do_not_matter(pa):
    case = _sweep_case()
    say("[decode] poison independence")
    _, _, a = gpu_step(pa, case)
    # Replace every NaN (free blocks, tail slots) with zeros: the output must not change.
    z = wl.DecodeCase(**{k: getattr(case, k) for k in case.__dataclass_fields__})
    z.k_pool = torch.nan_to_num(case.k_pool, nan=0.0)
    z.v_pool = torch.nan_to_num(case.v_pool, nan=0.0)
    _, _, b = gpu_step(pa, z)
    assert torch.isfinite(a).all()
    assert same_bits(a, b)


def test_shared_prefix_equals_private_copy(pa):
    case = wl.make_decode_case(batch=6, n_q=8, n_kv=2, head_dim=128,
                               context_lens=[300, 500, 900, 400, 640, 129], dtype="bf16",
                               free_fraction=0.2, shared_prefix_blocks=8, n_sharers=3, seed=9,
                               device="cuda", name="shared")
    say(f"[decode] shared prefix: sharers {case.sharers}")
    _, _, shared = gpu_step(pa, case)
    # Give every sharer its own copy of the prefix blocks, appended to the pool.
    priv = wl.DecodeCase(**{k: getattr(case, k) for k in case.__dataclass_fields__})
    bt = case.block_table.clone()
    kp, vp = [case.k_pool], [case.v_pool]
    nb = case.num_blocks
    for b in case.sharers:
        ids = bt[b, :8].long()
        kp.append(case.k_pool[ids])
        vp.append(case.v_pool[ids])
        bt[b, :8] = torch.arange(nb, nb + 8, device="cuda", dtype=torch.int32)
        nb += 8
    priv.k_pool = torch.cat(kp)
    priv.v_pool = torch.cat(vp)
    priv.block_table = bt
    priv.num_blocks = nb
    _, _, private = gpu_step(pa, priv)
    assert same_bits(shared, private)
    okp, ovp, oout = oracle_step(case)
    assert_parity(shared.cpu().numpy(), oout, "bf16", "shared prefix vs oracle")


def test_empty_context_and_bad_metadata(pa):
    case = wl.make_decode_case(batch=4, n_q=8, n_kv=2, head_dim=128, context_lens=[0, 40, 33, 20],
                               dtype="bf16", free_fraction=0.3, seed=11, device="cuda",
                               name="meta")
    say("[decode] empty context, over-long context, out-of-pool block id")
    kp = case.k_pool.clone()
    vp = case.v_pool.clone()
    pa.kv_append(case.new_k, case.new_v, case.slot_mapping, kp, vp)
    ctx = case.context_lens.clone()
    ctx[2] = case.max_blocks_per_seq * 16 + 1        # past the block table's reach
    bt = case.block_table.clone()
    bt[3, 0] = case.num_blocks + 5                   # names a block outside the pool
    out = pa.paged_attn_decode(case.q, kp, vp, bt, ctx, case.scale)
    torch.cuda.synchronize()
    out = out.cpu()
    assert (out[0] == 0).all(), "ctx=0 must give a zero row"
    assert torch.isnan(out[2]).all(), "over-long context must give a NaN row"
    assert torch.isnan(out[3]).all(), "out-of-pool block id must give a NaN row"
    _, _, want = oracle_step(case, sel=np.asarray([[1, h] for h in range(8)], np.int32))
    assert_parity(out[1].numpy(), want, "bf16", "row next to bad metadata")


def test_out_of_range_slots_are_skipped(pa):
    case = wl.make_config(1, device="cuda")
    kp = case.k_pool.clone()
    vp = case.v_pool.clone()
    slots = torch.tensor([-1, case.num_blocks * 16], dtype=torch.int64, device="cuda")
    say("[append] padding and out-of-pool slots")
    pa.kv_append(case.new_k, case.new_v, slots, kp, vp)
    torch.cuda.synchronize()
    assert same_bits(kp, case.k_pool) and same_bits(vp, case.v_pool)


def test_bf16_output(pa):
    case = _sweep_case()
    say("[decode] bf16 output")
    _, _, out = gpu_step(pa, case, out_dtype=torch.bfloat16)
    _, _, want = oracle_step(case)
    got = out.float().cpu().numpy()
    err = np.abs(got - want)
    assert (err <= 2e-3 + 2.0**-8 * np.abs(want)).all(), float(err.max())


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_config_all_rows(pa, cfg):
    """Every (sequence, query head) row of the full-size configuration against the
    oracle, into a NaN-filled output: a row the kernels never write fails."""
    case = wl.make_config(cfg, device="cuda")
    say(f"[decode] config {cfg} full size ({case.name}), B={case.batch}, all rows")
    kp, vp, out = gpu_step(pa, case)
    # kv_append: the pool after the append equals the oracle's appended pool.
    okp = stored_np(case.k_pool).copy()
    ovp = stored_np(case.v_pool).copy()
    oracle.kv_append(stored_np(case.new_k), stored_np(case.new_v),
                     case.slot_mapping.cpu().numpy(), okp, ovp)
    assert same_bits(kp.cpu(), torch.from_numpy(okp).view(kp.dtype))
    assert same_bits(vp.cpu(), torch.from_numpy(ovp).view(vp.dtype))
    want = oracle.decode(stored_np(case.q), okp, ovp, case.dtype, case.block_table.cpu().numpy(),
                         case.context_lens.cpu().numpy(), case.scale)
    stats = assert_parity(out.cpu().numpy(), want, case.dtype,
                          f"config {cfg} ({case.batch * case.n_q} rows)")
    say(f"    rows={case.batch * case.n_q} max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


# ---- fused append + decode ------------------------------------------------------------------

def _two_call(pa, case, slots=None):
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    s = case.slot_mapping if slots is None else slots
    pa.kv_append(case.new_k, case.new_v, s, kp, vp)
    out = pa.paged_attn_decode(case.q, kp, vp, case.block_table, case.context_lens, case.scale)
    torch.cuda.synchronize()
    return kp, vp, out


def _fused(pa, case, slots=None):
    kp, vp = case.k_pool.clone(), case.v_pool.clone()
    s = case.slot_mapping if slots is None else slots
    out = nan_out((case.batch, case.n_q, case.head_dim))
    pa.paged_attn_decode_append(case.q, case.new_k, case.new_v, s, kp, vp,
                                case.block_table, case.context_lens, case.scale, out=out)
    torch.cuda.synchronize()
    return kp, vp, out


def check_fused(pa, case, what, slots=None):
    say(f"[decode+append] {what}: B={case.batch} n_q={case.n_q} n_kv={case.n_kv} "
        f"ctx={case.context_lens.tolist()[:8]}")
    ka, va, oa = _two_call(pa, case, slots)
    kb, vb, ob = _fused(pa, case, slots)
    assert same_bits(ka, kb) and same_bits(va, vb), f"{what}: pools differ from kv_append"
    assert same_bits(oa, ob), f"{what}: fused output differs from kv_append + decode"
    return ob


FUSED = {
    "gqa4_bf16_d128_ragged": (8, 2, 128, [1, 15, 16, 17, 33, 300, 1000], "bf16"),
    "gqa4_f32_d64": (8, 2, 64, [31, 1, 2], "f32"),
    "gqa2_f32_d128": (4, 2, 128, [9, 77], "f32"),
    "bf16_d64": (8, 2, 64, [5, 64, 130], "bf16"),
    "mqa64_bf16": (64, 1, 128, [100, 17], "bf16"),
    "gqa8_bf16": (64, 8, 128, [1500, 2100], "bf16"),
}


@pytest.mark.parametrize("name", sorted(FUSED))
def test_fused_equals_two_calls(pa, name):
    n_q, n_kv, d, ctx, dt = FUSED[name]
    case = wl.make_decode_case(batch=len(ctx), n_q=n_q, n_kv=n_kv, head_dim=d, context_lens=ctx,
                               dtype=dt, free_fraction=0.25, seed=zlib.crc32(name.encode()) % 9999,
                               device="cuda", name=name)
    out = check_fused(pa, case, name)
    _, _, want = oracle_step(case)
    assert_parity(out.cpu().numpy(), want, dt, f"fused {name} vs oracle")


@pytest.mark.parametrize("tokens", [128, 512, 0])
def test_fused_with_split_contexts(pa, tokens):
    prev = pa.set_decode_partition_tokens(tokens)
    try:
        check_fused(pa, _sweep_case(), f"partition={tokens}")
    finally:
        pa.set_decode_partition_tokens(prev)


def test_fused_config1_and_shared_prefix(pa):
    check_fused(pa, wl.make_config(1, device="cuda"), "config1")
    case = wl.make_decode_case(batch=6, n_q=8, n_kv=2, head_dim=128,
                               context_lens=[300, 500, 900, 400, 640, 129], dtype="bf16",
                               free_fraction=0.2, shared_prefix_blocks=8, n_sharers=3, seed=9,
                               device="cuda", name="shared")
    check_fused(pa, case, "shared prefix")


def test_fused_padding_and_empty_context(pa):
    case = wl.make_decode_case(batch=4, n_q=8, n_kv=2, head_dim=128, context_lens=[0, 40, 33, 20],
                               dtype="bf16", free_fraction=0.3, seed=12, device="cuda",
                               name="pad")
    # Put the real new tokens in the cache first, then mark sequence 2 as padding: both
    # paths must read the cached row at its last position and write nothing for it.
    pa.kv_append(case.new_k, case.new_v, case.slot_mapping, case.k_pool, case.v_pool)
    slots = case.slot_mapping.clone()
    slots[2] = -1
    out = check_fused(pa, case, "padding + empty context", slots=slots)
    assert (out[0].cpu() == 0).all()
    assert torch.isfinite(out[1:]).all()


def test_fused_full_size_config2(pa):
    case = wl.make_config(2, device="cuda")
    out = check_fused(pa, case, "config 2 full size")
    _, _, want = oracle_step(case)
    assert_parity(out.cpu().numpy(), want, "bf16", "fused config 2, all rows")
