"""GPU parity of the ALiBi score bias, in every kernel, against the fp64 oracle.

With slopes m_h (float32 [n_q]) the score of query head h at position i for the
key at position j gets -m_h (i - j) added after the scale ("LLM 推理全过程的维度变化
与核心公式", position-encoding section). Decode (both kernels), split + reduce,
fused decode + append, multi-row decode (both kernels), chunked prefill,
contiguous prefill (with and without the f16 V staging) and decode over FP8 and
INT8 caches are each compared with the oracle's biased definition on the same
seeded inputs: max-abs 2e-3 and norm-wise relative 1e-2 for bf16/f16, 1e-5 for
fp32. The slopes are the geometric family of the ALiBi paper, plus a set of
mixed-sign random slopes and one of very steep slopes (each query sees almost
only its own key).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, nan_out, oracle_pools, same_bits, say, stored_np
from oracle_pins import alibi_slopes
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_gqa_attention_attn_amd as pa
    pa._lib.load()  # raises if the HIP library is missing: no fallback
    return pa


@pytest.fixture(params=["default", "valu"])
def decode_kernel(request, option):
    """Decode runs with the default kernel choice (matrix cores where the group allows)
    and with the VALU kernels forced."""
    option("decode_matrix_cores", 0 if request.param == "valu" else 1)
    return request.param


def _slopes(kind: str, n_q: int) -> np.ndarray:
    if kind == "geometric":
        return alibi_slopes(n_q)
    if kind == "mixed":      # any real slope is allowed, including negative ones
        return np.random.default_rng(n_q).uniform(-0.05, 0.3, n_q).astype(np.float32)
    if kind == "steep":      # softmax concentrates on the newest keys
        return np.full(n_q, 6.0, np.float32)
    raise ValueError(kind)


def _dev(slopes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(slopes).to("cuda")


def _np(t):
    return t.detach().cpu().contiguous().numpy()


# ---- single-row decode --------------------------------------------------------------------

DECODE = {
    # name: (n_q, n_kv, head_dim, context lengths, dtype)
    "gqa4_bf16_d128": (32, 8, 128, [1, 15, 16, 17, 100, 257, 1000, 5000], "bf16"),
    "gqa4_f16_d64": (8, 2, 64, [3, 64, 130, 2100], "f16"),
    "gqa2_f32_d128": (4, 2, 128, [9, 77, 600], "f32"),
    "mqa_bf16": (16, 1, 128, [40, 700, 3000], "bf16"),
}


def _decode_case(name, seed_extra=0):
    n_q, n_kv, d, ctx, dt = DECODE[name]
    return wl.make_decode_case(batch=len(ctx), n_q=n_q, n_kv=n_kv, head_dim=d, context_lens=ctx,
                               dtype=dt, free_fraction=0.2, seed=len(name) * 17 + seed_extra,
                               device="cuda", name=name)


def _appended(pa, c):
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.new_k, c.new_v, c.slot_mapping, kp, vp)
    return kp, vp


@pytest.mark.parametrize("window", [0, 100])
@pytest.mark.parametrize("kind", ["geometric", "mixed", "steep"])
@pytest.mark.parametrize("name", sorted(DECODE))
def test_decode_alibi_matches_oracle(pa, decode_kernel, name, kind, window):
    c = _decode_case(name)
    m = _slopes(kind, c.n_q)
    say(f"[alibi] decode {name} {kind} W={window} ctx={c.context_lens.tolist()}")
    kp, vp = _appended(pa, c)
    got = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale, window=window,
                               alibi_slopes=_dev(m))
    torch.cuda.synchronize()
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), c.dtype,
                         c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                         window=window, alibi=m)
    stats = assert_parity(got.cpu().numpy(), want, c.dtype, f"decode {name} {kind} W={window}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


@pytest.mark.parametrize("tokens", [256, 1024])
def test_decode_alibi_partition_sizes(pa, decode_kernel, tokens):
    c = _decode_case("gqa4_bf16_d128", seed_extra=1)
    m = _slopes("geometric", c.n_q) / 16      # gentle slopes: distant partitions still count
    say(f"[alibi] decode partitions of {tokens} tokens")
    kp, vp = _appended(pa, c)
    prev = pa.set_decode_partition_tokens(tokens)
    try:
        got = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale,
                                   alibi_slopes=_dev(m))
        torch.cuda.synchronize()
    finally:
        pa.set_decode_partition_tokens(prev)
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), c.dtype,
                         c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                         alibi=m)
    assert_parity(got.cpu().numpy(), want, c.dtype, f"partition {tokens}")


def test_decode_append_alibi_equals_two_calls_bitwise(pa, decode_kernel):
    c = _decode_case("gqa4_bf16_d128", seed_extra=2)
    m = _dev(_slopes("geometric", c.n_q))
    say("[alibi] fused decode + append vs kv_append + decode")
    kp, vp = _appended(pa, c)
    two = pa.paged_attn_decode(c.q, kp, vp, c.block_table, c.context_lens, c.scale, window=500,
                               alibi_slopes=m)
    kf, vf = c.k_pool.clone(), c.v_pool.clone()
    one = pa.paged_attn_decode_append(c.q, c.new_k, c.new_v, c.slot_mapping, kf, vf, c.block_table,
                                      c.context_lens, c.scale, window=500, alibi_slopes=m)
    torch.cuda.synchronize()
    assert same_bits(one, two)
    assert same_bits(kf, kp) and same_bits(vf, vp)


def test_decode_alibi_full_size_all_rows(pa):
    """The 8B decode shape (32 sequences of 2048 positions, 32/8 heads) with the fused
    append and geometric slopes, against the oracle on every row."""
    c = wl.make_decode_case(batch=32, n_q=32, n_kv=8, head_dim=128, context_lens=[2048] * 32,
                            dtype="bf16", seed=4242, device="cuda", name="8b")
    m = _slopes("geometric", 32)
    say("[alibi] 8B shape, fused decode + append, all rows")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    got = nan_out((32, 32, 128))
    pa.paged_attn_decode_append(c.q, c.new_k, c.new_v, c.slot_mapping, kp, vp, c.block_table,
                                c.context_lens, c.scale, alibi_slopes=_dev(m), out=got)
    torch.cuda.synchronize()
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), "bf16", _np(c.block_table),
                         _np(c.context_lens), c.scale, alibi=m)
    stats = assert_parity(got.cpu().numpy(), want, "bf16", "8B alibi, all 1024 rows")
    say(f"    max_abs={stats['max_abs']:.2e}")


# ---- multi-row decode and chunked prefill -------------------------------------------------

MULTI = [
    # (q_rows, prefix lengths, n_q, n_kv, head_dim, dtype, window)
    (4, [100, 2047, 9000], 32, 8, 128, "bf16", 0),
    (4, [100, 2047], 32, 8, 128, "bf16", 64),
    (8, [300, 4000], 64, 8, 128, "bf16", 0),
    (2, [0, 17, 33], 8, 2, 64, "f16", 0),
    (3, [700], 4, 4, 128, "bf16", 5),
]


@pytest.mark.parametrize("shape", MULTI, ids=[f"R{s[0]}_P{'-'.join(map(str, s[1]))}_{s[2]}x{s[3]}_d{s[4]}_{s[5]}_W{s[6]}"
                                              for s in MULTI])
def test_decode_multi_alibi_matches_oracle(pa, decode_kernel, shape):
    R, pre, n_q, n_kv, d, dt, W = shape
    c = wl.make_chunk_case(batch=len(pre), chunk_len=R, prefix_lens=pre, n_q=n_q, n_kv=n_kv,
                           head_dim=d, dtype=dt, free_fraction=0.2, seed=sum(pre) + 11 * R + W,
                           device="cuda")
    m = _slopes("geometric", n_q)
    say(f"[alibi] multi-row decode R={R} prefix={pre} {n_q}x{n_kv} d={d} {dt} W={W}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    got = pa.paged_attn_decode_multi(c.q, kp, vp, c.block_table, c.context_lens, c.scale, window=W,
                                     alibi_slopes=_dev(m))
    torch.cuda.synchronize()
    want = oracle.chunked_prefill(stored_np(c.q), *oracle_pools(c), dt,
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                                  window=W, alibi=m)
    stats = assert_parity(got.cpu().numpy(), want, dt, f"multi W={W}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


CHUNKED = [
    # (chunk_len, prefix lengths, n_q, n_kv, head_dim, dtype, window)
    (300, [1000, 17], 16, 4, 128, "f16", 0),
    (64, [0, 0], 8, 2, 128, "bf16", 0),
    (130, [64, 500], 8, 2, 64, "bf16", 0),
    (200, [700], 4, 4, 128, "bf16", 128),
]


@pytest.mark.parametrize("shape", CHUNKED, ids=[f"C{s[0]}_P{'-'.join(map(str, s[1]))}_{s[2]}x{s[3]}_d{s[4]}_{s[5]}_W{s[6]}"
                                                for s in CHUNKED])
def test_chunked_prefill_alibi_matches_oracle(pa, shape):
    C, pre, n_q, n_kv, d, dt, W = shape
    c = wl.make_chunk_case(batch=len(pre), chunk_len=C, prefix_lens=pre, n_q=n_q, n_kv=n_kv,
                           head_dim=d, dtype=dt, free_fraction=0.2, seed=sum(pre) + 5 * C + W,
                           device="cuda")
    m = _slopes("geometric", n_q)
    say(f"[alibi] chunked prefill C={C} prefix={pre} {n_q}x{n_kv} d={d} {dt} W={W}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    got = pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, c.scale,
                                        window=W, alibi_slopes=_dev(m))
    torch.cuda.synchronize()
    want = oracle.chunked_prefill(stored_np(c.q), *oracle_pools(c), dt,
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), c.scale,
                                  window=W, alibi=m)
    stats = assert_parity(got.cpu().numpy(), want, dt, f"chunked W={W}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


# ---- contiguous prefill -------------------------------------------------------------------

PREFILL = {
    # name: (B, S, n_q, n_kv, d, dtype, window)
    "gqa4_bf16_ragged": (2, 200, 8, 2, 128, "bf16", 0),
    "mha_f16": (2, 97, 2, 2, 128, "f16", 0),
    "d64_bf16": (2, 150, 4, 2, 64, "bf16", 0),
    "long_bf16": (1, 1000, 4, 2, 128, "bf16", 0),
    "window_bf16": (1, 600, 8, 2, 128, "bf16", 100),
    "one_token": (1, 1, 4, 2, 128, "bf16", 0),
}


@pytest.fixture(params=["staged", "unstaged"])
def stage_v(request, option):
    """The prefill kernel with its f16 copy of V (the default) and with it switched off."""
    option("prefill_stage_v", 1 if request.param == "staged" else 0)
    return request.param


@pytest.mark.parametrize("name", sorted(PREFILL))
def test_prefill_alibi_matches_oracle(pa, stage_v, name):
    B, S, n_q, n_kv, d, dt, W = PREFILL[name]
    g = torch.Generator(device="cuda").manual_seed(zlib.crc32(name.encode()))
    t = wl.TORCH_DTYPES[dt]
    q = torch.randn(B, S, n_q, d, generator=g, device="cuda").to(t)
    k = torch.randn(B, S, n_kv, d, generator=g, device="cuda").to(t)
    v = torch.randn(B, S, n_kv, d, generator=g, device="cuda").to(t)
    m = _slopes("geometric", n_q)
    say(f"[alibi] prefill {name} ({stage_v}): B={B} S={S} {n_q}x{n_kv} d={d} {dt} W={W}")
    out = pa.paged_attn_prefill(q, k, v, True, d ** -0.5, window=W, alibi_slopes=_dev(m))
    torch.cuda.synchronize()
    want = oracle.prefill(stored_np(q), stored_np(k), stored_np(v), dt, True, d ** -0.5, window=W,
                          alibi=m)
    stats = assert_parity(out.cpu().numpy(), want, dt, f"prefill {name}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


def test_prefill_alibi_full_size_all_rows(pa):
    """Causal prefill of 2 x 4096 tokens, 32/8 heads, d=128, with geometric slopes, on
    every row."""
    case = wl.make_prefill_case(batch=2, seq_len=4096, n_q=32, n_kv=8, head_dim=128, seed=77,
                                device="cuda")
    m = _slopes("geometric", 32)
    say("[alibi] prefill 2 x 4096, all rows")
    out = nan_out(case.q.shape)
    pa.paged_attn_prefill(case.q, case.k, case.v, True, case.scale, alibi_slopes=_dev(m), out=out)
    torch.cuda.synchronize()
    want = oracle.prefill(stored_np(case.q), stored_np(case.k), stored_np(case.v), "bf16", True,
                          case.scale, alibi=m)
    stats = assert_parity(out.cpu().numpy(), want, "bf16", "prefill alibi 2x4096, all rows")
    say(f"    max_abs={stats['max_abs']:.2e}")


# ---- quantised caches ---------------------------------------------------------------------

QUANT = {
    # name: (q dtype, n_q, n_kv, head_dim, context lengths)
    "gqa4_d128": ("bf16", 8, 2, 128, [1, 16, 17, 300, 1000]),
    "gqa4_d64_f16": ("f16", 8, 2, 64, [5, 64, 130]),
    "mqa16_d128": ("bf16", 16, 1, 128, [40, 2100]),
}


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("name", sorted(QUANT))
def test_decode_quant_alibi_matches_oracle(pa, fmt, name):
    """Fused quantising append + decode with ALiBi, against the oracle's append then decode."""
    qd, n_q, n_kv, d, ctx = QUANT[name]
    c = wl.make_quant_decode_case(fmt=fmt, q_dtype=qd, batch=len(ctx), n_q=n_q, n_kv=n_kv,
                                  head_dim=d, context_lens=ctx, free_fraction=0.2,
                                  seed=zlib.crc32(f"alibi{fmt}{name}".encode()) % 9973, device="cuda",
                                  name=name)
    m = _slopes("geometric", n_q)
    say(f"[alibi] quant {fmt} {name}: ctx={ctx}")
    kc, vc, ks, vs = c.k_pool.clone(), c.v_pool.clone(), c.k_scale.clone(), c.v_scale.clone()
    got = pa.paged_attn_decode_quant_append(c.q, c.new_k, c.new_v, c.slot_mapping, kc, vc, ks, vs, fmt,
                                            c.block_table, c.context_lens, c.scale, alibi_slopes=_dev(m))
    again = pa.paged_attn_decode_quant(c.q, kc, vc, ks, vs, fmt, c.block_table, c.context_lens, c.scale,
                                       alibi_slopes=_dev(m))
    torch.cuda.synchronize()
    okc, ovc, oks, ovs = _np(c.k_pool).copy(), _np(c.v_pool).copy(), _np(c.k_scale).copy(), _np(c.v_scale).copy()
    oracle.kv_append_quant(stored_np(c.new_k), stored_np(c.new_v), c.q_dtype, _np(c.slot_mapping),
                           okc, ovc, oks, ovs, fmt)
    want = oracle.decode(stored_np(c.q), okc, ovc, fmt, _np(c.block_table), _np(c.context_lens), c.scale,
                         q_dtype=c.q_dtype, k_scale=oks, v_scale=ovs, alibi=m)
    stats = assert_parity(got.cpu().numpy(), want, qd, f"{fmt} {name} fused")
    assert same_bits(got, again), "fused and unfused decode differ"
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


def test_binding_rejects_bad_slopes(pa):
    c = _decode_case("gqa4_f16_d64")
    with pytest.raises(ValueError):
        pa.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                             alibi_slopes=torch.zeros(c.n_q + 1, device="cuda"))
    with pytest.raises(ValueError):
        pa.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale,
                             alibi_slopes=torch.zeros(c.n_q, dtype=torch.float64, device="cuda"))
