"""GPU parity of the quantised KV cache (FP8 E4M3 / INT8 codes + one fp32 scale per row).

kv_append_quant must give the oracle's codes and scales bit for bit (every step of
the per-row quantiser is a correctly rounded fp32 operation). decode_quant over
seeded code/scale pools must match the fp64 oracle, which attends over
code * scale values, within max-abs 2e-3 and norm-wise relative 1e-2. Unused
slots hold the FP8 NaN code (INT8: -128) and NaN scales and may not change any
output bit; relabelling physical blocks may not either.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, nan_out, same_bits, say, stored_np
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_gqa_attention_attn_amd as pa
    pa._lib.load()  # raises if the HIP library is missing: no fallback
    return pa


def _np(t):
    return t.detach().cpu().contiguous().numpy()


def _oracle_decode(c, k_pool=None, v_pool=None, k_scale=None, v_scale=None, window=0, sel=None):
    return oracle.decode(stored_np(c.q), _np(c.k_pool if k_pool is None else k_pool),
                         _np(c.v_pool if v_pool is None else v_pool), c.fmt,
                         _np(c.block_table), _np(c.context_lens), c.scale, sel=sel, window=window,
                         q_dtype=c.q_dtype, k_scale=_np(c.k_scale if k_scale is None else k_scale),
                         v_scale=_np(c.v_scale if v_scale is None else v_scale))


def _gpu_decode(pa, c, window=0, **kw):
    out = pa.paged_attn_decode_quant(c.q, kw.get("k_pool", c.k_pool), kw.get("v_pool", c.v_pool),
                                     kw.get("k_scale", c.k_scale), kw.get("v_scale", c.v_scale), c.fmt,
                                     kw.get("block_table", c.block_table), c.context_lens, c.scale,
                                     window=window, out_dtype=kw.get("out_dtype", torch.float32),
                                     out=kw.get("out"))
    torch.cuda.synchronize()
    return out


# ---- kv_append_quant --------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("src", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [128, 64])
def test_append_quant_bit_exact(pa, fmt, src, d):
    T, n_kv, nb = 300, 2, 40
    g = torch.Generator(device="cuda").manual_seed(zlib.crc32(f"{fmt}{src}{d}".encode()))
    dt = wl.TORCH_DTYPES[src]
    k = (torch.randn((T, n_kv, d), generator=g, device="cuda") * 2.0).to(dt)
    v = (torch.randn((T, n_kv, d), generator=g, device="cuda") * 0.01).to(dt)
    k[3] = 0                      # an all-zero row: scale 0, codes 0
    v[5, 1] = 0 if src == "f16" else 1e-38  # a row whose scale falls below the smallest normal
    k[7, 0, :] = 448.0            # a row at the format's edge
    slots = torch.as_tensor(np.random.default_rng(1).permutation(nb * 16)[:T], device="cuda")
    slots[10] = -1                # padding
    slots[11] = nb * 16 + 3       # past the pool: skipped
    code_dt = wl.QUANT_CODE_DTYPES[fmt]
    kc = torch.full((nb, n_kv, 16, d), 0x55, dtype=torch.uint8, device="cuda").view(code_dt)
    vc = kc.clone()
    ks = torch.full((nb, n_kv, 16), -7.0, dtype=torch.float32, device="cuda")
    vs = ks.clone()
    okc, ovc, oks, ovs = _np(kc).copy(), _np(vc).copy(), _np(ks).copy(), _np(vs).copy()
    say(f"[quant append] {fmt} from {src}, d={d}, T={T}")
    pa.kv_append_quant(k, v, slots, kc, vc, ks, vs, fmt)
    torch.cuda.synchronize()
    oslots = _np(slots).copy()
    oslots[11] = -1               # the oracle rejects out-of-pool slots; the kernel skips them
    oracle.kv_append_quant(stored_np(k), stored_np(v), src, oslots, okc, ovc, oks, ovs, fmt)
    assert np.array_equal(_np(kc), okc), "K codes differ from the oracle"
    assert np.array_equal(_np(vc), ovc), "V codes differ from the oracle"
    assert np.array_equal(_np(ks).view(np.uint32), oks.view(np.uint32)), "K scales differ"
    assert np.array_equal(_np(vs).view(np.uint32), ovs.view(np.uint32)), "V scales differ"


# ---- decode over a quantised cache --------------------------------------------------------

SHAPES = {
    # name: (n_q, n_kv, head_dim, context lengths, q dtype)
    "gqa4_d128": (8, 2, 128, [1, 15, 16, 17, 33, 300, 1000], "bf16"),
    "gqa4_d64_f16": (8, 2, 64, [5, 64, 130], "f16"),
    "gqa8_d128": (16, 2, 128, [2, 700, 2100], "bf16"),
    "mha_d128": (4, 4, 128, [3, 90], "bf16"),
    "gqa2_f16": (4, 2, 128, [7, 513], "f16"),
    "mqa16_d128": (16, 1, 128, [40, 400], "bf16"),
    "mqa32_d64": (32, 1, 64, [260], "bf16"),
}


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("name", sorted(SHAPES))
def test_decode_quant_matches_oracle(pa, fmt, name):
    n_q, n_kv, d, ctx, qdt = SHAPES[name]
    c = wl.make_quant_decode_case(fmt=fmt, q_dtype=qdt, batch=len(ctx), n_q=n_q, n_kv=n_kv,
                                  head_dim=d, context_lens=ctx, free_fraction=0.25,
                                  seed=zlib.crc32(f"{fmt}{name}".encode()) % 9973, device="cuda",
                                  name=name)
    say(f"[quant decode] {fmt} {name}: ctx={ctx}")
    got = _gpu_decode(pa, c)
    want = _oracle_decode(c)
    stats = assert_parity(got.cpu().numpy(), want, qdt, f"{fmt} {name}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


def _sweep_case(fmt):
    return wl.make_quant_decode_case(fmt=fmt, batch=4, n_q=16, n_kv=4, head_dim=128,
                                     context_lens=[3000, 1, 700, 2048], free_fraction=0.1,
                                     seed=5, device="cuda", name="sweep")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("tokens", [256, 1024, 0])
def test_decode_quant_partitions(pa, fmt, tokens):
    c = _sweep_case(fmt)
    prev = pa.set_decode_partition_tokens(tokens)
    try:
        say(f"[quant decode] {fmt} partition={tokens}")
        got = _gpu_decode(pa, c)
    finally:
        pa.set_decode_partition_tokens(prev)
    assert_parity(got.cpu().numpy(), _oracle_decode(c), "bf16", f"{fmt} partition={tokens}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("window", [1, 100, 2000])
def test_decode_quant_window(pa, fmt, window):
    c = _sweep_case(fmt)
    say(f"[quant decode] {fmt} window={window}")
    got = _gpu_decode(pa, c, window=window)
    assert_parity(got.cpu().numpy(), _oracle_decode(c, window=window), "bf16", f"{fmt} W={window}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_decode_quant_unused_slots_and_relabelling(pa, fmt):
    c = _sweep_case(fmt)
    say(f"[quant decode] {fmt}: poison independence, relabelling, run twice")
    base = _gpu_decode(pa, c)
    assert torch.isfinite(base).all()
    assert same_bits(base, _gpu_decode(pa, c)), "two runs differ"
    # Unused slots: replace the poison (NaN codes / -128, NaN scales) with zeros.
    nan_k = torch.isnan(c.k_scale)
    zk, zv = c.k_pool.clone(), c.v_pool.clone()
    zk[nan_k] = 0
    zv[torch.isnan(c.v_scale)] = 0
    zks = torch.nan_to_num(c.k_scale, nan=0.0)
    zvs = torch.nan_to_num(c.v_scale, nan=0.0)
    assert same_bits(base, _gpu_decode(pa, c, k_pool=zk, v_pool=zv, k_scale=zks, v_scale=zvs))
    # Physical relabelling.
    relabel = torch.as_tensor(np.random.default_rng(7).permutation(c.num_blocks), device="cuda")
    moved = {}
    for key in ("k_pool", "v_pool", "k_scale", "v_scale"):
        t = getattr(c, key)
        m = torch.empty_like(t)
        m[relabel] = t
        moved[key] = m
    moved["block_table"] = relabel[c.block_table.long()].to(torch.int32)
    assert same_bits(base, _gpu_decode(pa, c, **moved)), "relabelling changed output bits"


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_append_then_decode_end_to_end(pa, fmt):
    """The step's new token quantised into the cache by each side, then attended."""
    c = wl.make_quant_decode_case(fmt=fmt, batch=5, n_q=32, n_kv=8, head_dim=128,
                                  context_lens=[1, 16, 17, 500, 1301], free_fraction=0.2, seed=31,
                                  device="cuda", name="e2e")
    say(f"[quant] {fmt}: append + decode vs oracle append + decode")
    kc, vc, ks, vs = c.k_pool.clone(), c.v_pool.clone(), c.k_scale.clone(), c.v_scale.clone()
    pa.kv_append_quant(c.new_k, c.new_v, c.slot_mapping, kc, vc, ks, vs, fmt)
    got = _gpu_decode(pa, c, k_pool=kc, v_pool=vc, k_scale=ks, v_scale=vs)
    okc, ovc, oks, ovs = _np(c.k_pool).copy(), _np(c.v_pool).copy(), _np(c.k_scale).copy(), _np(c.v_scale).copy()
    oracle.kv_append_quant(stored_np(c.new_k), stored_np(c.new_v), c.q_dtype, _np(c.slot_mapping),
                           okc, ovc, oks, ovs, fmt)
    assert np.array_equal(_np(kc), okc) and np.array_equal(_np(vc), ovc)
    assert np.array_equal(_np(ks).view(np.uint32), oks.view(np.uint32))
    want = oracle.decode(stored_np(c.q), okc, ovc, fmt, _np(c.block_table), _np(c.context_lens), c.scale,
                         q_dtype=c.q_dtype, k_scale=oks, v_scale=ovs)
    assert_parity(got.cpu().numpy(), want, "bf16", f"{fmt} append + decode")


def test_decode_quant_bf16_output_and_rejections(pa):
    c = _sweep_case("fp8")
    out = _gpu_decode(pa, c, out_dtype=torch.bfloat16)
    want = _oracle_decode(c)
    err = np.abs(out.float().cpu().numpy() - want)
    assert (err <= 2e-3 + 2.0 ** -8 * np.abs(want)).all(), float(err.max())
    # A quantised cache is refused by the bf16/f16 entry points, and q must be bf16/f16.
    with pytest.raises(TypeError):
        pa.paged_attn_decode(c.q, c.k_pool, c.v_pool, c.block_table, c.context_lens, c.scale)
    with pytest.raises(TypeError):
        pa.paged_attn_decode_quant(c.q.float(), c.k_pool, c.v_pool, c.k_scale, c.v_scale, "fp8",
                                   c.block_table, c.context_lens, c.scale)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_full_size_8b_all_rows(pa, fmt):
    ctx = [2048] * 32
    c = wl.make_quant_decode_case(fmt=fmt, batch=32, n_q=32, n_kv=8, head_dim=128,
                                  context_lens=ctx, seed=2002, device="cuda", name=f"8b_{fmt}")
    say(f"[quant decode] 8B shape, {fmt}, full size, all rows")
    out = nan_out((32, 32, 128))
    got = _gpu_decode(pa, c, out=out)
    want = _oracle_decode(c)
    stats = assert_parity(got.cpu().numpy(), want, "bf16", f"8B {fmt}, all 1024 rows")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


# ---- fused quantising append + decode ------------------------------------------------------

FUSED_SHAPES = {
    # name: (q_dtype, batch, n_q, n_kv, head_dim, context_lens)
    "gqa4_bf16": ("bf16", 5, 32, 8, 128, [1, 16, 17, 500, 1301]),
    "gqa4_f16_d64": ("f16", 3, 8, 2, 64, [33, 64, 700]),
    "mqa_g16": ("bf16", 2, 16, 1, 128, [5, 2100]),
    "g2": ("bf16", 3, 4, 2, 128, [15, 16, 300]),
}


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("name", sorted(FUSED_SHAPES))
@pytest.mark.parametrize("variant", ["plain", "split", "window", "padding"])
def test_fused_quant_step_equals_two_calls(pa, fmt, name, variant):
    """decode_quant_append gives the codes, scales and outputs of kv_append_quant
    followed by decode_quant, bit for bit."""
    qd, B, n_q, n_kv, d, ctx = FUSED_SHAPES[name]
    c = wl.make_quant_decode_case(fmt=fmt, q_dtype=qd, batch=B, n_q=n_q, n_kv=n_kv, head_dim=d,
                                  context_lens=ctx, free_fraction=0.2,
                                  seed=zlib.crc32(f"{fmt}{name}{variant}".encode()) % 100000,
                                  device="cuda", name="fused")
    say(f"[quant fused] {fmt} {name} {variant}: B={B} n_q={n_q} n_kv={n_kv} d={d} ctx={ctx}")
    slots = c.slot_mapping.clone()
    if variant == "padding":
        slots[1] = -1
    window = 100 if variant == "window" else 0
    old = pa.set_decode_partition_tokens(256 if variant == "split" else 0)
    try:
        kc, vc, ks, vs = c.k_pool.clone(), c.v_pool.clone(), c.k_scale.clone(), c.v_scale.clone()
        pa.kv_append_quant(c.new_k, c.new_v, slots, kc, vc, ks, vs, fmt)
        two = pa.paged_attn_decode_quant(c.q, kc, vc, ks, vs, fmt, c.block_table, c.context_lens, c.scale,
                                         window=window)
        fkc, fvc, fks, fvs = c.k_pool.clone(), c.v_pool.clone(), c.k_scale.clone(), c.v_scale.clone()
        one = pa.paged_attn_decode_quant_append(c.q, c.new_k, c.new_v, slots, fkc, fvc, fks, fvs, fmt,
                                                c.block_table, c.context_lens, c.scale, window=window)
        torch.cuda.synchronize()
    finally:
        pa.set_decode_partition_tokens(old)
    assert same_bits(fkc, kc) and same_bits(fvc, vc), "codes differ"
    assert same_bits(fks, ks) and same_bits(fvs, vs), "scales differ"
    assert same_bits(one, two), "outputs differ"


def test_fused_quant_step_matches_oracle_full_size(pa):
    """The 8B decode shape over an FP8 cache as one fused step, against the oracle's
    append followed by its decode, on every row."""
    c = wl.make_quant_decode_case(fmt="fp8", batch=32, n_q=32, n_kv=8, head_dim=128,
                                  context_lens=[2048] * 32, seed=2003, device="cuda", name="8b_fp8")
    say("[quant fused] 8B shape, fp8, full size, fused step vs oracle (all rows)")
    kc, vc, ks, vs = c.k_pool.clone(), c.v_pool.clone(), c.k_scale.clone(), c.v_scale.clone()
    got = nan_out((32, 32, 128))
    pa.paged_attn_decode_quant_append(c.q, c.new_k, c.new_v, c.slot_mapping, kc, vc, ks, vs, "fp8",
                                      c.block_table, c.context_lens, c.scale, out=got)
    torch.cuda.synchronize()
    okc, ovc, oks, ovs = _np(c.k_pool).copy(), _np(c.v_pool).copy(), _np(c.k_scale).copy(), _np(c.v_scale).copy()
    oracle.kv_append_quant(stored_np(c.new_k), stored_np(c.new_v), c.q_dtype, _np(c.slot_mapping),
                           okc, ovc, oks, ovs, "fp8")
    assert np.array_equal(_np(kc), okc) and np.array_equal(_np(vc), ovc)
    assert np.array_equal(_np(ks).view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(_np(vs).view(np.uint32), ovs.view(np.uint32))
    want = oracle.decode(stored_np(c.q), okc, ovc, "fp8", _np(c.block_table), _np(c.context_lens), c.scale,
                         q_dtype=c.q_dtype, k_scale=oks, v_scale=ovs)
    stats = assert_parity(got.cpu().numpy(), want, "bf16", "fused fp8 step, all 1024 rows")
    say(f"    max_abs={stats['max_abs']:.2e}")


# ---- several rows per sequence over the quantised cache -----------------------------------

def _rows_case(fmt, q_dtype, B, R, ctx, n_q, n_kv, d, seed, free=0.2):
    c = wl.make_quant_decode_case(fmt=fmt, q_dtype=q_dtype, batch=B, n_q=n_q, n_kv=n_kv, head_dim=d,
                                  context_lens=ctx, free_fraction=free, seed=seed, device="cuda", name="rows")
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    q = torch.randn(B, R, n_q, d, generator=g, device="cuda").to(wl.TORCH_DTYPES[q_dtype])
    return c, q


def _oracle_rows(c, q, window=0, alibi=None, ctx=None, bt=None):
    return oracle.chunked_prefill(stored_np(q), _np(c.k_pool), _np(c.v_pool), c.fmt,
                                  _np(c.block_table if bt is None else bt),
                                  _np(c.context_lens if ctx is None else ctx), c.scale, window=window,
                                  alibi=alibi, q_dtype=c.q_dtype, k_scale=_np(c.k_scale), v_scale=_np(c.v_scale))


ROWS = [
    # (fmt, q dtype, batch, rows, context lengths, n_q, n_kv, head_dim)
    ("fp8", "bf16", 2, 4, [40, 700], 8, 2, 128),
    ("int8", "bf16", 3, 2, [2, 100, 2000], 16, 2, 128),
    ("fp8", "f16", 2, 5, [33, 64], 4, 4, 64),
    ("int8", "f16", 1, 8, [1500], 32, 8, 128),
    ("fp8", "bf16", 2, 3, [300, 901], 6, 2, 128),     # 9 pairs per KV head: one column per slice
    ("int8", "bf16", 2, 7, [7, 50], 8, 1, 64),         # a context shorter than the rows
]


@pytest.mark.parametrize("case", ROWS, ids=[f"{r[0]}_{r[1]}_B{r[2]}_R{r[3]}_C{'-'.join(map(str, r[4]))}_{r[5]}x{r[6]}_d{r[7]}"
                                            for r in ROWS])
def test_decode_multi_quant_matches_oracle(pa, case):
    fmt, qd, B, R, ctx, n_q, n_kv, d = case
    c, q = _rows_case(fmt, qd, B, R, ctx, n_q, n_kv, d, seed=zlib.crc32(repr(case).encode()) % 10007)
    say(f"[quant rows] multi-row decode {case}")
    out = nan_out(q.shape)
    pa.paged_attn_decode_multi_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, fmt, c.block_table,
                                     c.context_lens, c.scale, out=out)
    torch.cuda.synchronize()
    want = _oracle_rows(c, q)
    stats = assert_parity(out.cpu().numpy(), want, "bf16", f"{fmt} multi-row decode")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


CHUNKS = [
    # (fmt, q dtype, batch, chunk, context lengths, n_q, n_kv, head_dim, window, alibi)
    ("fp8", "bf16", 2, 100, [100, 433], 8, 2, 128, 0, False),
    ("int8", "f16", 1, 257, [300], 4, 1, 64, 0, False),
    ("fp8", "bf16", 3, 64, [64, 1000, 200], 32, 8, 128, 0, True),
    ("int8", "bf16", 2, 90, [590, 110], 8, 2, 128, 64, False),
    ("fp8", "f16", 1, 48, [2100], 12, 4, 128, 300, True),
]


@pytest.mark.parametrize("case", CHUNKS, ids=[f"{r[0]}_{r[1]}_B{r[2]}_C{r[3]}_ctx{'-'.join(map(str, r[4]))}_{r[5]}x{r[6]}"
                                              f"_d{r[7]}_W{r[8]}{'_alibi' if r[9] else ''}" for r in CHUNKS])
def test_chunked_prefill_quant_matches_oracle(pa, case):
    fmt, qd, B, C, ctx, n_q, n_kv, d, window, alibi = case
    c, q = _rows_case(fmt, qd, B, C, ctx, n_q, n_kv, d, seed=zlib.crc32(repr(case).encode()) % 10007)
    m = (2.0 ** (-8.0 * (np.arange(n_q) + 1) / n_q)).astype(np.float32) if alibi else None
    say(f"[quant rows] chunked prefill {case}")
    out = nan_out(q.shape)
    pa.paged_attn_chunked_prefill_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, fmt, c.block_table,
                                        c.context_lens, c.scale, out=out, window=window,
                                        alibi_slopes=None if m is None else torch.as_tensor(m, device="cuda"))
    torch.cuda.synchronize()
    want = _oracle_rows(c, q, window=window, alibi=m)
    stats = assert_parity(out.cpu().numpy(), want, "bf16", f"{fmt} chunked prefill")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


@pytest.mark.parametrize("tokens", [256, 1024])
def test_rows_quant_split_contexts_match_oracle(pa, tokens):
    """Contexts split into partitions (log-sum-exp merge of per-partition partials)."""
    c, q = _rows_case("fp8", "bf16", 2, 6, [2500, 900], 8, 2, 128, seed=tokens)
    prev = pa.set_decode_partition_tokens(tokens)
    try:
        say(f"[quant rows] multi-row decode with {tokens}-token partitions")
        out = pa.paged_attn_decode_multi_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, "fp8",
                                               c.block_table, c.context_lens, c.scale)
        win = pa.paged_attn_decode_multi_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, "fp8",
                                               c.block_table, c.context_lens, c.scale, window=700)
        torch.cuda.synchronize()
    finally:
        pa.set_decode_partition_tokens(prev)
    assert_parity(out.cpu().numpy(), _oracle_rows(c, q), "bf16", "split multi-row decode")
    assert_parity(win.cpu().numpy(), _oracle_rows(c, q, window=700), "bf16", "split windowed multi-row decode")


def test_rows_quant_relabelling_and_repeat_are_bitwise(pa):
    c, q = _rows_case("int8", "bf16", 2, 4, [1200, 77], 16, 4, 128, seed=5)
    say("[quant rows] relabelled blocks and a repeated call, bitwise")
    a = pa.paged_attn_chunked_prefill_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, "int8", c.block_table,
                                            c.context_lens, c.scale)
    again = pa.paged_attn_chunked_prefill_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, "int8",
                                                c.block_table, c.context_lens, c.scale)
    multi = pa.paged_attn_decode_multi_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, "int8", c.block_table,
                                             c.context_lens, c.scale)
    perm = torch.as_tensor(np.random.default_rng(9).permutation(c.num_blocks), device="cuda")
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(c.num_blocks, device="cuda")
    b = pa.paged_attn_chunked_prefill_quant(q, c.k_pool[inv].contiguous(), c.v_pool[inv].contiguous(),
                                            c.k_scale[inv].contiguous(), c.v_scale[inv].contiguous(), "int8",
                                            perm[c.block_table.long()].int(), c.context_lens, c.scale)
    torch.cuda.synchronize()
    assert same_bits(a, again) and same_bits(a, multi) and same_bits(a, b)


def test_rows_quant_bad_metadata_and_bf16_output(pa):
    c, q = _rows_case("fp8", "bf16", 4, 5, [60, 60, 60, 3], 8, 2, 128, seed=11, free=0.3)
    say("[quant rows] over-long context, out-of-pool block, context shorter than the rows; bf16 out")
    ctx = c.context_lens.clone()
    ctx[0] = c.block_table.shape[1] * 16 + 1
    bt = c.block_table.clone()
    bt[1, 2] = c.num_blocks + 5
    out = nan_out(q.shape)
    pa.paged_attn_decode_multi_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, "fp8", bt, ctx, c.scale, out=out)
    o16 = pa.paged_attn_decode_multi_quant(q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, "fp8", c.block_table,
                                           c.context_lens, c.scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    out = out.cpu()
    assert torch.isnan(out[0]).all() and torch.isnan(out[1]).all()
    assert (out[3, :2] == 0).all(), "rows at negative positions must be zero"
    want = _oracle_rows(c, q)
    assert_parity(out[2:].numpy(), want[2:], "bf16", "sequences next to bad metadata")
    # bf16 output: the fp32 result's rounding (half an ulp, 2^-9 relative) on top of the tolerance.
    got16 = o16.float().cpu().numpy()
    assert (np.abs(got16 - want) <= 2e-3 + 2.0 ** -8 * np.abs(want)).all(), "bf16 output"


# ---- per-channel scales ------------------------------------------------------------------
#
# The same codes with one fixed fp32 scale per (KV head, channel), given by the caller. The
# append must give the oracle's codes bit for bit (saturating past QMAX * scale, code 0 for a
# scale below the smallest normal float); the attention calls meet the oracle over
# code * channel scale.

def _chan_scales(seed, n_kv, d, fmt, device="cuda"):
    g = torch.Generator(device=device).manual_seed(seed)
    qmax = wl.QUANT_QMAX[fmt]
    k = (3.0 / qmax) * (0.5 + torch.rand((n_kv, d), generator=g, device=device))
    v = (3.0 / qmax) * (0.5 + torch.rand((n_kv, d), generator=g, device=device))
    return k.float().contiguous(), v.float().contiguous()


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("src", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [128, 64])
def test_append_quant_per_channel_bit_exact(pa, fmt, src, d):
    T, n_kv, nb = 300, 2, 40
    g = torch.Generator(device="cuda").manual_seed(zlib.crc32(f"chan{fmt}{src}{d}".encode()))
    dt = wl.TORCH_DTYPES[src]
    k = (torch.randn((T, n_kv, d), generator=g, device="cuda") * 2.0).to(dt)   # many past 3 * scale: saturate
    v = (torch.randn((T, n_kv, d), generator=g, device="cuda") * 0.5).to(dt)
    ks, vs = _chan_scales(7, n_kv, d, fmt)
    ks[0, 3] = 0.0                 # a channel with scale 0: codes 0
    vs[1, 5] = 1e-39               # a subnormal scale: codes 0
    slots = torch.as_tensor(np.random.default_rng(2).permutation(nb * 16)[:T], device="cuda")
    slots[10] = -1
    slots[11] = nb * 16 + 3
    code_dt = wl.QUANT_CODE_DTYPES[fmt]
    kc = torch.full((nb, n_kv, 16, d), 0x55, dtype=torch.uint8, device="cuda").view(code_dt)
    vc = kc.clone()
    okc, ovc = _np(kc).copy(), _np(vc).copy()
    ks0, vs0 = ks.clone(), vs.clone()
    say(f"[quant append] per-channel {fmt} from {src}, d={d}, T={T}")
    pa.kv_append_quant(k, v, slots, kc, vc, ks, vs, f"{fmt}_per_channel")
    torch.cuda.synchronize()
    oslots = _np(slots).copy()
    oslots[11] = -1
    oracle.kv_append_quant_channel(stored_np(k), stored_np(v), src, oslots, okc, ovc, _np(ks), _np(vs), fmt)
    assert np.array_equal(_np(kc), okc), "K codes differ from the oracle"
    assert np.array_equal(_np(vc), ovc), "V codes differ from the oracle"
    assert same_bits(ks, ks0) and same_bits(vs, vs0), "the channel scales must only be read"
    qmax = wl.QUANT_QMAX[fmt]
    cv = okc.view(np.uint8) if fmt == "fp8" else okc
    assert (np.abs(oracle.upcast(cv, fmt)) == qmax).sum() > 100, "the case must saturate some values"


def _chan_case(fmt, q_dtype, ctx, n_q, n_kv, d, seed, free=0.25):
    c = wl.make_quant_decode_case(fmt=fmt, q_dtype=q_dtype, batch=len(ctx), n_q=n_q, n_kv=n_kv, head_dim=d,
                                  context_lens=ctx, free_fraction=free, seed=seed, device="cuda", name="chan")
    ks, vs = _chan_scales(seed + 3, n_kv, d, fmt)
    return c, ks, vs


def _oracle_chan(c, ks, vs, q=None, rows=False, **kw):
    args = (stored_np(c.q if q is None else q), _np(c.k_pool), _np(c.v_pool), c.fmt, _np(c.block_table),
            _np(c.context_lens), c.scale)
    kw.update(q_dtype=c.q_dtype, k_scale=_np(ks), v_scale=_np(vs), scale_mode="channel")
    return oracle.chunked_prefill(*args, **kw) if rows else oracle.decode(*args, **kw)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("name", ["gqa4_d128", "gqa4_d64_f16", "gqa8_d128", "mha_d128", "gqa2_f16", "mqa32_d64"])
def test_decode_quant_per_channel_matches_oracle(pa, fmt, name):
    n_q, n_kv, d, ctx, qdt = SHAPES[name]
    c, ks, vs = _chan_case(fmt, qdt, ctx, n_q, n_kv, d, seed=zlib.crc32(f"chan{fmt}{name}".encode()) % 9973)
    say(f"[quant decode] per-channel {fmt} {name}: ctx={ctx}")
    out = nan_out((c.batch, n_q, d))
    pa.paged_attn_decode_quant(c.q, c.k_pool, c.v_pool, ks, vs, f"{fmt}_per_channel", c.block_table,
                               c.context_lens, c.scale, out=out)
    torch.cuda.synchronize()
    stats = assert_parity(out.cpu().numpy(), _oracle_chan(c, ks, vs), qdt, f"per-channel {fmt} {name}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_decode_quant_per_channel_split_window_alibi(pa, fmt):
    c, ks, vs = _chan_case(fmt, "bf16", [3000, 1, 700, 2048], 16, 4, 128, seed=17)
    m = (2.0 ** (-8.0 * (np.arange(16) + 1) / 16)).astype(np.float32)
    prev = pa.set_decode_partition_tokens(256)
    try:
        say(f"[quant decode] per-channel {fmt}: 256-token partitions, window 900, ALiBi")
        a = pa.paged_attn_decode_quant(c.q, c.k_pool, c.v_pool, ks, vs, f"{fmt}_per_channel", c.block_table,
                                       c.context_lens, c.scale)
        w = pa.paged_attn_decode_quant(c.q, c.k_pool, c.v_pool, ks, vs, f"{fmt}_per_channel", c.block_table,
                                       c.context_lens, c.scale, window=900,
                                       alibi_slopes=torch.as_tensor(m, device="cuda"))
        torch.cuda.synchronize()
    finally:
        pa.set_decode_partition_tokens(prev)
    assert_parity(a.cpu().numpy(), _oracle_chan(c, ks, vs), "bf16", "split per-channel decode")
    assert_parity(w.cpu().numpy(), _oracle_chan(c, ks, vs, window=900, alibi=m), "bf16",
                  "split windowed ALiBi per-channel decode")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_decode_quant_append_per_channel_equals_two_calls(pa, fmt):
    c, ks, vs = _chan_case(fmt, "bf16", [17, 300, 1], 8, 2, 128, seed=23)
    say(f"[quant decode] per-channel {fmt}: fused append vs append + decode, bitwise")
    kc1, vc1 = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append_quant(c.new_k, c.new_v, c.slot_mapping, kc1, vc1, ks, vs, f"{fmt}_per_channel")
    two = pa.paged_attn_decode_quant(c.q, kc1, vc1, ks, vs, f"{fmt}_per_channel", c.block_table, c.context_lens,
                                     c.scale)
    kc2, vc2 = c.k_pool.clone(), c.v_pool.clone()
    one = pa.paged_attn_decode_quant_append(c.q, c.new_k, c.new_v, c.slot_mapping, kc2, vc2, ks, vs,
                                            f"{fmt}_per_channel", c.block_table, c.context_lens, c.scale)
    torch.cuda.synchronize()
    assert same_bits(kc1, kc2) and same_bits(vc1, vc2), "the fused append wrote other codes"
    assert same_bits(one, two), "the fused step differs from append + decode"
    okc, ovc = _np(c.k_pool).copy(), _np(c.v_pool).copy()   # the oracle's own append
    oracle.kv_append_quant_channel(stored_np(c.new_k), stored_np(c.new_v), c.q_dtype, _np(c.slot_mapping),
                                   okc, ovc, _np(ks), _np(vs), fmt)
    want = oracle.decode(stored_np(c.q), okc, ovc, fmt, _np(c.block_table), _np(c.context_lens),
                         c.scale, q_dtype="bf16", k_scale=_np(ks), v_scale=_np(vs), scale_mode="channel")
    assert_parity(one.cpu().numpy(), want, "bf16", "fused per-channel step")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_rows_quant_per_channel_matches_oracle(pa, fmt):
    c, ks, vs = _chan_case(fmt, "f16", [100, 433, 40], 8, 2, 128, seed=29)
    g = torch.Generator(device="cuda").manual_seed(29)
    q = torch.randn(3, 37, 8, 128, generator=g, device="cuda").half()
    say(f"[quant rows] per-channel {fmt}: chunked prefill of 37 rows and multi-row decode of 4")
    out = pa.paged_attn_chunked_prefill_quant(q, c.k_pool, c.v_pool, ks, vs, f"{fmt}_per_channel", c.block_table,
                                              c.context_lens, c.scale, window=120)
    q4 = q[:, -4:].contiguous()
    out4 = pa.paged_attn_decode_multi_quant(q4, c.k_pool, c.v_pool, ks, vs, f"{fmt}_per_channel", c.block_table,
                                            c.context_lens, c.scale)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), _oracle_chan(c, ks, vs, q=q, rows=True, window=120), "f16",
                  "per-channel chunked prefill")
    assert_parity(out4.cpu().numpy(), _oracle_chan(c, ks, vs, q=q4, rows=True), "f16", "per-channel multi-row")


def test_decode_quant_per_channel_relabelling_is_bitwise(pa):
    c, ks, vs = _chan_case("fp8", "bf16", [1200, 77], 16, 4, 128, seed=31)
    say("[quant decode] per-channel fp8 under a relabelling of physical blocks")
    a = pa.paged_attn_decode_quant(c.q, c.k_pool, c.v_pool, ks, vs, "fp8_per_channel", c.block_table,
                                   c.context_lens, c.scale)
    perm = torch.as_tensor(np.random.default_rng(4).permutation(c.num_blocks), device="cuda")
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(c.num_blocks, device="cuda")
    b = pa.paged_attn_decode_quant(c.q, c.k_pool[inv].contiguous(), c.v_pool[inv].contiguous(), ks, vs,
                                   "fp8_per_channel", perm[c.block_table.long()].int(), c.context_lens, c.scale)
    torch.cuda.synchronize()
    assert same_bits(a, b)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_decode_quant_per_head_scales_meet_the_fp32_cache(pa, fmt):
    """One scale per KV head (or per tensor) is the per-channel format with each head's row
    constant. With power-of-two head scales every code * scale is exact in fp32, so the call
    must meet the oracle's plain fp32-cache decode of those dequantized values."""
    c, _, _ = _chan_case(fmt, "bf16", [1500, 37, 800, 1], 16, 4, 128, seed=41)
    kexp = np.array([-7, -6, -8, -5], dtype=np.float64)
    vexp = np.array([-6, -9, -7, -7], dtype=np.float64)
    ks = torch.as_tensor(np.repeat((2.0 ** kexp)[:, None], 128, axis=1), dtype=torch.float32, device="cuda")
    vs = torch.as_tensor(np.repeat((2.0 ** vexp)[:, None], 128, axis=1), dtype=torch.float32, device="cuda")
    say(f"[quant decode] per-head {fmt} scales as constant per-channel rows")
    out = nan_out((c.batch, 16, 128))
    pa.paged_attn_decode_quant(c.q, c.k_pool, c.v_pool, ks, vs, f"{fmt}_per_channel", c.block_table,
                               c.context_lens, c.scale, out=out)
    torch.cuda.synchronize()

    def dequant(pool, exps):
        codes = _np(pool)
        codes = codes.view(np.uint8) if fmt == "fp8" else codes
        return (oracle.upcast(codes, fmt) * (2.0 ** exps)[None, :, None, None]).astype(np.float32)

    q32 = c.q.float().cpu().numpy()   # bf16 values, exact in fp32
    want = oracle.decode(q32, dequant(c.k_pool, kexp), dequant(c.v_pool, vexp), "f32", _np(c.block_table),
                         _np(c.context_lens), c.scale)
    stats = assert_parity(out.cpu().numpy(), want, "bf16", f"per-head {fmt}")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_full_size_8b_per_channel_all_rows(pa, fmt):
    c, ks, vs = _chan_case(fmt, "bf16", [2048] * 32, 32, 8, 128, seed=2012)
    say(f"[quant decode] 8B shape, per-channel {fmt}, full size, all rows")
    out = nan_out((32, 32, 128))
    pa.paged_attn_decode_quant(c.q, c.k_pool, c.v_pool, ks, vs, f"{fmt}_per_channel", c.block_table,
                               c.context_lens, c.scale, out=out)
    torch.cuda.synchronize()
    stats = assert_parity(out.cpu().numpy(), _oracle_chan(c, ks, vs), "bf16", f"8B per-channel {fmt}, all rows")
    say(f"    max_abs={stats['max_abs']:.2e} rel={stats['rel']:.2e}")
