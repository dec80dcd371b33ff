"""GPU parity of every attention entry point at a zero and a negative scale.

The scale multiplies q.k ("注意力演进与推理流程" section 1.1 writes it as
1/sqrt(d)); the library takes any finite value. At scale 0 every score is
exactly 0, so an output row is the plain mean of the V rows it attends to
(plus the ALiBi bias where slopes are given); a negative scale negates q.k.
Each case is compared with the fp64 oracle, which takes the scale as given
(its scale-0 result is pinned to mean(V) by the oracle pins), within
max-abs 2e-3 and norm-wise relative 1e-2 (1e-5 for fp32). One decode case is
also checked against a mean of V computed here with numpy.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_parity, nan_out, oracle_pools, say, stored_np
from paged_gqa_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu

SCALES = [0.0, -0.3]


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_gqa_attention_attn_amd as pa
    pa._lib.load()  # raises if the HIP library is missing: no fallback
    return pa


@pytest.fixture(params=["default", "valu"])
def decode_kernel(request, option):
    option("decode_matrix_cores", 0 if request.param == "valu" else 1)
    return request.param


def _slopes(n_q):
    return (2.0 ** (-8.0 * (np.arange(n_q) + 1) / n_q)).astype(np.float32)


def _dev(a):
    return torch.as_tensor(a, device="cuda")


DECODE = {
    # name: (n_q, n_kv, d, context lengths, dtype)
    "gqa4_bf16": (8, 2, 128, [1, 17, 300, 2500], "bf16"),
    "gqa2_f16_d64": (4, 2, 64, [5, 130], "f16"),
    "gqa4_f32": (8, 2, 128, [9, 700], "f32"),
}


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("name", sorted(DECODE))
def test_decode(pa, decode_kernel, name, alibi, scale):
    n_q, n_kv, d, ctx, dt = DECODE[name]
    c = wl.make_decode_case(batch=len(ctx), n_q=n_q, n_kv=n_kv, head_dim=d, context_lens=ctx, dtype=dt,
                            free_fraction=0.2, seed=zlib.crc32(name.encode()) % 9973, device="cuda",
                            name=name)
    m = _slopes(n_q) if alibi else None
    say(f"[scale] decode {name} scale={scale} alibi={alibi} ({decode_kernel})")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    out = nan_out((c.batch, n_q, d))
    prev = pa.set_decode_partition_tokens(256)      # split contexts: the merge sees the fold too
    try:
        pa.paged_attn_decode_append(c.q, c.new_k, c.new_v, c.slot_mapping, kp, vp, c.block_table,
                                    c.context_lens, scale, out=out,
                                    alibi_slopes=None if m is None else _dev(m))
        torch.cuda.synchronize()
    finally:
        pa.set_decode_partition_tokens(prev)
    want = oracle.decode(stored_np(c.q), *oracle_pools(c), dt, c.block_table.cpu().numpy(),
                         c.context_lens.cpu().numpy(), scale, alibi=m)
    stats = assert_parity(out.cpu().numpy(), want, dt, f"decode {name} scale={scale}")
    say(f"    max_abs={stats['max_abs']:.2e}")
    if scale == 0.0 and not alibi:
        # The plain mean of each sequence's V rows, gathered here through the block table.
        vals = oracle.upcast(oracle_pools(c)[1], dt)
        bt = c.block_table.cpu().numpy()
        for b, n in enumerate(ctx):
            rows = np.stack([vals[bt[b, t // 16], :, t % 16, :] for t in range(n)])   # [n][n_kv][d]
            mean = rows.mean(axis=0)
            got = out[b].cpu().numpy().reshape(n_kv, n_q // n_kv, d)
            assert np.abs(got - mean[:, None, :]).max() <= (1e-5 if dt == "f32" else 2e-3)


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_decode_quant(pa, fmt, scale):
    c = wl.make_quant_decode_case(fmt=fmt, batch=3, n_q=8, n_kv=2, head_dim=128, context_lens=[3, 200, 900],
                                  free_fraction=0.2, seed=31, device="cuda", name="quant")
    say(f"[scale] decode over a {fmt} cache, scale={scale}")
    out = nan_out((3, 8, 128))
    pa.paged_attn_decode_quant(c.q, c.k_pool, c.v_pool, c.k_scale, c.v_scale, fmt, c.block_table,
                               c.context_lens, scale, out=out)
    torch.cuda.synchronize()
    want = oracle.decode(stored_np(c.q), c.k_pool.cpu().numpy(), c.v_pool.cpu().numpy(), fmt,
                         c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), scale,
                         q_dtype=c.q_dtype, k_scale=c.k_scale.cpu().numpy(), v_scale=c.v_scale.cpu().numpy())
    assert_parity(out.cpu().numpy(), want, "bf16", f"{fmt} scale={scale}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("rows,n_q", [(4, 8), (5, 16)])   # matrix-core decode; the multi-row kernel
def test_decode_multi(pa, rows, n_q, scale):
    c = wl.make_chunk_case(batch=2, chunk_len=rows, prefix_lens=[40, 700], n_q=n_q, n_kv=2, head_dim=128,
                           dtype="bf16", free_fraction=0.2, seed=rows * 7 + n_q, device="cuda", name="multi")
    say(f"[scale] multi-row decode rows={rows} n_q={n_q} scale={scale}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    out = nan_out(c.q.shape)
    pa.paged_attn_decode_multi(c.q, kp, vp, c.block_table, c.context_lens, scale, out=out)
    torch.cuda.synchronize()
    want = oracle.chunked_prefill(stored_np(c.q), *oracle_pools(c), "bf16",
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), scale)
    assert_parity(out.cpu().numpy(), want, "bf16", f"multi rows={rows} scale={scale}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("stage", ["1", "0"])
def test_prefill(pa, option, stage, alibi, scale):
    option("prefill_stage_v", int(stage))
    B, S, n_q, n_kv, d = 2, 200, 8, 2, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn(B, S, n_q, d, generator=g, device="cuda").bfloat16()
    k = torch.randn(B, S, n_kv, d, generator=g, device="cuda").bfloat16()
    v = torch.randn(B, S, n_kv, d, generator=g, device="cuda").bfloat16()
    m = _slopes(n_q) if alibi else None
    say(f"[scale] prefill scale={scale} alibi={alibi} staged={stage}")
    out = nan_out(q.shape)
    pa.paged_attn_prefill(q, k, v, True, scale, out=out, alibi_slopes=None if m is None else _dev(m))
    torch.cuda.synchronize()
    want = oracle.prefill(stored_np(q), stored_np(k), stored_np(v), "bf16", True, scale, alibi=m)
    assert_parity(out.cpu().numpy(), want, "bf16", f"prefill scale={scale}")
    if not alibi:
        full = nan_out(q.shape)
        pa.paged_attn_prefill(q, k, v, False, scale, out=full)
        torch.cuda.synchronize()
        want = oracle.prefill(stored_np(q), stored_np(k), stored_np(v), "bf16", False, scale)
        assert_parity(full.cpu().numpy(), want, "bf16", f"full prefill scale={scale}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("alibi", [False, True])
def test_chunked_prefill(pa, alibi, scale):
    c = wl.make_chunk_case(batch=2, chunk_len=100, prefix_lens=[0, 333], n_q=8, n_kv=2, head_dim=128,
                           dtype="bf16", free_fraction=0.2, seed=77, device="cuda", name="chunk")
    m = _slopes(8) if alibi else None
    say(f"[scale] chunked prefill scale={scale} alibi={alibi}")
    kp, vp = c.k_pool.clone(), c.v_pool.clone()
    pa.kv_append(c.chunk_k, c.chunk_v, c.chunk_slots, kp, vp)
    out = nan_out(c.q.shape)
    pa.paged_attn_chunked_prefill(c.q, kp, vp, c.block_table, c.context_lens, scale, out=out,
                                  alibi_slopes=None if m is None else _dev(m))
    torch.cuda.synchronize()
    want = oracle.chunked_prefill(stored_np(c.q), *oracle_pools(c), "bf16",
                                  c.block_table.cpu().numpy(), c.context_lens.cpu().numpy(), scale, alibi=m)
    assert_parity(out.cpu().numpy(), want, "bf16", f"chunked scale={scale}")
