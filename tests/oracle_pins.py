"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` instance and raises
``AssertionError`` when the oracle disagrees with the fixed value. They are
run against the real oracle (test_oracle_pins.py) and against deliberately
broken builds of it (test_oracle_mutants.py), which each pin set must catch.

The expected values never come from the oracle's own formula retyped:
  * library routines that compute the same textbook result independently
    (torch's scaled_dot_product_attention in float64, torch's dtype casts);
  * closed forms (one key -> its value; equal keys or zero scale -> mean of
    the values; two keys -> logistic weights; hand-worked fixtures);
  * invariants the definition implies (GQA equals MHA with the KV heads
    repeated, causal row i equals decode over positions <= i, relabelling
    physical blocks changes nothing, poisoned unread bytes change nothing,
    affine maps of V commute, uniform score shifts cancel, duplicated tokens
    cancel, outputs stay in the convex hull of V).

Page sources: "注意力演进与推理流程" (jerryiiii.gitbook.io), section 3.1 GQA
(g = floor(h/G)) and section 3.2 (repeat_interleave of KV heads); the vLLM
concepts page (yyzxw.github.io), self-attention Steps 2-4, decode attention
over K<=t, V<=t, and the block table / slot mapping paragraph; "LLM 推理全过程的
维度变化与核心公式" (research.frankk.site), sections on decode shapes, the causal
mask and Paged Attention's 16-token blocks.
"""
from __future__ import annotations

import decimal
import json
import math
from pathlib import Path

import numpy as np
import torch

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---- test-side helpers (no oracle code) ---------------------------------------

def stored(x: torch.Tensor, dtype: str) -> np.ndarray:
    """Stored bit patterns of a float tensor in the oracle's calling convention."""
    if dtype == "f32":
        return x.to(torch.float32).contiguous().numpy()
    t = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return x.to(t).contiguous().view(torch.int16).numpy().view(np.uint16)


def exact(x_stored: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 tensor of stored values, via torch's own casts."""
    if dtype == "f32":
        return torch.from_numpy(x_stored.astype(np.float64))
    t = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return torch.from_numpy(x_stored.view(np.int16).copy()).view(t).to(torch.float64)


def pack_pool(seqs, block_size: int, num_blocks: int, rng, fill):
    """Scatter per-sequence rows [ctx][n_kv][d] into a [nb][n_kv][bs][d] pool.

    Logical block j of sequence b goes to physical block ``bt[b][j]``; physical
    ids are a seeded permutation. Unused block-table entries point at the
    remaining (fill-valued) blocks, or at block 0 if none remain.
    """
    n_kv, d = seqs[0].shape[1], seqs[0].shape[2]
    nblk = [-(-s.shape[0] // block_size) for s in seqs]
    maxb = max(1, max(nblk))
    perm = rng.permutation(num_blocks)
    assert sum(nblk) <= num_blocks
    pool = np.full((num_blocks, n_kv, block_size, d), fill, dtype=seqs[0].dtype)
    bt = np.zeros((len(seqs), maxb), dtype=np.int32)
    cur = 0
    for b, s in enumerate(seqs):
        for j in range(nblk[b]):
            phys = perm[cur]
            cur += 1
            bt[b, j] = phys
            rows = s[j * block_size:(j + 1) * block_size]            # [n][n_kv][d]
            pool[phys, :, :rows.shape[0], :] = rows.transpose(1, 0, 2)
    spare = perm[cur:]
    for b in range(len(seqs)):
        for j in range(nblk[b], maxb):
            bt[b, j] = spare[(b + j) % len(spare)] if len(spare) else 0
    return pool, bt


def sdpa64(q, k, v, scale, causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU; q [H][Lq][d], k/v [H][Lk][d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), scale=scale, is_causal=causal)[0]


def rand_seqs(rng_t: torch.Generator, ctxs, n_kv, d, dtype):
    return [stored(torch.randn(c, n_kv, d, generator=rng_t), dtype) for c in ctxs]


def decode_case(seed, ctxs, n_q, n_kv, d, dtype="f32", bs=4, extra_blocks=3, fill=np.nan):
    """Random contiguous sequences plus their paged form; returns everything a pin needs."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    ks = rand_seqs(g, ctxs, n_kv, d, dtype)
    vs = rand_seqs(g, ctxs, n_kv, d, dtype)
    q = stored(torch.randn(len(ctxs), n_q, d, generator=g), dtype)
    nb = sum(-(-c // bs) for c in ctxs) + extra_blocks
    fill_s = stored(torch.tensor([fill], dtype=torch.float64), dtype)[0]
    kp, bt = pack_pool(ks, bs, nb, np.random.default_rng(seed + 1), fill_s)
    vp, bt2 = pack_pool(vs, bs, nb, np.random.default_rng(seed + 1), fill_s)
    assert (bt == bt2).all()
    return dict(q=q, ks=ks, vs=vs, kp=kp, vp=vp, bt=bt, ctx=np.asarray(ctxs, np.int32),
                scale=1.0 / math.sqrt(d), n_q=n_q, n_kv=n_kv, d=d, dtype=dtype, rng=rng)


def run_decode(orc, c, **over):
    args = dict(q=c["q"], k_pool=c["kp"], v_pool=c["vp"], dtype=c["dtype"],
                block_table=c["bt"], context_lens=c["ctx"], scale=c["scale"])
    args.update(over)
    return orc.decode(**args)


def close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.isfinite(a).all(), f"{what}: non-finite oracle output"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---- widening of stored values --------------------------------------------------

def pin_upcast_bf16_every_pattern(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.upcast(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all(), "bf16 NaN patterns differ"
    assert (got[~nan] == want[~nan]).all(), "bf16 widening differs from torch's cast"


def pin_upcast_f16_every_pattern(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.upcast(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all(), "f16 NaN patterns differ"
    assert (got[~nan] == want[~nan]).all(), "f16 widening differs from numpy's cast"


# ---- decode: library routine ---------------------------------------------------------

def _decode_vs_sdpa(orc, n_q, n_kv, dtype, seed):
    ctxs = [1, 5, 9, 16, 23]
    c = decode_case(seed, ctxs, n_q, n_kv, 8, dtype=dtype)
    got = run_decode(orc, c)
    G = n_q // n_kv
    for b, L in enumerate(ctxs):
        q = exact(c["q"][b], dtype).unsqueeze(1)                           # [n_q][1][d]
        k = exact(c["ks"][b], dtype).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [n_q][L][d]
        v = exact(c["vs"][b], dtype).permute(1, 0, 2).repeat_interleave(G, dim=0)
        want = sdpa64(q, k.contiguous(), v.contiguous(), c["scale"])[:, 0, :]
        close(got[b], want.numpy(), 1e-12, f"decode vs sdpa b={b} ctx={L}")


def pin_decode_gqa_matches_library_sdpa(orc):
    _decode_vs_sdpa(orc, n_q=8, n_kv=2, dtype="f32", seed=11)


def pin_decode_mha_matches_library_sdpa(orc):
    _decode_vs_sdpa(orc, n_q=3, n_kv=3, dtype="f32", seed=12)


def pin_decode_mqa_matches_library_sdpa(orc):
    _decode_vs_sdpa(orc, n_q=4, n_kv=1, dtype="bf16", seed=13)


def pin_decode_f16_matches_library_sdpa(orc):
    _decode_vs_sdpa(orc, n_q=4, n_kv=2, dtype="f16", seed=14)


# ---- decode: closed forms --------------------------------------------------------

def pin_decode_single_key_returns_its_value(orc):
    c = decode_case(21, [1, 1], 4, 2, 8)
    got = run_decode(orc, c)
    for b in range(2):
        for h in range(4):
            want = c["vs"][b][0, h // 2].astype(np.float64)
            assert (got[b, h] == want).all(), "ctx=1 must return v exactly"


def pin_decode_equal_keys_give_mean_value(orc):
    c = decode_case(22, [7, 12], 4, 2, 8)
    for b in range(2):
        c["kp"][c["bt"][b]] = c["kp"][c["bt"][b][0], :, 0:1, :]   # every slot of b's blocks
    got = run_decode(orc, c)
    for b in range(2):
        for h in range(4):
            want = c["vs"][b][:, h // 2].astype(np.float64).mean(axis=0)
            close(got[b, h], want, 1e-14, "equal keys -> mean(V)")


def pin_decode_zero_scale_gives_mean_value(orc):
    c = decode_case(23, [5, 13], 2, 1, 8)
    got = run_decode(orc, c, scale=0.0)
    for b in range(2):
        want = c["vs"][b][:, 0].astype(np.float64).mean(axis=0)
        close(got[b, 0], want, 1e-14, "scale=0 -> mean(V)")


def pin_decode_two_keys_logistic(orc):
    c = decode_case(24, [2], 2, 1, 8)
    got = run_decode(orc, c)
    k = c["ks"][0][:, 0].astype(np.float64)
    v = c["vs"][0][:, 0].astype(np.float64)
    for h in range(2):
        q = c["q"][0, h].astype(np.float64)
        delta = c["scale"] * float(q @ (k[1] - k[0]))       # s1 - s0
        w1 = 1.0 / (1.0 + math.exp(-delta))
        close(got[0, h], (1 - w1) * v[0] + w1 * v[1], 1e-14, "two keys -> logistic weights")


def _decimal_decode(q, ks, vs, scale):
    """Softmax attention of one query over a few keys in 40-digit decimal arithmetic."""
    with decimal.localcontext() as ctx:
        ctx.prec = 40
        D = decimal.Decimal
        sc = D(float(scale))
        s = [sc * sum((D(float(a)) * D(float(b)) for a, b in zip(q, k)), D(0)) for k in ks]
        m = max(s)
        w = [(x - m).exp() for x in s]
        tot = sum(w, D(0))
        return np.asarray([float(sum((wi * D(float(v[c])) for wi, v in zip(w, vs)), D(0)) / tot)
                           for c in range(len(vs[0]))], np.float64)


def pin_decode_matches_decimal_bruteforce(orc):
    # Tiny inputs (d <= 4, ctx <= 5) against the definition in 40-digit decimals.
    for seed, ctxs, d in ((41, [1, 3, 5], 4), (42, [2, 4], 3), (43, [5], 2)):
        c = decode_case(seed, ctxs, 2, 1, d, bs=2)
        got = run_decode(orc, c)
        for b, L in enumerate(ctxs):
            for h in range(2):
                want = _decimal_decode(c["q"][b, h], c["ks"][b][:L, 0], c["vs"][b][:L, 0], c["scale"])
                close(got[b, h], want, 1e-14, f"decimal brute force b={b} h={h}")


def pin_decode_hand_worked_fixture(orc):
    fx = json.loads((GOLDEN / "decode_hand_worked.json").read_text())
    bs, d = fx["block_size"], fx["head_dim"]
    k = np.zeros((1, 1, bs, d), np.float32)
    v = np.zeros((1, 1, bs, d), np.float32)
    k[0, 0, :2] = np.asarray(fx["k"], np.float32)
    v[0, 0, :2] = np.asarray(fx["v"], np.float32)
    q = np.asarray(fx["q"], np.float32).reshape(1, 1, d)
    got = orc.decode(q, k, v, "f32", np.zeros((1, 1), np.int32), np.asarray([2], np.int32),
                     fx["scale"])
    close(got[0, 0], fx["expected"], fx["atol"], "hand-worked decode fixture")


def pin_decode_dominant_key(orc):
    c = decode_case(25, [9], 1, 1, 8)
    q = c["q"][0, 0].astype(np.float64)
    j = 5
    c["kp"][c["bt"][0][j // 4], 0, j % 4] = (q * 400.0).astype(np.float32)  # score >> others
    got = run_decode(orc, c)
    close(got[0, 0], c["vs"][0][j, 0], 1e-9, "dominant key selects its value")


def pin_decode_empty_context_is_zero(orc):
    c = decode_case(26, [0, 6], 2, 1, 8)
    got = run_decode(orc, c)
    assert (got[0] == 0).all(), "ctx=0 must give a zero row"
    assert np.isfinite(got[1]).all()


# ---- decode: invariants --------------------------------------------------------------

def pin_decode_gqa_equals_mha_with_repeated_heads(orc):
    n_q, n_kv = 8, 2
    G = n_q // n_kv
    c = decode_case(31, [3, 17, 30], n_q, n_kv, 8)
    got = run_decode(orc, c)
    rep = {k2: np.ascontiguousarray(np.repeat(c[k2], G, axis=1)) for k2 in ("kp", "vp")}
    mha = orc.decode(c["q"], rep["kp"], rep["vp"], "f32", c["bt"], c["ctx"], c["scale"])
    close(got, mha, 1e-15, "GQA vs MHA with repeat_interleaved KV heads")


def pin_decode_block_relabelling_is_bitwise_invariant(orc):
    c = decode_case(32, [6, 21, 14], 4, 2, 8)
    base = run_decode(orc, c)
    nb = c["kp"].shape[0]
    relabel = np.random.default_rng(99).permutation(nb)
    kp = np.empty_like(c["kp"])
    vp = np.empty_like(c["vp"])
    kp[relabel] = c["kp"]
    vp[relabel] = c["vp"]
    got = orc.decode(c["q"], kp, vp, "f32", relabel[c["bt"]].astype(np.int32), c["ctx"],
                     c["scale"])
    assert (got.view(np.uint64) == base.view(np.uint64)).all(), "relabelling changed bits"


def pin_decode_ignores_poisoned_unread_bytes(orc):
    c_nan = decode_case(33, [6, 21, 14], 4, 2, 8, fill=np.nan)
    c_zero = decode_case(33, [6, 21, 14], 4, 2, 8, fill=0.0)
    a = run_decode(orc, c_nan)
    b = run_decode(orc, c_zero)
    assert np.isfinite(a).all(), "NaN in unread slots leaked into the output"
    assert (a == b).all(), "output depends on bytes outside the context"


def _short_mantissa(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to 8 significant bits, so small affine maps stay exact in fp32."""
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def pin_decode_affine_in_values(orc):
    c = decode_case(34, [11, 4], 4, 2, 8)
    c["vp"] = _short_mantissa(c["vp"])
    base = run_decode(orc, c)
    c2 = dict(c)
    c2["vp"] = (c["vp"].astype(np.float64) * 2.0 + 3.0).astype(np.float32)
    got = run_decode(orc, c2)
    close(got, base * 2.0 + 3.0, 1e-13, "out(2V+3) = 2 out(V) + 3")


def pin_decode_uniform_score_shift_cancels(orc):
    c = decode_case(35, [13], 2, 1, 8)
    c["kp"] = _short_mantissa(c["kp"])
    base = run_decode(orc, c)
    c2 = dict(c)
    c2["kp"] = (c["kp"].astype(np.float64) + 0.75).astype(np.float32)   # every key + u
    got = run_decode(orc, c2)
    close(got, base, 1e-13, "adding one vector to every key leaves softmax unchanged")


def pin_decode_duplicated_tokens_cancel(orc):
    c = decode_case(36, [9], 2, 1, 8)
    base = run_decode(orc, c)
    ks = [np.repeat(c["ks"][0], 2, axis=0)]
    vs = [np.repeat(c["vs"][0], 2, axis=0)]
    nb = 8
    kp, bt = pack_pool(ks, 4, nb, np.random.default_rng(5), np.float32(np.nan))
    vp, _ = pack_pool(vs, 4, nb, np.random.default_rng(5), np.float32(np.nan))
    got = orc.decode(c["q"], kp, vp, "f32", bt, np.asarray([18], np.int32), c["scale"])
    close(got, base, 1e-14, "every token twice leaves the output unchanged")


def pin_decode_output_in_convex_hull(orc):
    c = decode_case(37, [25, 8], 4, 2, 8)
    got = run_decode(orc, c)
    for b in range(2):
        for h in range(4):
            v = c["vs"][b][:, h // 2]
            assert (got[b, h] >= v.min(axis=0) - 1e-12).all()
            assert (got[b, h] <= v.max(axis=0) + 1e-12).all()


def pin_decode_selected_rows_match_full(orc):
    c = decode_case(38, [9, 14], 4, 2, 8)
    full = run_decode(orc, c)
    sel = np.asarray([[1, 3], [0, 0], [1, 0]], np.int32)
    part = run_decode(orc, c, sel=sel)
    for r, (b, h) in enumerate(sel):
        assert (part[r] == full[b, h]).all()


def pin_walkthrough_shapes(orc):
    # Decode attention output [B, n_q, 1, d] = [2, 32, 1, 128] for the walk-through's
    # B=2, n_q=32, n_kv=8, d=128 (here with cache_len 3).
    c = decode_case(39, [3, 3], 32, 8, 128, extra_blocks=0)
    assert run_decode(orc, c).shape == (2, 32, 128)
    # Prefill attention output [B, n_q, S, d] for S=10 is stored [B][S][n_q][d].
    g = torch.Generator().manual_seed(40)
    q = stored(torch.randn(2, 10, 32, 128, generator=g), "bf16")
    k = stored(torch.randn(2, 10, 8, 128, generator=g), "bf16")
    out = orc.prefill(q, k, k.copy(), "bf16", True, 1 / math.sqrt(128))
    assert out.shape == (2, 10, 32, 128)


# ---- prefill -----------------------------------------------------------------------------

def _prefill_inputs(seed, B, S, n_q, n_kv, d, dtype="f32"):
    g = torch.Generator().manual_seed(seed)
    q = stored(torch.randn(B, S, n_q, d, generator=g), dtype)
    k = stored(torch.randn(B, S, n_kv, d, generator=g), dtype)
    v = stored(torch.randn(B, S, n_kv, d, generator=g), dtype)
    return q, k, v


def _prefill_vs_sdpa(orc, causal):
    B, S, n_q, n_kv, d = 2, 11, 6, 2, 8
    q, k, v = _prefill_inputs(41 + causal, B, S, n_q, n_kv, d)
    scale = 1 / math.sqrt(d)
    got = orc.prefill(q, k, v, "f32", causal, scale)
    G = n_q // n_kv
    for b in range(B):
        qq = exact(q[b], "f32").permute(1, 0, 2)
        kk = exact(k[b], "f32").permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        vv = exact(v[b], "f32").permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        want = sdpa64(qq.contiguous(), kk, vv, scale, causal=causal).permute(1, 0, 2)
        close(got[b], want.numpy(), 1e-12, f"prefill causal={causal} vs sdpa")


def pin_prefill_causal_matches_library_sdpa(orc):
    _prefill_vs_sdpa(orc, True)


def pin_prefill_noncausal_matches_library_sdpa(orc):
    _prefill_vs_sdpa(orc, False)


def pin_prefill_first_row_is_first_value(orc):
    q, k, v = _prefill_inputs(43, 1, 7, 4, 2, 8)
    got = orc.prefill(q, k, v, "f32", True, 0.35)
    for h in range(4):
        assert (got[0, 0, h] == v[0, 0, h // 2].astype(np.float64)).all()


def pin_prefill_row_equals_decode_over_prefix(orc):
    B, S, n_q, n_kv, d = 2, 13, 4, 2, 8
    q, k, v = _prefill_inputs(44, B, S, n_q, n_kv, d, "bf16")
    scale = 1 / math.sqrt(d)
    pre = orc.prefill(q, k, v, "bf16", True, scale)
    kp, bt = pack_pool([k[b] for b in range(B)], 4, 12, np.random.default_rng(3), np.uint16(0x7FC0))
    vp, _ = pack_pool([v[b] for b in range(B)], 4, 12, np.random.default_rng(3), np.uint16(0x7FC0))
    for i in (0, 3, 7, 12):
        dec = orc.decode(np.ascontiguousarray(q[:, i]), kp, vp, "bf16", bt,
                         np.asarray([i + 1] * B, np.int32), scale)
        close(pre[:, i], dec, 1e-15, f"prefill row {i} vs decode over positions <= {i}")


def pin_prefill_noncausal_row_equals_decode_over_all(orc):
    B, S, n_q, n_kv, d = 1, 9, 2, 1, 8
    q, k, v = _prefill_inputs(45, B, S, n_q, n_kv, d)
    pre = orc.prefill(q, k, v, "f32", False, 0.3)
    kp, bt = pack_pool([k[0]], 4, 3, np.random.default_rng(4), np.float32(np.nan))
    vp, _ = pack_pool([v[0]], 4, 3, np.random.default_rng(4), np.float32(np.nan))
    for i in (0, 4, 8):
        dec = orc.decode(np.ascontiguousarray(q[:, i]), kp, vp, "f32", bt,
                         np.asarray([S], np.int32), 0.3)
        close(pre[:, i], dec, 1e-15, f"non-causal row {i} vs decode over all keys")


# ---- chunked prefill over a paged prefix ---------------------------------------------------

def pin_chunked_prefill_without_prefix_equals_causal_prefill(orc):
    B, S, n_q, n_kv, d = 2, 11, 4, 2, 8
    q, k, v = _prefill_inputs(46, B, S, n_q, n_kv, d)
    want = orc.prefill(q, k, v, "f32", True, 0.3)
    kp, bt = pack_pool([k[b] for b in range(B)], 4, 8, np.random.default_rng(6), np.float32(np.nan))
    vp, _ = pack_pool([v[b] for b in range(B)], 4, 8, np.random.default_rng(6), np.float32(np.nan))
    got = orc.chunked_prefill(q, kp, vp, "f32", bt, np.asarray([S, S], np.int32), 0.3)
    close(got, want, 1e-14, "chunk == whole prompt: causal prefill")


def pin_chunked_prefill_matches_library_sdpa_bottom_right(orc):
    # Sequences of 13 and 21 keys; the last C = 6 are the chunk. Reference: torch's
    # float64 SDPA with an explicit mask (row i sees keys <= prefix + i) and the KV heads
    # repeated G times.
    n_q, n_kv, d, C = 4, 2, 8, 6
    g = torch.Generator().manual_seed(47)
    lens = [13, 21]
    ks = [stored(torch.randn(L, n_kv, d, generator=g), "f32") for L in lens]
    vs = [stored(torch.randn(L, n_kv, d, generator=g), "f32") for L in lens]
    q = stored(torch.randn(len(lens), C, n_q, d, generator=g), "f32")
    kp, bt = pack_pool(ks, 4, 12, np.random.default_rng(7), np.float32(np.nan))
    vp, _ = pack_pool(vs, 4, 12, np.random.default_rng(7), np.float32(np.nan))
    got = orc.chunked_prefill(q, kp, vp, "f32", bt, np.asarray(lens, np.int32), 0.25)
    G = n_q // n_kv
    for b, L in enumerate(lens):
        P = L - C
        mask = torch.arange(L)[None, :] <= (P + torch.arange(C))[:, None]          # [C][L]
        qq = torch.from_numpy(q[b].astype(np.float64)).transpose(0, 1)             # [n_q][C][d]
        kk = torch.from_numpy(ks[b].astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
        vv = torch.from_numpy(vs[b].astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
        want = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), kk.unsqueeze(0), vv.unsqueeze(0), attn_mask=mask, scale=0.25)[0]
        close(got[b], want.transpose(0, 1).numpy(), 1e-12, f"chunked prefill b={b} vs sdpa")


def pin_chunked_prefill_rows_before_the_sequence_are_zero(orc):
    n_q, n_kv, d, C = 2, 1, 8, 5
    g = torch.Generator().manual_seed(48)
    ks = [stored(torch.randn(3, n_kv, d, generator=g), "f32")]
    vs = [stored(torch.randn(3, n_kv, d, generator=g), "f32")]
    q = stored(torch.randn(1, C, n_q, d, generator=g), "f32")
    kp, bt = pack_pool(ks, 4, 2, np.random.default_rng(8), np.float32(np.nan))
    vp, _ = pack_pool(vs, 4, 2, np.random.default_rng(8), np.float32(np.nan))
    got = orc.chunked_prefill(q, kp, vp, "f32", bt, np.asarray([3], np.int32), 0.3)
    assert (got[0, :2] == 0).all(), "rows at positions -2 and -1 must be zero"
    close(got[0, 2, 0], vs[0][0, 0], 1e-15, "row at position 0 returns v_0")


# ---- sliding window ----------------------------------------------------------------------

def pin_decode_window_equals_decode_over_the_last_w(orc):
    # The window W keeps positions ctx-W .. ctx-1: the same as an unwindowed decode of
    # sequences that hold only those rows, packed into a different pool.
    c = decode_case(50, [21, 9, 40], 4, 2, 8)
    W = 7
    got = run_decode(orc, c, window=W)
    tails = [ks[-W:] for ks in c["ks"]], [vs[-W:] for vs in c["vs"]]
    kp, bt = pack_pool(tails[0], 4, 12, np.random.default_rng(51), np.float32(np.nan))
    vp, _ = pack_pool(tails[1], 4, 12, np.random.default_rng(51), np.float32(np.nan))
    want = orc.decode(c["q"], kp, vp, "f32", bt, np.asarray([min(W, L) for L in (21, 9, 40)], np.int32),
                      c["scale"])
    close(got, want, 1e-14, "window W vs decode over the last W rows")


def pin_decode_window_one_returns_the_newest_value(orc):
    c = decode_case(52, [13, 5], 2, 1, 8)
    got = run_decode(orc, c, window=1)
    for b, L in enumerate((13, 5)):
        for h in range(2):
            assert (got[b, h] == c["vs"][b][L - 1, 0].astype(np.float64)).all()


def pin_decode_window_covering_the_context_changes_nothing(orc):
    c = decode_case(53, [10, 17], 4, 2, 8)
    assert (run_decode(orc, c, window=17) == run_decode(orc, c)).all()
    assert (run_decode(orc, c, window=1000) == run_decode(orc, c)).all()


def _band(n_rows, n_keys, first_pos, W):
    pos = first_pos + torch.arange(n_rows)[:, None]
    j = torch.arange(n_keys)[None, :]
    return (j <= pos) & (j > pos - W)


def pin_prefill_window_matches_library_sdpa_band(orc):
    B, S, n_q, n_kv, d, W = 2, 23, 4, 2, 8, 6
    q, k, v = _prefill_inputs(54, B, S, n_q, n_kv, d)
    got = orc.prefill(q, k, v, "f32", True, 0.3, window=W)
    G = n_q // n_kv
    for b in range(B):
        qq = torch.from_numpy(q[b].astype(np.float64)).transpose(0, 1)
        kk = torch.from_numpy(k[b].astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
        vv = torch.from_numpy(v[b].astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
        want = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), kk.unsqueeze(0), vv.unsqueeze(0), attn_mask=_band(S, S, 0, W), scale=0.3)[0]
        close(got[b], want.transpose(0, 1).numpy(), 1e-12, f"windowed prefill b={b} vs sdpa band")


def pin_chunked_prefill_window_matches_library_sdpa_band(orc):
    n_q, n_kv, d, C, W = 4, 2, 8, 5, 9
    g = torch.Generator().manual_seed(55)
    lens = [14, 30]
    ks = [stored(torch.randn(L, n_kv, d, generator=g), "f32") for L in lens]
    vs = [stored(torch.randn(L, n_kv, d, generator=g), "f32") for L in lens]
    q = stored(torch.randn(len(lens), C, n_q, d, generator=g), "f32")
    kp, bt = pack_pool(ks, 4, 14, np.random.default_rng(56), np.float32(np.nan))
    vp, _ = pack_pool(vs, 4, 14, np.random.default_rng(56), np.float32(np.nan))
    got = orc.chunked_prefill(q, kp, vp, "f32", bt, np.asarray(lens, np.int32), 0.25, window=W)
    G = n_q // n_kv
    for b, L in enumerate(lens):
        qq = torch.from_numpy(q[b].astype(np.float64)).transpose(0, 1)
        kk = torch.from_numpy(ks[b].astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
        vv = torch.from_numpy(vs[b].astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
        want = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), kk.unsqueeze(0), vv.unsqueeze(0), attn_mask=_band(C, L, L - C, W),
            scale=0.25)[0]
        close(got[b], want.transpose(0, 1).numpy(), 1e-12, f"windowed chunk b={b} vs sdpa band")


# ---- quantised cache: codes, quantiser, attention over codes * scales -------------------
#
# Quantised cache: the walk-through's KV-cache section, INT8 / FP8 item (per channel or per
# token); per token read as symmetric absolute-maximum scaling of each row, FP8 = OCP E4M3.

def _fp8_values(codes: np.ndarray) -> np.ndarray:
    """float64 values of E4M3 codes through torch's own float8_e4m3fn dtype."""
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _code_values(codes: np.ndarray, fmt: str) -> np.ndarray:
    return _fp8_values(codes) if fmt == "fp8" else codes.astype(np.float64)


def pin_upcast_fp8_every_pattern(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.upcast(codes, "fp8")
    want = _fp8_values(codes)
    nan = np.isnan(want)
    assert nan.sum() == 2 and (np.isnan(got) == nan).all(), "E4M3 NaN patterns differ"
    assert (got[~nan] == want[~nan]).all(), "E4M3 widening differs from torch's float8_e4m3fn"
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def pin_upcast_int8_every_pattern(orc):
    codes = np.arange(-128, 128, dtype=np.int8)
    assert (orc.upcast(codes, "int8") == codes.astype(np.float64)).all()


def pin_encode_fp8_matches_library_cast(orc):
    vals = _fp8_values(np.arange(256, dtype=np.uint8))
    vals = np.unique(vals[np.isfinite(vals)]).astype(np.float32)          # every finite value
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)   # exact in fp32
    y = np.concatenate([vals, mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(-np.inf)),
                        np.random.default_rng(60).normal(0, 60, 20000).astype(np.float32),
                        np.random.default_rng(61).normal(0, 0.01, 5000).astype(np.float32)])
    y = y[np.abs(y) <= 448].astype(np.float32)
    got = orc.encode_fp8(y)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"E4M3 encoding differs from torch at y={y[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"


def pin_quantize_hand_worked_fixture(orc):
    fx = json.loads((GOLDEN / "quantize_hand_worked.json").read_text())
    for row in fx["rows"]:
        x = np.asarray(row["x"], np.float32)[None, :]
        codes, scales = orc.quantize_rows(x, "f32", row["fmt"])
        assert scales[0] == np.float32(row["scale"]), f"{row['fmt']}: scale {scales[0]} vs {row['scale']}"
        want = np.asarray(row["codes"], np.uint8 if row["fmt"] == "fp8" else np.int8)
        assert (codes[0] == want).all(), f"{row['fmt']}: codes {codes[0]} vs {want}"


def pin_quantize_exact_rows_round_trip(orc):
    # Rows whose values are codes times a power of two, with a largest-magnitude element at
    # QMAX times that power: the scale is exactly the power and the codes are the values.
    rng = np.random.default_rng(62)
    fp8_vals = _fp8_values(np.arange(256, dtype=np.uint8))
    finite = np.nonzero(np.isfinite(fp8_vals))[0].astype(np.uint8)
    for fmt, qmax in (("fp8", 448.0), ("int8", 127.0)):
        for p in (0, -5, 7):
            if fmt == "fp8":
                c = rng.choice(finite, size=(6, 16))
                c[:, 3] = 0x7E if p != 7 else 0xFE                        # +-448
            else:
                c = rng.integers(-127, 128, size=(6, 16)).astype(np.int8)
                c[:, 5] = 127 if p != 7 else -127
            x = (_code_values(c, fmt) * 2.0 ** p).astype(np.float32)
            codes, scales = orc.quantize_rows(x, "f32", fmt)
            assert (scales == np.float32(2.0 ** p)).all(), f"{fmt} p={p}: scales {scales}"
            assert (_code_values(codes, fmt) == _code_values(c, fmt)).all(), f"{fmt} p={p}: codes differ"


def pin_quantize_error_bound_and_extremes(orc):
    g = torch.Generator().manual_seed(63)
    x = stored(torch.randn(200, 64, generator=g) * torch.rand(200, 1, generator=g) * 10, "bf16")
    xv = exact(x, "bf16").numpy()
    amax = np.abs(xv).max(axis=1)
    for fmt, qmax in (("fp8", 448.0), ("int8", 127.0)):
        codes, scales = orc.quantize_rows(x, "bf16", fmt)
        s = scales.astype(np.float64)
        assert np.allclose(s, amax / qmax, rtol=2.0 ** -23, atol=0), f"{fmt}: scale is not amax / QMAX"
        deq = _code_values(codes, fmt) * s[:, None]
        err = np.abs(deq - xv)
        if fmt == "int8":   # half a step, plus the fp32 rounding of 1/scale and of x * (1/scale)
            bound = s[:, None] * (0.5 + 128 * 2.0 ** -22)
        else:   # half a unit in the last place of y: 2^-4 |y|, or 2^-10 in the subnormal range
            bound = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 2.0 ** -20)
        assert (err <= bound).all(), f"{fmt}: round-trip error {float((err - bound).max()):.3e} over the bound"
        top = np.abs(xv) == amax[:, None]
        assert (np.abs(_code_values(codes, fmt))[top] == qmax).all(), f"{fmt}: the largest element must map to QMAX"


def pin_quantize_zero_and_tiny_rows(orc):
    x = np.zeros((3, 8), np.float32)
    x[1, 2] = 1e-38            # amax / 448 is below the smallest normal float: stored as zero
    x[2, 5] = -3.0
    for fmt in ("fp8", "int8"):
        codes, scales = orc.quantize_rows(x, "f32", fmt)
        assert scales[0] == 0 and scales[1] == 0 and (_code_values(codes[:2], fmt) == 0).all()
        assert abs(_code_values(codes[2:], fmt)[0, 5] * scales[2] + 3.0) < 1e-6


def pin_kv_append_quant_places_quantised_rows(orc):
    g = torch.Generator().manual_seed(64)
    nb, n_kv, bs, d, T = 5, 2, 4, 16, 7
    k = stored(torch.randn(T, n_kv, d, generator=g), "bf16")
    v = stored(torch.randn(T, n_kv, d, generator=g) * 3, "bf16")
    slots = np.random.default_rng(64).choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[4] = -1
    for fmt in ("fp8", "int8"):
        cdt = np.uint8 if fmt == "fp8" else np.int8
        kp = np.full((nb, n_kv, bs, d), 0x11, cdt)
        vp = kp.copy()
        ks = np.full((nb, n_kv, bs), -7.0, np.float32)
        vs = ks.copy()
        assert orc.kv_append_quant(k, v, "bf16", slots, kp, vp, ks, vs, fmt) == T - 1
        kc, kscale = orc.quantize_rows(k, "bf16", fmt)
        vc, vscale = orc.quantize_rows(v, "bf16", fmt)
        # Independent placement view: slot s is row s of a [nb*bs][n_kv] transpose.
        kt = kp.transpose(0, 2, 1, 3).reshape(nb * bs, n_kv, d)
        vt = vp.transpose(0, 2, 1, 3).reshape(nb * bs, n_kv, d)
        kst = ks.transpose(0, 2, 1).reshape(nb * bs, n_kv)
        vst = vs.transpose(0, 2, 1).reshape(nb * bs, n_kv)
        keep = np.ones(nb * bs, bool)
        for t, s in enumerate(slots):
            if s < 0:
                continue
            keep[s] = False
            assert (kt[s] == kc[t]).all() and (vt[s] == vc[t]).all(), f"{fmt}: codes of token {t}"
            assert (kst[s] == kscale[t]).all() and (vst[s] == vscale[t]).all(), f"{fmt}: scales of token {t}"
        assert (kt[keep] == 0x11).all() and (kst[keep] == -7.0).all(), f"{fmt}: untouched slots changed"


def pin_decode_quantised_matches_library_sdpa(orc):
    ctxs, n_q, n_kv, d, bs = [1, 6, 13, 20], 8, 2, 16, 4
    G = n_q // n_kv
    g = torch.Generator().manual_seed(65)
    q = stored(torch.randn(len(ctxs), n_q, d, generator=g), "bf16")
    for fmt in ("fp8", "int8"):
        kc, vc, ksc, vsc = [], [], [], []
        for L in ctxs:
            krow = stored(torch.randn(L, n_kv, d, generator=g), "bf16")
            vrow = stored(torch.randn(L, n_kv, d, generator=g) * 2, "bf16")
            a, sa = orc.quantize_rows(krow, "bf16", fmt)
            b_, sb = orc.quantize_rows(vrow, "bf16", fmt)
            kc.append(a); vc.append(b_); ksc.append(sa); vsc.append(sb)
        nb = sum(-(-L // bs) for L in ctxs) + 2
        fill = np.array(0x7F if fmt == "fp8" else 99).astype(kc[0].dtype)   # NaN code / junk
        kp, bt = pack_pool(kc, bs, nb, np.random.default_rng(66), fill)
        vp, _ = pack_pool(vc, bs, nb, np.random.default_rng(66), fill)
        ksp, _ = pack_pool([s[..., None] for s in ksc], bs, nb, np.random.default_rng(66), np.float32(np.nan))
        vsp, _ = pack_pool([s[..., None] for s in vsc], bs, nb, np.random.default_rng(66), np.float32(np.nan))
        got = orc.decode(q, kp, vp, fmt, bt, np.asarray(ctxs, np.int32), 0.3, q_dtype="bf16",
                         k_scale=np.ascontiguousarray(ksp[..., 0]), v_scale=np.ascontiguousarray(vsp[..., 0]))
        for b, L in enumerate(ctxs):
            kk = _code_values(kc[b], fmt) * ksc[b][..., None].astype(np.float64)     # [L][n_kv][d]
            vv = _code_values(vc[b], fmt) * vsc[b][..., None].astype(np.float64)
            qq = exact(q[b], "bf16").unsqueeze(1)
            k_t = torch.from_numpy(kk).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
            v_t = torch.from_numpy(vv).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
            want = sdpa64(qq, k_t, v_t, 0.3)[:, 0, :]
            close(got[b], want.numpy(), 1e-12, f"{fmt} decode vs sdpa over codes * scales, b={b}")


def pin_chunked_prefill_quantised_matches_library_sdpa(orc):
    # Chunk rows over a per-token quantised cache: torch's float64 SDPA with the bottom-right
    # causal mask over K and V rebuilt as codes * row scales.
    n_q, n_kv, d, bs, C = 4, 2, 8, 4, 5
    G = n_q // n_kv
    g = torch.Generator().manual_seed(67)
    lens = [9, 14]
    q = stored(torch.randn(len(lens), C, n_q, d, generator=g), "f16")
    for fmt in ("fp8", "int8"):
        kc, vc, ksc, vsc = [], [], [], []
        for L in lens:
            a, sa = orc.quantize_rows(stored(torch.randn(L, n_kv, d, generator=g), "f16"), "f16", fmt)
            b_, sb = orc.quantize_rows(stored(torch.randn(L, n_kv, d, generator=g) * 3, "f16"), "f16", fmt)
            kc.append(a); vc.append(b_); ksc.append(sa); vsc.append(sb)
        fill = np.array(0x7F if fmt == "fp8" else 77).astype(kc[0].dtype)
        kp, bt = pack_pool(kc, bs, 9, np.random.default_rng(68), fill)
        vp, _ = pack_pool(vc, bs, 9, np.random.default_rng(68), fill)
        ksp, _ = pack_pool([x[..., None] for x in ksc], bs, 9, np.random.default_rng(68), np.float32(np.nan))
        vsp, _ = pack_pool([x[..., None] for x in vsc], bs, 9, np.random.default_rng(68), np.float32(np.nan))
        got = orc.chunked_prefill(q, kp, vp, fmt, bt, np.asarray(lens, np.int32), 0.35, q_dtype="f16",
                                  k_scale=np.ascontiguousarray(ksp[..., 0]), v_scale=np.ascontiguousarray(vsp[..., 0]))
        for b, L in enumerate(lens):
            kk = _code_values(kc[b], fmt) * ksc[b][..., None].astype(np.float64)
            vv = _code_values(vc[b], fmt) * vsc[b][..., None].astype(np.float64)
            mask = torch.arange(L)[None, :] <= (L - C + torch.arange(C))[:, None]
            qq = exact(q[b], "f16").transpose(0, 1)
            k_t = torch.from_numpy(kk).transpose(0, 1).repeat_interleave(G, 0).contiguous()
            v_t = torch.from_numpy(vv).transpose(0, 1).repeat_interleave(G, 0).contiguous()
            want = torch.nn.functional.scaled_dot_product_attention(
                qq.unsqueeze(0), k_t.unsqueeze(0), v_t.unsqueeze(0), attn_mask=mask, scale=0.35)[0]
            close(got[b], want.transpose(0, 1).numpy(), 1e-12, f"{fmt} chunk rows vs sdpa over codes * scales, b={b}")


# ---- per-channel scales ------------------------------------------------------------------
#
# The same item's other granularity: one fixed fp32 scale per (KV head, channel), given by the
# caller, the same fp32 code steps as per token, saturating at QMAX.

def pin_quantize_channels_hand_worked_fixture(orc):
    fx = json.loads((GOLDEN / "quantize_channels_hand_worked.json").read_text())
    x = np.asarray(fx["x"], np.float32)[None]              # [1][n_kv][d]
    scales = np.asarray(fx["scales"], np.float32)
    assert scales[1, 2] > 0, "the subnormal scale must survive the float32 cast"
    for fmt, want in fx["codes"].items():
        codes = orc.quantize_channels(x, "f32", fmt, scales)
        want = np.asarray(want, np.uint8 if fmt == "fp8" else np.int8)
        assert (codes[0] == want).all(), f"{fmt}: codes {codes[0].tolist()} vs {want.tolist()}"


def pin_quantize_channels_exact_round_trip(orc):
    # Values that are codes times their channel's power-of-two scale come back as those codes.
    rng = np.random.default_rng(69)
    finite = np.nonzero(np.isfinite(_fp8_values(np.arange(256, dtype=np.uint8))))[0].astype(np.uint8)
    n_kv, d = 3, 16
    pw = rng.integers(-6, 7, size=(n_kv, d))
    scales = (2.0 ** pw).astype(np.float32)
    for fmt in ("fp8", "int8"):
        c = rng.choice(finite, size=(5, n_kv, d)) if fmt == "fp8" else rng.integers(-127, 128, (5, n_kv, d)).astype(np.int8)
        x = (_code_values(c, fmt) * scales.astype(np.float64)).astype(np.float32)
        codes = orc.quantize_channels(x, "f32", fmt, scales)
        assert (_code_values(codes, fmt) == _code_values(c, fmt)).all(), f"{fmt}: codes differ"


def pin_quantize_channels_error_bound_and_saturation(orc):
    g = torch.Generator().manual_seed(70)
    n_kv, d = 2, 32
    x = stored(torch.randn(300, n_kv, d, generator=g) * 4, "bf16")
    xv = exact(x, "bf16").numpy()
    for fmt, qmax in (("fp8", 448.0), ("int8", 127.0)):
        # Scales that cover about 90% of each channel's values; the rest must saturate.
        cover = np.quantile(np.abs(xv), 0.9, axis=0)                      # [n_kv][d]
        scales = (cover / qmax).astype(np.float32)
        s = scales.astype(np.float64)[None]
        codes = orc.quantize_channels(x, "bf16", fmt, scales)
        deq = _code_values(codes, fmt) * s
        inside = np.abs(xv) <= qmax * s * (1 - 2.0 ** -20)
        if fmt == "int8":
            bound = s * (0.5 + 128 * 2.0 ** -22)
        else:
            bound = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 2.0 ** -20)
        err = np.abs(deq - xv)
        assert (err[inside] <= np.broadcast_to(bound, err.shape)[inside]).all(), f"{fmt}: error over the bound"
        out = np.abs(xv) > qmax * s * (1 + 2.0 ** -20)
        assert out.sum() > 100, "the case must exercise saturation"
        cv = _code_values(codes, fmt)
        assert (np.abs(cv[out]) == qmax).all() and (np.sign(cv[out]) == np.sign(xv[out])).all(), \
            f"{fmt}: values past QMAX * scale must saturate to +-QMAX"


def pin_quantize_channels_with_the_row_scale_match_per_token(orc):
    # One KV head whose channel scales all equal a row's per-token scale quantises that row
    # exactly as the per-token quantiser does.
    g = torch.Generator().manual_seed(71)
    x = stored(torch.randn(20, 1, 24, generator=g) * 5, "f16")
    for fmt in ("fp8", "int8"):
        codes_t, sc = orc.quantize_rows(x, "f16", fmt)
        for r in range(x.shape[0]):
            codes_c = orc.quantize_channels(x[r:r + 1], "f16", fmt, np.full((1, 24), sc[r, 0], np.float32))
            assert (codes_c[0] == codes_t[r]).all(), f"{fmt}: row {r} differs from the per-token codes"


def pin_kv_append_quant_channel_places_codes(orc):
    g = torch.Generator().manual_seed(72)
    nb, n_kv, bs, d, T = 5, 2, 4, 16, 7
    k = stored(torch.randn(T, n_kv, d, generator=g), "bf16")
    v = stored(torch.randn(T, n_kv, d, generator=g) * 3, "bf16")
    kch = (np.abs(np.random.default_rng(72).normal(0, 0.02, (n_kv, d))) + 1e-3).astype(np.float32)
    vch = (np.abs(np.random.default_rng(73).normal(0, 0.05, (n_kv, d))) + 1e-3).astype(np.float32)
    slots = np.random.default_rng(74).choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[2] = -1
    for fmt in ("fp8", "int8"):
        cdt = np.uint8 if fmt == "fp8" else np.int8
        kp = np.full((nb, n_kv, bs, d), 0x11, cdt)
        vp = kp.copy()
        assert orc.kv_append_quant_channel(k, v, "bf16", slots, kp, vp, kch, vch, fmt) == T - 1
        kc = orc.quantize_channels(k, "bf16", fmt, kch)
        vc = orc.quantize_channels(v, "bf16", fmt, vch)
        kt = kp.transpose(0, 2, 1, 3).reshape(nb * bs, n_kv, d)
        vt = vp.transpose(0, 2, 1, 3).reshape(nb * bs, n_kv, d)
        keep = np.ones(nb * bs, bool)
        for t, s_ in enumerate(slots):
            if s_ < 0:
                continue
            keep[s_] = False
            assert (kt[s_] == kc[t]).all() and (vt[s_] == vc[t]).all(), f"{fmt}: codes of token {t}"
        assert (kt[keep] == 0x11).all() and (vt[keep] == 0x11).all(), f"{fmt}: untouched slots changed"


def pin_decode_channel_quantised_matches_library_sdpa(orc):
    ctxs, n_q, n_kv, d, bs = [1, 7, 13, 22], 8, 2, 16, 4
    G = n_q // n_kv
    g = torch.Generator().manual_seed(75)
    rng = np.random.default_rng(75)
    q = stored(torch.randn(len(ctxs), n_q, d, generator=g), "bf16")
    kch = (rng.uniform(0.002, 0.02, (n_kv, d))).astype(np.float32)
    vch = (rng.uniform(0.005, 0.05, (n_kv, d))).astype(np.float32)
    for fmt in ("fp8", "int8"):
        kc = [orc.quantize_channels(stored(torch.randn(L, n_kv, d, generator=g), "bf16"), "bf16", fmt, kch)
              for L in ctxs]
        vc = [orc.quantize_channels(stored(torch.randn(L, n_kv, d, generator=g) * 2, "bf16"), "bf16", fmt, vch)
              for L in ctxs]
        nb = sum(-(-L // bs) for L in ctxs) + 2
        fill = np.array(0x7F if fmt == "fp8" else 99).astype(kc[0].dtype)
        kp, bt = pack_pool(kc, bs, nb, np.random.default_rng(76), fill)
        vp, _ = pack_pool(vc, bs, nb, np.random.default_rng(76), fill)
        got = orc.decode(q, kp, vp, fmt, bt, np.asarray(ctxs, np.int32), 0.3, q_dtype="bf16",
                         k_scale=kch, v_scale=vch, scale_mode="channel")
        for b, L in enumerate(ctxs):
            kk = _code_values(kc[b], fmt) * kch.astype(np.float64)[None]       # [L][n_kv][d]
            vv = _code_values(vc[b], fmt) * vch.astype(np.float64)[None]
            qq = exact(q[b], "bf16").unsqueeze(1)
            k_t = torch.from_numpy(kk).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
            v_t = torch.from_numpy(vv).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
            want = sdpa64(qq, k_t, v_t, 0.3)[:, 0, :]
            close(got[b], want.numpy(), 1e-12, f"{fmt} per-channel decode vs sdpa, b={b}")


def pin_chunked_prefill_channel_quantised_matches_library_sdpa(orc):
    n_q, n_kv, d, bs, C = 6, 3, 8, 4, 4
    G = n_q // n_kv
    g = torch.Generator().manual_seed(77)
    rng = np.random.default_rng(77)
    lens = [6, 11]
    q = stored(torch.randn(len(lens), C, n_q, d, generator=g), "bf16")
    kch = rng.uniform(0.002, 0.03, (n_kv, d)).astype(np.float32)
    vch = rng.uniform(0.002, 0.03, (n_kv, d)).astype(np.float32)
    for fmt in ("fp8", "int8"):
        kc = [orc.quantize_channels(stored(torch.randn(L, n_kv, d, generator=g), "bf16"), "bf16", fmt, kch)
              for L in lens]
        vc = [orc.quantize_channels(stored(torch.randn(L, n_kv, d, generator=g), "bf16"), "bf16", fmt, vch)
              for L in lens]
        fill = np.array(0x7F if fmt == "fp8" else 55).astype(kc[0].dtype)
        kp, bt = pack_pool(kc, bs, 7, np.random.default_rng(78), fill)
        vp, _ = pack_pool(vc, bs, 7, np.random.default_rng(78), fill)
        got = orc.chunked_prefill(q, kp, vp, fmt, bt, np.asarray(lens, np.int32), 0.4, q_dtype="bf16",
                                  k_scale=kch, v_scale=vch, scale_mode="channel")
        for b, L in enumerate(lens):
            kk = _code_values(kc[b], fmt) * kch.astype(np.float64)[None]
            vv = _code_values(vc[b], fmt) * vch.astype(np.float64)[None]
            mask = torch.arange(L)[None, :] <= (L - C + torch.arange(C))[:, None]
            qq = exact(q[b], "bf16").transpose(0, 1)
            k_t = torch.from_numpy(kk).transpose(0, 1).repeat_interleave(G, 0).contiguous()
            v_t = torch.from_numpy(vv).transpose(0, 1).repeat_interleave(G, 0).contiguous()
            want = torch.nn.functional.scaled_dot_product_attention(
                qq.unsqueeze(0), k_t.unsqueeze(0), v_t.unsqueeze(0), attn_mask=mask, scale=0.4)[0]
            close(got[b], want.transpose(0, 1).numpy(), 1e-12, f"{fmt} per-channel chunk rows vs sdpa, b={b}")


# ---- kv_append ---------------------------------------------------------------------------

def pin_kv_append_hand_worked_fixture(orc):
    fx = json.loads((GOLDEN / "kv_append_small.json").read_text())
    nb, n_kv, bs, d = fx["num_blocks"], fx["n_kv"], fx["block_size"], fx["head_dim"]
    kp = np.full((nb, n_kv, bs, d), fx["pool_fill"], np.float32)
    vp = kp.copy()
    k = np.asarray(fx["k"], np.float32)
    v = np.asarray(fx["v"], np.float32)
    n = orc.kv_append(k, v, np.asarray(fx["slot_mapping"], np.int64), kp, vp)
    assert n == fx["expected_written"]
    want_k = np.full_like(kp, fx["pool_fill"])
    want_v = want_k.copy()
    for blk, head, off, krow, vrow in fx["expected_rows"]:
        want_k[blk, head, off] = krow
        want_v[blk, head, off] = vrow
    assert (kp == want_k).all(), "K pool differs from the hand-worked placement"
    assert (vp == want_v).all(), "V pool differs from the hand-worked placement"


def pin_kv_append_is_a_bitwise_copy(orc):
    g = torch.Generator().manual_seed(51)
    nb, n_kv, bs, d, T = 6, 3, 4, 8, 9
    kp = stored(torch.randn(nb, n_kv, bs, d, generator=g), "bf16")
    vp = stored(torch.randn(nb, n_kv, bs, d, generator=g), "bf16")
    k = stored(torch.randn(T, n_kv, d, generator=g), "bf16")
    v = stored(torch.randn(T, n_kv, d, generator=g), "bf16")
    slots = np.random.default_rng(51).choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[2] = -1
    kp0, vp0 = kp.copy(), vp.copy()
    assert orc.kv_append(k, v, slots, kp, vp) == T - 1
    # Independent view of the same placement: a [nb*bs] row index over a
    # [nb][bs][n_kv][d] transpose of the pool.
    kt = kp.transpose(0, 2, 1, 3).reshape(nb * bs, n_kv, d)
    vt = vp.transpose(0, 2, 1, 3).reshape(nb * bs, n_kv, d)
    kt0 = kp0.transpose(0, 2, 1, 3).reshape(nb * bs, n_kv, d)
    keep = np.ones(nb * bs, bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        keep[s] = False
        assert (kt[s] == k[t]).all() and (vt[s] == v[t]).all(), f"token {t} not at slot {s}"
    assert (kt[keep] == kt0[keep]).all(), "kv_append touched a slot it was not given"


def pin_kv_append_rejects_out_of_range_slot(orc):
    kp = np.zeros((2, 1, 4, 2), np.float32)
    vp = kp.copy()
    k = np.ones((1, 1, 2), np.float32)
    try:
        orc.kv_append(k, k.copy(), np.asarray([8], np.int64), kp, vp)
    except ValueError:
        assert (kp == 0).all(), "a rejected append must not write"
        return
    raise AssertionError("slot 8 in an 8-slot pool was accepted")


# ---- ALiBi bias ("LLM 推理全过程的维度变化与核心公式", position-encoding section:
# scores_ij = q_i.k_j / sqrt(d) - m_h (i - j), one slope m_h per head) -------------------

def alibi_slopes(n_q: int) -> np.ndarray:
    """Distinct per-head slopes (the geometric 2^(-8 (h+1) / n_q) family)."""
    return (2.0 ** (-8.0 * (np.arange(n_q) + 1) / n_q)).astype(np.float32)


def sdpa64_bias(q, k, v, scale, bias):
    """torch's float64 SDPA with an additive float mask; q [H][Lq][d], k/v [H][Lk][d], bias [H][Lq][Lk]."""
    return torch.nn.functional.scaled_dot_product_attention(
        q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), attn_mask=bias.unsqueeze(0), scale=scale)[0]


def _alibi_decode_vs_sdpa(orc, window):
    n_q, n_kv, d = 8, 2, 8
    ctxs = [1, 5, 9, 16, 23]
    c = decode_case(71 + window, ctxs, n_q, n_kv, d)
    slopes = alibi_slopes(n_q)
    got = run_decode(orc, c, alibi=slopes, window=window)
    G = n_q // n_kv
    m = torch.from_numpy(slopes.astype(np.float64))
    for b, L in enumerate(ctxs):
        first = L - window if 0 < window < L else 0
        q = exact(c["q"][b], "f32").unsqueeze(1)
        k = exact(c["ks"][b][first:], "f32").permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        v = exact(c["vs"][b][first:], "f32").permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        pos = torch.arange(first, L, dtype=torch.float64)                 # key positions
        bias = (-m[:, None] * ((L - 1) - pos)[None, :]).unsqueeze(1)      # query at L - 1
        want = sdpa64_bias(q, k, v, c["scale"], bias)[:, 0, :]
        close(got[b], want.numpy(), 1e-12, f"alibi decode vs sdpa b={b} ctx={L} window={window}")


def pin_decode_alibi_matches_library_sdpa(orc):
    _alibi_decode_vs_sdpa(orc, window=0)


def pin_decode_alibi_with_window_matches_library_sdpa(orc):
    _alibi_decode_vs_sdpa(orc, window=6)


def pin_prefill_alibi_matches_library_sdpa(orc):
    B, S, n_q, n_kv, d = 2, 11, 6, 2, 8
    q, k, v = _prefill_inputs(72, B, S, n_q, n_kv, d)
    scale = 1 / math.sqrt(d)
    slopes = alibi_slopes(n_q)
    got = orc.prefill(q, k, v, "f32", True, scale, alibi=slopes)
    G = n_q // n_kv
    i = torch.arange(S, dtype=torch.float64)
    dist = i[:, None] - i[None, :]                                        # i - j
    m = torch.from_numpy(slopes.astype(np.float64))
    bias = -m[:, None, None] * dist[None]
    bias = bias.masked_fill((dist < 0)[None], float("-inf"))             # causal
    for b in range(B):
        qq = exact(q[b], "f32").permute(1, 0, 2).contiguous()
        kk = exact(k[b], "f32").permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        vv = exact(v[b], "f32").permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        want = sdpa64_bias(qq, kk, vv, scale, bias).permute(1, 0, 2)
        close(got[b], want.numpy(), 1e-12, "alibi prefill vs sdpa")


def pin_chunked_prefill_alibi_matches_library_sdpa(orc):
    # Sequences of 13 and 21 keys, the last C = 6 the chunk: row r is position L - C + r.
    n_q, n_kv, d, C = 4, 2, 8, 6
    g = torch.Generator().manual_seed(73)
    lens = [13, 21]
    ks = rand_seqs(g, lens, n_kv, d, "f32")
    vs = rand_seqs(g, lens, n_kv, d, "f32")
    q = stored(torch.randn(2, C, n_q, d, generator=g), "f32")
    kp, bt = pack_pool(ks, 4, 12, np.random.default_rng(8), np.float32(np.nan))
    vp, _ = pack_pool(vs, 4, 12, np.random.default_rng(8), np.float32(np.nan))
    slopes = alibi_slopes(n_q)
    got = orc.chunked_prefill(q, kp, vp, "f32", bt, np.asarray(lens, np.int32), 0.3, alibi=slopes)
    m = torch.from_numpy(slopes.astype(np.float64))
    for b, L in enumerate(lens):
        rows = torch.arange(L - C, L, dtype=torch.float64)
        keys = torch.arange(L, dtype=torch.float64)
        dist = rows[:, None] - keys[None, :]
        bias = (-m[:, None, None] * dist[None]).masked_fill((dist < 0)[None], float("-inf"))
        qq = exact(q[b], "f32").permute(1, 0, 2).contiguous()
        kk = exact(ks[b], "f32").permute(1, 0, 2).repeat_interleave(2, dim=0).contiguous()
        vv = exact(vs[b], "f32").permute(1, 0, 2).repeat_interleave(2, dim=0).contiguous()
        want = sdpa64_bias(qq, kk, vv, 0.3, bias).permute(1, 0, 2)
        close(got[b], want.numpy(), 1e-12, f"alibi chunked prefill vs sdpa, length {L}")


def pin_decode_alibi_closed_form(orc):
    # q = 0 leaves only the bias: position t weighs r^(L-1-t), r = e^-m. With V[t] = t
    # the output is (L - 1) - S1 / S0, S0 = sum_k r^k = (1 - r^L) / (1 - r) and
    # S1 = sum_k k r^k = r (1 - L r^(L-1) + (L - 1) r^L) / (1 - r)^2, k = 0 .. L - 1.
    d, L = 4, 37
    pos = np.arange(L, dtype=np.float32)
    rows = np.repeat(pos[:, None, None], d, axis=2)                      # [L][1][d], row t = t
    kp, bt = pack_pool([np.ones((L, 1, d), np.float32)], 4, 12, np.random.default_rng(9), np.float32(np.nan))
    vp, _ = pack_pool([rows], 4, 12, np.random.default_rng(9), np.float32(np.nan))
    slopes = np.asarray([0.5, 0.125, 0.03125], np.float32)
    q = np.zeros((1, 3, d), np.float32)
    got = orc.decode(q, kp, vp, "f32", bt, np.asarray([L], np.int32), 1.0, alibi=slopes)
    for h, m in enumerate(slopes.astype(np.float64)):
        r = math.exp(-m)
        s0 = (1 - r ** L) / (1 - r)
        s1 = r * (1 - L * r ** (L - 1) + (L - 1) * r ** L) / (1 - r) ** 2
        close(got[0, h], np.full(d, (L - 1) - s1 / s0), 1e-12, f"alibi closed form, slope {m}")


def pin_decode_alibi_zero_slopes_change_nothing(orc):
    c = decode_case(74, [3, 17, 30], 4, 2, 8, dtype="bf16")
    plain = run_decode(orc, c)
    zero = run_decode(orc, c, alibi=np.zeros(4, np.float32))
    assert (plain == zero).all(), "zero ALiBi slopes changed the output"


ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
