"""Seeded synthetic inputs for paged GQA attention.

This module only draws random numbers, permutations and poison patterns and
lays them out in the documented buffer formats. It holds none of the
attention arithmetic, and it is the one module that both the GPU path's
callers (tests, the benchmark) and the CPU oracle's callers share.

Shapes follow the LLaMA-3 walk-through on the pages ("LLM 推理全过程的维度变化与
核心公式", research.frankk.site, symbol table and "Decode 阶段维度流转": n_q=32,
n_kv=8, d=128; and the LLaMA-3 symbol table of "注意力演进与推理流程",
jerryiiii.gitbook.io). The paged layout uses blocks of 16 tokens (same
walk-through, "KV Cache 的形状与增长", Paged Attention item).

Recipe (every config):
  * values ~ N(0, 1) drawn in fp32 with a seeded ``torch.Generator`` on the
    target device, then cast to the storage dtype (round to nearest even);
  * block permutations, shared-prefix choice and context lengths from
    ``numpy.random.default_rng(seed)``;
  * every pool byte the kernels must not read -- free blocks, slots at or past
    each sequence's new-token position, the new-token slot itself before the
    append -- holds NaN;
  * block-table entries past a sequence's last block point at free (poisoned)
    blocks when the pool has any.

Pool layout: ``[num_blocks][n_kv][block_size][head_dim]``, head_dim fastest.
Block table: int32 ``[B][max_blocks_per_seq]``, entry j = physical block of
logical block j. context_lens: int32 ``[B]``, tokens attended *including* the
token appended in the same step. slot_mapping: int64, flat slot =
physical_block * block_size + offset.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass
class DecodeCase:
    """One decode step over a paged cache: append one new token per sequence, then attend."""

    name: str
    dtype: str
    batch: int
    n_q: int
    n_kv: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: torch.Tensor             # [B][n_q][d]
    k_pool: torch.Tensor        # [num_blocks][n_kv][bs][d]  (before the append)
    v_pool: torch.Tensor
    block_table: torch.Tensor   # int32 [B][max_blocks_per_seq]
    context_lens: torch.Tensor  # int32 [B]  (including the new token)
    new_k: torch.Tensor         # [B][n_kv][d]  one new token per sequence
    new_v: torch.Tensor
    slot_mapping: torch.Tensor  # int64 [B]   slot of each new token
    shared_prefix_blocks: int = 0
    sharers: list = field(default_factory=list)
    free_blocks: np.ndarray | None = None

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def to(self, device) -> "DecodeCase":
        out = DecodeCase(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        for k in ("q", "k_pool", "v_pool", "block_table", "context_lens", "new_k", "new_v",
                  "slot_mapping"):
            setattr(out, k, getattr(self, k).to(device))
        return out


@dataclass
class PrefillCase:
    """Causal prefill of a prompt, its cache write, then one decode step (config-5 flow)."""

    name: str
    dtype: str
    batch: int
    seq_len: int
    n_q: int
    n_kv: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: torch.Tensor             # [B][S][n_q][d]
    k: torch.Tensor             # [B][S][n_kv][d]
    v: torch.Tensor
    block_table: torch.Tensor   # int32 [B][blocks_per_seq]
    prompt_slots: torch.Tensor  # int64 [B*S]   slot of prompt token (b, t) at b*S + t
    k_pool: torch.Tensor        # [num_blocks][n_kv][bs][d], all NaN before the prompt append
    v_pool: torch.Tensor
    q_new: torch.Tensor         # [B][n_q][d]   the first decode step after the prompt
    new_k: torch.Tensor         # [B][n_kv][d]
    new_v: torch.Tensor
    new_slots: torch.Tensor     # int64 [B]     slot of position S
    context_lens: torch.Tensor  # int32 [B] = S + 1


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, dtype: str, gen: torch.Generator, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(TORCH_DTYPES[dtype])


def geometric_alibi_slopes(n_q: int, device="cpu") -> torch.Tensor:
    """Per-query-head ALiBi slopes m_h = 2^(-8 (h+1) / n_q), float32 [n_q]: the family the
    ALiBi paper uses (Press et al., ICLR 2022, cited by "LLM 推理全过程的维度变化与核心公式").
    They are model constants that the attention calls take as an input."""
    h = torch.arange(1, n_q + 1, dtype=torch.float64)
    return (2.0 ** (-8.0 * h / n_q)).to(torch.float32).to(device)


def make_decode_case(*, batch: int, n_q: int, n_kv: int, head_dim: int, context_lens,
                     dtype: str = "bf16", block_size: int = 16, free_fraction: float = 0.0,
                     num_blocks: int | None = None, max_blocks_per_seq: int | None = None,
                     shared_prefix_blocks: int = 0, n_sharers: int = 0, seed: int = 0,
                     device="cpu", name: str = "custom", values: bool = True) -> DecodeCase:
    """Build a paged decode step with seeded values and a seeded physical scatter.

    ``context_lens`` counts the token appended in this step, so the new token of
    sequence b sits at logical position ``context_lens[b] - 1``. Sequences chosen
    as sharers point their first ``shared_prefix_blocks`` logical blocks at the
    same physical blocks; a sharer's context must extend past that prefix so its
    new token never lands in a shared block. ``values=False`` builds the same
    structure with zero-filled tensors (for structure-only checks).
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    if ctx.shape[0] != batch:
        raise ValueError("context_lens must have one entry per sequence")
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    nblk = (ctx + block_size - 1) // block_size
    maxb = int(max_blocks_per_seq or max(1, int(nblk.max(initial=0))))
    if (nblk > maxb).any():
        raise ValueError("a context does not fit max_blocks_per_seq")

    sharers: list[int] = []
    if shared_prefix_blocks and n_sharers:
        eligible = np.nonzero(ctx > shared_prefix_blocks * block_size)[0]
        if eligible.size < n_sharers:
            raise ValueError("not enough sequences longer than the shared prefix")
        sharers = sorted(int(b) for b in rng.choice(eligible, size=n_sharers, replace=False))
    n_pref = shared_prefix_blocks if sharers else 0

    used = n_pref + int(sum(int(nblk[b]) - (n_pref if b in sharers else 0) for b in range(batch)))
    if num_blocks is None:
        num_blocks = max(1, math.ceil(used / (1.0 - free_fraction)))
    if num_blocks < used:
        raise ValueError("pool too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    prefix_ids = perm[:n_pref]
    cursor = n_pref
    bt = np.zeros((batch, maxb), dtype=np.int32)
    for b in range(batch):
        j0 = 0
        if b in sharers:
            bt[b, :n_pref] = prefix_ids
            j0 = n_pref
        own = int(nblk[b]) - j0
        bt[b, j0:j0 + own] = perm[cursor:cursor + own]
        cursor += own
    free = perm[cursor:]
    for b in range(batch):
        tail = maxb - int(nblk[b])
        if tail:
            bt[b, int(nblk[b]):] = rng.choice(free, size=tail) if free.size else 0

    gen = _gen(device, seed)
    draw = _randn if values else (lambda shp, dt, g, dev: torch.zeros(shp, dtype=TORCH_DTYPES[dt],
                                                                       device=dev))
    shape = (num_blocks, n_kv, block_size, head_dim)
    k_pool = draw(shape, dtype, gen, device)
    v_pool = draw(shape, dtype, gen, device)
    q = draw((batch, n_q, head_dim), dtype, gen, device)
    new_k = draw((batch, n_kv, head_dim), dtype, gen, device)
    new_v = draw((batch, n_kv, head_dim), dtype, gen, device)

    # Poison: free blocks, and every slot from the new-token position to the end
    # of the sequence's last block.
    nan = float("nan")
    if free.size:
        idx = torch.as_tensor(free.astype(np.int64), device=device)
        k_pool[idx] = nan
        v_pool[idx] = nan
    slots = np.full(batch, -1, dtype=np.int64)
    for b in range(batch):
        if ctx[b] == 0:
            continue
        pos = int(ctx[b]) - 1
        slots[b] = int(bt[b, pos // block_size]) * block_size + pos % block_size
        last = int(bt[b, pos // block_size])
        k_pool[last, :, pos % block_size:, :] = nan
        v_pool[last, :, pos % block_size:, :] = nan

    return DecodeCase(
        name=name, dtype=dtype, batch=batch, n_q=n_q, n_kv=n_kv, head_dim=head_dim,
        block_size=block_size, num_blocks=num_blocks, scale=1.0 / math.sqrt(head_dim),
        q=q, k_pool=k_pool, v_pool=v_pool,
        block_table=torch.as_tensor(bt, device=device),
        context_lens=torch.as_tensor(ctx.astype(np.int32), device=device),
        new_k=new_k, new_v=new_v,
        slot_mapping=torch.as_tensor(slots, device=device),
        shared_prefix_blocks=n_pref, sharers=sharers, free_blocks=free)


@dataclass
class QuantDecodeCase:
    """A decode step over a quantised cache: one-byte codes and one fp32 scale per row."""

    name: str
    fmt: str                    # "fp8" (OCP E4M3 bit patterns, uint8) or "int8"
    q_dtype: str                # "bf16" or "f16"
    batch: int
    n_q: int
    n_kv: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: torch.Tensor             # [B][n_q][d] in q_dtype
    k_pool: torch.Tensor        # codes [num_blocks][n_kv][bs][d]
    v_pool: torch.Tensor
    k_scale: torch.Tensor       # float32 [num_blocks][n_kv][bs]
    v_scale: torch.Tensor
    block_table: torch.Tensor
    context_lens: torch.Tensor
    new_k: torch.Tensor         # [B][n_kv][d] in q_dtype: the step's new token, unquantised
    new_v: torch.Tensor
    slot_mapping: torch.Tensor
    free_blocks: np.ndarray
    max_blocks_per_seq: int = 0


QUANT_CODE_DTYPES = {"fp8": torch.uint8, "int8": torch.int8}
QUANT_QMAX = {"fp8": 448.0, "int8": 127.0}


def make_quant_decode_case(*, fmt: str, q_dtype: str = "bf16", batch: int, n_q: int, n_kv: int,
                           head_dim: int, context_lens, free_fraction: float = 0.0,
                           num_blocks: int | None = None, max_blocks_per_seq: int | None = None,
                           seed: int = 0, device="cpu", name: str = "quant",
                           row_amax: float = 3.5) -> QuantDecodeCase:
    """Same table, slots and poisoned positions as make_decode_case, with the pools drawn
    directly as codes and scales: codes uniform over the format's finite codes (FP8 E4M3
    without its two NaN patterns, INT8 in [-127, 127]), scales row_amax / QMAX times
    U[0.5, 1.5] (a row of N(0,1) values has |x| max around 3.5). Free blocks and the
    slots past each context hold the FP8 NaN code 0x7F (INT8: -128) and a NaN scale.
    q and the new rows are N(0,1)."""
    if fmt not in QUANT_CODE_DTYPES:
        raise ValueError("fmt must be 'fp8' or 'int8'")
    base = make_decode_case(batch=batch, n_q=n_q, n_kv=n_kv, head_dim=head_dim,
                            context_lens=context_lens, dtype=q_dtype, free_fraction=free_fraction,
                            num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq,
                            seed=seed, device=device, name=name, values=False)
    gen = _gen(device, seed + 7919)
    shape = (base.num_blocks, n_kv, base.block_size, head_dim)

    def codes():
        if fmt == "fp8":
            c = torch.randint(0, 254, shape, generator=gen, device=device, dtype=torch.int32)
            c = c + (c >= 0x7F).to(torch.int32)          # skip 0x7F; 0xFF is never drawn
            return c.to(torch.uint8)
        return torch.randint(-127, 128, shape, generator=gen, device=device, dtype=torch.int32).to(torch.int8)

    def scales():
        u = torch.rand(shape[:3], generator=gen, device=device, dtype=torch.float32)
        return (row_amax / QUANT_QMAX[fmt]) * (0.5 + u)

    k_pool, v_pool = codes(), codes()
    k_scale, v_scale = scales(), scales()
    # Poison the free blocks and, in each sequence's last block, the slots past its
    # context. The new token's row (position ctx - 1) holds a valid code row, so the
    # case decodes as it stands; an append of new_k / new_v overwrites it.
    poison = 0x7F if fmt == "fp8" else -128
    nan = float("nan")
    if base.free_blocks.size:
        idx = torch.as_tensor(base.free_blocks.astype(np.int64), device=device)
        for t in (k_pool, v_pool):
            t[idx] = poison
        for t in (k_scale, v_scale):
            t[idx] = nan
    bs = base.block_size
    for b, ctx in enumerate(base.context_lens.tolist()):
        if ctx == 0:
            continue
        if ctx % bs == 0:
            continue
        last = int(base.block_table[b, (ctx - 1) // bs])
        for t in (k_pool, v_pool):
            t[last, :, ctx % bs:, :] = poison
        for t in (k_scale, v_scale):
            t[last, :, ctx % bs:] = nan
    q = _randn((batch, n_q, head_dim), q_dtype, gen, device)
    new_k = _randn((batch, n_kv, head_dim), q_dtype, gen, device)
    new_v = _randn((batch, n_kv, head_dim), q_dtype, gen, device)
    return QuantDecodeCase(
        name=name, fmt=fmt, q_dtype=q_dtype, batch=batch, n_q=n_q, n_kv=n_kv, head_dim=head_dim,
        block_size=bs, num_blocks=base.num_blocks, scale=base.scale, q=q, k_pool=k_pool,
        v_pool=v_pool, k_scale=k_scale, v_scale=v_scale, block_table=base.block_table,
        context_lens=base.context_lens, new_k=new_k, new_v=new_v, slot_mapping=base.slot_mapping,
        free_blocks=base.free_blocks, max_blocks_per_seq=base.block_table.shape[1])


def make_prefill_case(*, batch: int, seq_len: int, n_q: int, n_kv: int, head_dim: int,
                      dtype: str = "bf16", block_size: int = 16, seed: int = 0, device="cpu",
                      name: str = "custom") -> PrefillCase:
    """Prompt Q/K/V, a permuted pool with room for the prompt plus one token, and a decode step."""
    rng = np.random.default_rng(seed)
    per_seq = (seq_len + 1 + block_size - 1) // block_size
    num_blocks = batch * per_seq
    bt = rng.permutation(num_blocks).astype(np.int32).reshape(batch, per_seq)
    pos = np.arange(seq_len, dtype=np.int64)
    prompt_slots = np.concatenate(
        [bt[b, pos // block_size].astype(np.int64) * block_size + pos % block_size
         for b in range(batch)])
    new_slots = bt[:, seq_len // block_size].astype(np.int64) * block_size + seq_len % block_size

    gen = _gen(device, seed)
    q = _randn((batch, seq_len, n_q, head_dim), dtype, gen, device)
    k = _randn((batch, seq_len, n_kv, head_dim), dtype, gen, device)
    v = _randn((batch, seq_len, n_kv, head_dim), dtype, gen, device)
    q_new = _randn((batch, n_q, head_dim), dtype, gen, device)
    new_k = _randn((batch, n_kv, head_dim), dtype, gen, device)
    new_v = _randn((batch, n_kv, head_dim), dtype, gen, device)
    shape = (num_blocks, n_kv, block_size, head_dim)
    k_pool = torch.full(shape, float("nan"), dtype=TORCH_DTYPES[dtype], device=device)
    v_pool = torch.full(shape, float("nan"), dtype=TORCH_DTYPES[dtype], device=device)
    return PrefillCase(
        name=name, dtype=dtype, batch=batch, seq_len=seq_len, n_q=n_q, n_kv=n_kv,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
        scale=1.0 / math.sqrt(head_dim), q=q, k=k, v=v,
        block_table=torch.as_tensor(bt, device=device),
        prompt_slots=torch.as_tensor(prompt_slots, device=device),
        k_pool=k_pool, v_pool=v_pool, q_new=q_new, new_k=new_k, new_v=new_v,
        new_slots=torch.as_tensor(new_slots, device=device),
        context_lens=torch.full((batch,), seq_len + 1, dtype=torch.int32, device=device))


@dataclass
class ChunkCase:
    """A prompt chunk against a paged prefix: append the chunk's K/V, then attend."""

    name: str
    dtype: str
    batch: int
    chunk_len: int
    n_q: int
    n_kv: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: torch.Tensor             # [B][C][n_q][d]
    k_pool: torch.Tensor        # [num_blocks][n_kv][bs][d], prefixes written, the rest NaN
    v_pool: torch.Tensor
    block_table: torch.Tensor   # int32 [B][max_blocks_per_seq]
    context_lens: torch.Tensor  # int32 [B] = prefix + C
    chunk_k: torch.Tensor       # [B*C][n_kv][d]  K/V of chunk token (b, i) at row b*C + i
    chunk_v: torch.Tensor
    chunk_slots: torch.Tensor   # int64 [B*C]     its slot (position prefix_b + i)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])


def make_chunk_case(*, batch: int, chunk_len: int, prefix_lens, n_q: int, n_kv: int,
                    head_dim: int, dtype: str = "bf16", block_size: int = 16,
                    free_fraction: float = 0.0, seed: int = 0, device="cpu",
                    name: str = "chunk") -> ChunkCase:
    """Paged prefixes of the given lengths plus one chunk of ``chunk_len`` new tokens each.

    Blocks are a seeded permutation of the pool; every slot from a sequence's
    prefix length on, and every free block, holds NaN until the chunk is appended.
    """
    rng = np.random.default_rng(seed)
    pre = np.asarray(prefix_lens, dtype=np.int64).reshape(-1)
    if pre.shape[0] != batch:
        raise ValueError("prefix_lens must have one entry per sequence")
    ctx = pre + chunk_len
    nblk = (ctx + block_size - 1) // block_size
    maxb = max(1, int(nblk.max(initial=0)))
    used = int(nblk.sum())
    num_blocks = max(1, math.ceil(used / (1.0 - free_fraction)))
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.zeros((batch, maxb), dtype=np.int32)
    cursor = 0
    for b in range(batch):
        bt[b, :nblk[b]] = perm[cursor:cursor + nblk[b]]
        cursor += int(nblk[b])
    free = perm[cursor:]
    for b in range(batch):
        if maxb > nblk[b]:
            bt[b, nblk[b]:] = rng.choice(free, size=maxb - nblk[b]) if free.size else 0

    gen = _gen(device, seed)
    shape = (num_blocks, n_kv, block_size, head_dim)
    k_pool = _randn(shape, dtype, gen, device)
    v_pool = _randn(shape, dtype, gen, device)
    q = _randn((batch, chunk_len, n_q, head_dim), dtype, gen, device)
    chunk_k = _randn((batch * chunk_len, n_kv, head_dim), dtype, gen, device)
    chunk_v = _randn((batch * chunk_len, n_kv, head_dim), dtype, gen, device)
    nan = float("nan")
    if free.size:
        idx = torch.as_tensor(free.astype(np.int64), device=device)
        k_pool[idx] = nan
        v_pool[idx] = nan
    slots = np.zeros(batch * chunk_len, dtype=np.int64)
    for b in range(batch):
        for t in range(int(pre[b]), int(ctx[b])):
            blk = int(bt[b, t // block_size])
            k_pool[blk, :, t % block_size, :] = nan
            v_pool[blk, :, t % block_size, :] = nan
            slots[b * chunk_len + t - int(pre[b])] = blk * block_size + t % block_size
        last = int(ctx[b]) - 1 if ctx[b] > 0 else -1
        if last >= 0 and (last + 1) % block_size:
            blk = int(bt[b, last // block_size])
            k_pool[blk, :, (last + 1) % block_size:, :] = nan
            v_pool[blk, :, (last + 1) % block_size:, :] = nan
    return ChunkCase(
        name=name, dtype=dtype, batch=batch, chunk_len=chunk_len, n_q=n_q, n_kv=n_kv,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
        scale=1.0 / math.sqrt(head_dim), q=q, k_pool=k_pool, v_pool=v_pool,
        block_table=torch.as_tensor(bt, device=device),
        context_lens=torch.as_tensor(ctx.astype(np.int32), device=device),
        chunk_k=chunk_k, chunk_v=chunk_v, chunk_slots=torch.as_tensor(slots, device=device))


# ---- the five named workloads -------------------------------------------------

CONFIG_SEEDS = {1: 1001, 2: 1002, 3: 1003, 4: 1004, 5: 1005}

CONFIG_NAMES = {
    1: "tiny_paged_decode_fp32",
    2: "llama3_8b_decode_b32_ctx2048",
    3: "varlen_decode_b64_ctx128_8192_shared_prefix",
    4: "llama3_70b_decode_b8_ctx32768",
    5: "causal_prefill_b2_s4096_then_decode",
}


# Sliding-window decode: the decode_8b shape over 16384-token contexts, each query
# restricted to its last WINDOW_TOKENS positions.
WINDOW_TOKENS = 4096
WINDOW_CASE_NAME = "sliding_window_decode_b32_ctx16384_w4096"
WINDOW_CASE_SEED = 1008


def make_window_decode_case(device="cpu", seed: int | None = None, values: bool = True):
    """B=32, n_q=32, n_kv=8, d=128, bf16, every context 16384; attend with window=WINDOW_TOKENS."""
    return make_decode_case(batch=32, n_q=32, n_kv=8, head_dim=128, context_lens=[16384] * 32,
                            dtype="bf16", seed=WINDOW_CASE_SEED if seed is None else seed,
                            device=device, name=WINDOW_CASE_NAME, values=values)


def varlen_context_lens(seed: int, batch: int = 64, lo: int = 128, hi: int = 8192) -> np.ndarray:
    """Context lengths drawn uniformly from the integers [lo, hi]."""
    return np.random.default_rng(seed + 7).integers(lo, hi + 1, size=batch)


def make_config(i: int, device="cpu", seed: int | None = None, values: bool = True):
    """Named workload ``i`` (1..5) with its fixed seed, or ``seed`` to draw another set.

    ``values=False`` (decode configs only) keeps the structure and zero-fills the tensors.
    """
    s = CONFIG_SEEDS[i] if seed is None else seed
    name = CONFIG_NAMES[i]
    kw = dict(seed=s, device=device, name=name, values=values)
    if i == 1:
        # B=2, contexts {7, 33}, n_q=4, n_kv=2, d=64, fp32, 16-block pool (4 used, 12 free).
        return make_decode_case(batch=2, n_q=4, n_kv=2, head_dim=64, context_lens=[7, 33],
                                dtype="f32", num_blocks=16, **kw)
    if i == 2:
        # B=32, n_q=32, n_kv=8, d=128, every context 2048, pool sized exactly (4096 blocks).
        return make_decode_case(batch=32, n_q=32, n_kv=8, head_dim=128,
                                context_lens=[2048] * 32, dtype="bf16", **kw)
    if i == 3:
        # B=64, contexts U[128, 8192]; 16 of 64 sequences share a 1024-token (64-block) prefix;
        # 20% of the pool is free.
        ctx = varlen_context_lens(s)
        return make_decode_case(batch=64, n_q=32, n_kv=8, head_dim=128, context_lens=ctx,
                                dtype="bf16", free_fraction=0.2, max_blocks_per_seq=512,
                                shared_prefix_blocks=64, n_sharers=16, **kw)
    if i == 4:
        # B=8, n_q=64, n_kv=8 (G=8), d=128, every context 32768 (1 GiB of KV).
        return make_decode_case(batch=8, n_q=64, n_kv=8, head_dim=128,
                                context_lens=[32768] * 8, dtype="bf16", **kw)
    if i == 5:
        return make_prefill_case(batch=2, seq_len=4096, n_q=32, n_kv=8, head_dim=128,
                                 dtype="bf16", seed=s, device=device, name=name)
    raise ValueError(f"unknown config {i}")
