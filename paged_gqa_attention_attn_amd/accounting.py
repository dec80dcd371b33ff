"""Algorithmic byte and FLOP counts: the denominators of every GB/s and TFLOP/s figure.

Only the work the method must do is counted: every K/V byte of the attended
context read once, q read once, the output written once. Partial-result
traffic of a split context is implementation overhead and is not counted.

Closed forms from the pages:
  * KV cache size = 2 * layers * tokens * n_kv * head_dim * bytes_per_elem
    (xinc.fun/index.php/archives/233, section 4 "MHA、MQA、GQA 与 MLA"; the
    vLLM concepts page, yyzxw.github.io, per-request KV cache formula and its
    LLaMA3-70B worked value).
  * attention FLOPs per matmul = 2 * n_q * L_q * L_k * d per sequence
    ("LLM 推理全过程的维度变化与核心公式", research.frankk.site, table
    "每层每步的计算 / 内存读写", rows Attn QK^T and Attn·V).
"""
from __future__ import annotations

from typing import Iterable

ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1, "int8": 1}
SCALE_BYTES = 4   # one fp32 scale per (token, KV head) row of a quantised cache


def kv_cache_bytes(layers: int, tokens: int, n_kv: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of K plus V for ``tokens`` positions over ``layers`` layers."""
    return 2 * layers * tokens * n_kv * head_dim * elem_bytes


def attended(ctx: int, window: int = 0) -> int:
    """Positions one decode query attends to: all ctx, or the last ``window`` of them."""
    return min(int(ctx), window) if window > 0 else int(ctx)


def decode_kv_bytes(context_lens: Iterable[int], n_kv: int, head_dim: int, elem_bytes: int,
                    window: int = 0) -> int:
    """K/V bytes one decode step must read: every attended position, every KV head, once."""
    return sum(kv_cache_bytes(1, attended(c, window), n_kv, head_dim, elem_bytes)
               for c in context_lens)


def quant_decode_kv_bytes(context_lens: Iterable[int], n_kv: int, head_dim: int,
                          window: int = 0) -> int:
    """Bytes one decode step reads from a one-byte (FP8 / INT8) cache: the codes of every
    attended K and V row (the pages' one byte per element) plus each row's fp32 scale."""
    return sum(2 * attended(c, window) * n_kv * (head_dim + SCALE_BYTES) for c in context_lens)


def decode_unique_kv_bytes(context_lens: Iterable[int], n_kv: int, head_dim: int,
                           elem_bytes: int, shared_prefix_tokens: int = 0,
                           n_sharers: int = 0) -> int:
    """K/V bytes counting a prefix shared by ``n_sharers`` sequences once rather than per sharer."""
    dup = max(0, n_sharers - 1) * kv_cache_bytes(1, shared_prefix_tokens, n_kv, head_dim,
                                                 elem_bytes)
    return decode_kv_bytes(context_lens, n_kv, head_dim, elem_bytes) - dup


def decode_io_bytes(batch: int, n_q: int, head_dim: int, elem_bytes: int, out_bytes: int,
                    max_blocks_per_seq: int) -> int:
    """q read + output write + block table + context lengths of one decode step."""
    return (batch * n_q * head_dim * (elem_bytes + out_bytes) + batch * max_blocks_per_seq * 4
            + batch * 4)


def decode_flops(context_lens: Iterable[int], n_q: int, head_dim: int, window: int = 0) -> int:
    """QK^T plus PV: 2 * 2 * n_q * ctx * d per sequence (one query row)."""
    return sum(4 * n_q * attended(c, window) * head_dim for c in context_lens)


def prefill_flops_causal(batch: int, seq_len: int, n_q: int, head_dim: int) -> int:
    """QK^T plus PV over the causal lower triangle, diagonal included: S(S+1)/2 pairs per head."""
    return 4 * batch * n_q * head_dim * (seq_len * (seq_len + 1) // 2)


def chunked_prefill_flops(context_lens, chunk_len: int, n_q: int, head_dim: int) -> int:
    """QK^T plus PV for a chunk of C rows at positions ctx-C .. ctx-1: row at position p sees p+1 keys."""
    total = 0
    for ctx in context_lens:
        ctx = int(ctx)
        first = max(0, ctx - chunk_len)                  # keys seen by the first row, minus one
        rows = ctx - first
        total += rows * (first + 1) + rows * (rows - 1) // 2
    return 4 * n_q * head_dim * total


def prefill_flops_full_square(batch: int, seq_len: int, n_q: int, head_dim: int) -> int:
    """The pages' convention: 2 * B * n_q * S * S * d per matmul, both matmuls."""
    return 2 * 2 * batch * n_q * seq_len * seq_len * head_dim


def prefill_io_bytes(batch: int, seq_len: int, n_q: int, n_kv: int, head_dim: int,
                     elem_bytes: int, out_bytes: int) -> int:
    """Q, K, V read once and O written once."""
    return batch * seq_len * head_dim * ((n_q + 2 * n_kv) * elem_bytes + n_q * out_bytes)


def kv_append_bytes(num_tokens: int, n_kv: int, head_dim: int, elem_bytes: int) -> int:
    """K and V rows read from the inputs and written to the pools, plus the int64 slots."""
    return 2 * 2 * num_tokens * n_kv * head_dim * elem_bytes + 8 * num_tokens
