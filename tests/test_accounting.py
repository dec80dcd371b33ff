"""Byte and FLOP accounting against the figures the pages print."""
import json
from pathlib import Path

import pytest

from paged_gqa_attention_attn_amd import accounting as acc

FX = json.loads((Path(__file__).parent / "golden" / "kv_bytes_from_pages.json").read_text())


@pytest.mark.parametrize("case", FX["cases"], ids=lambda c: c["what"])
def test_kv_cache_bytes_matches_pages(case):
    n = acc.kv_cache_bytes(case["layers"], case["tokens"], case["n_kv"], case["head_dim"],
                           case["elem_bytes"])
    if "bytes" in case:
        assert n == case["bytes"]
    if "mib" in case:
        assert n == case["mib"] * 2**20
    if "gib" in case:
        assert n == case["gib"] * 2**30


def test_decode_kv_read_matches_pages():
    c = FX["decode_read"]
    assert acc.decode_kv_bytes([c["ctx"]], c["n_kv"], c["head_dim"], c["elem_bytes"]) == c["mib"] * 2**20


def test_decode_flops_matches_pages():
    c = FX["decode_qk_flops"]
    one = c["flops_one_matmul"]
    assert round(one / 1e6, 1) == c["printed_mflops"]
    assert acc.decode_flops([c["ctx"]], c["n_q"], c["head_dim"]) == 2 * one


def test_prefill_full_square_flops_matches_pages():
    c = FX["prefill_qk_flops"]
    one = c["flops_one_matmul"]
    assert round(one / 1e9, 1) == c["printed_gflops"]
    assert acc.prefill_flops_full_square(c["batch"], c["seq_len"], c["n_q"], c["head_dim"]) == 2 * one


def test_causal_flops_is_lower_triangle():
    # S(S+1)/2 query-key pairs per head: for S=1 one pair, for S=2 three pairs.
    assert acc.prefill_flops_causal(1, 1, 1, 1) == 4
    assert acc.prefill_flops_causal(1, 2, 1, 1) == 12
    assert acc.prefill_flops_causal(2, 4096, 32, 128) == 274_945_015_808


def test_config_byte_totals():
    # 8B-shaped decode: 32 sequences x 2048 tokens x 4096 B per token.
    assert acc.decode_kv_bytes([2048] * 32, 8, 128, 2) == 268_435_456
    # 70B-shaped long context: 1 GiB of KV.
    assert acc.decode_kv_bytes([32768] * 8, 8, 128, 2) == 2**30
    assert acc.decode_unique_kv_bytes([2000] * 4, 8, 128, 2, 1024, 4) == \
        acc.decode_kv_bytes([2000] * 4, 8, 128, 2) - 3 * 1024 * 4096


def test_chunked_prefill_flops():
    # A chunk that is the whole prompt is a causal prefill.
    assert acc.chunked_prefill_flops([4096, 4096], 4096, 32, 128) == acc.prefill_flops_causal(2, 4096, 32, 128)
    # ctx 5, chunk 2: rows at positions 3 and 4 see 4 and 5 keys -> 9 (q, k) pairs.
    assert acc.chunked_prefill_flops([5], 2, 1, 1) == 4 * 9
    # ctx 2, chunk 4: rows at positions -2, -1 see nothing; 0 and 1 see 1 and 2 keys.
    assert acc.chunked_prefill_flops([2], 4, 1, 1) == 4 * 3


def test_windowed_decode_bytes_and_flops():
    # Window 4096 over 16384-token contexts reads a quarter of the cache; a window wider
    # than the context changes nothing.
    assert acc.decode_kv_bytes([16384] * 32, 8, 128, 2, window=4096) == 32 * 4096 * 4096   # 512 MiB
    assert acc.decode_kv_bytes([100, 5000], 8, 128, 2, window=4096) == (100 + 4096) * 4096
    assert acc.decode_flops([16384], 32, 128, window=4096) == acc.decode_flops([4096], 32, 128)
    assert acc.decode_flops([10], 1, 1, window=0) == 40


def test_quant_bytes_are_one_byte_codes_plus_row_scales():
    # The pages count FP8 as one byte per element; each row adds its fp32 scale.
    ctx = [2048] * 32
    codes = acc.decode_kv_bytes(ctx, 8, 128, acc.ELEM_BYTES["fp8"])
    assert codes == 134_217_728
    assert acc.quant_decode_kv_bytes(ctx, 8, 128) == codes + 2 * 32 * 2048 * 8 * 4
    assert acc.quant_decode_kv_bytes([100, 5000], 2, 64, window=300) == 2 * (100 + 300) * 2 * (64 + 4)
