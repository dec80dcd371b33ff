"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented codes before any HIP call.

Only error paths and pure host queries are called here: fake device pointers
are never dereferenced because validation fails first.
"""
import ctypes
import re
from pathlib import Path

import pytest

from paged_gqa_attention_attn_amd import _lib

HEADER = Path(__file__).resolve().parent.parent / "include" / "pagedattn.h"

PA_OK, INVALID, UNSUPPORTED = _lib.PA_OK, _lib.PA_ERR_INVALID_ARG, _lib.PA_ERR_UNSUPPORTED
FAKE = 1 << 20          # a 16-byte aligned fake device address (never dereferenced)
MISALIGNED = FAKE + 8


@pytest.fixture(scope="module")
def L():
    if not _lib.LIB_PATH.exists():
        pytest.skip("libpagedattn.so not built")
    return _lib.load()


def desc(nb=64, bs=16, n_kv=2, d=128, dtype=_lib.PA_BF16):
    return ctypes.byref(_lib.CacheDesc(nb, bs, n_kv, d, dtype))


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_and_exports_agree(L):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"


def test_version(L):
    assert L.pa_version() == 301


def test_options_set_get_and_ranges(L):
    ranges = {"decode_matrix_cores": (0, 1), "decode_ring": (1, 2), "decode_waves": (0, 8),
              "prefill_stage_v": (0, 1), "validate": (0, 1)}
    assert set(ranges) == set(_lib.OPTIONS)
    assert L.pa_get_option(-1) == -1 and L.pa_get_option(len(ranges)) == -1
    assert L.pa_set_option(len(ranges), 0) == -1
    for name, (lo, hi) in ranges.items():
        o = _lib.OPTIONS[name][0]
        start = L.pa_get_option(o)
        assert lo <= start <= hi
        assert L.pa_set_option(o, lo - 1) == -1 and L.pa_set_option(o, hi + 1) == -1
        assert L.pa_get_option(o) == start            # a rejected value changes nothing
        assert L.pa_set_option(o, hi) == start
        assert L.pa_set_option(o, lo) == hi
        assert L.pa_get_option(o) == lo
        assert L.pa_set_option(o, start) == lo


def test_options_start_from_the_environment():
    """Each option's first value comes from its variable; bad values give the default."""
    import os
    import subprocess
    import sys
    if not _lib.LIB_PATH.exists():
        pytest.skip("libpagedattn.so not built")
    env = dict(os.environ, PA_DECODE_MFMA="0", PA_DECODE_RING="2", PA_DECODE_WAVES="9",
               PA_PREFILL_STAGE_V="x", PA_VALIDATE="1")
    code = ("from paged_gqa_attention_attn_amd import _lib; L = _lib.load(); "
            "print([L.pa_get_option(i) for i in range(5)])")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True,
                         cwd=Path(__file__).resolve().parent.parent).stdout.strip()
    assert out == "[0, 2, 0, 1, 1]"


def decode(L, **kw):
    a = dict(q=FAKE, batch=2, n_q=8, k=FAKE, v=FAKE, cache=desc(), bt=FAKE, maxb=4, ctx=FAKE,
             scale=0.125, window=0, alibi=None, out=FAKE, out_dtype=_lib.PA_F32, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.pa_paged_attn_decode(a["q"], a["batch"], a["n_q"], a["k"], a["v"], a["cache"],
                                  a["bt"], a["maxb"], a["ctx"], a["scale"], a["window"], a["alibi"], a["out"],
                                  a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(cache=None), INVALID, "descriptor"),
    (dict(cache=desc(bs=8)), UNSUPPORTED, "block_size"),
    (dict(cache=desc(d=96)), UNSUPPORTED, "head_dim"),
    (dict(cache=desc(dtype=7)), UNSUPPORTED, "dtype"),
    (dict(cache=desc(nb=0)), INVALID, "positive"),
    (dict(n_q=7), INVALID, "multiple"),
    (dict(n_q=0), INVALID, "n_q"),
    (dict(batch=-1), INVALID, "batch"),
    (dict(maxb=0), INVALID, "max_blocks"),
    (dict(q=None), INVALID, "NULL"),
    (dict(out=MISALIGNED), INVALID, "aligned"),
    (dict(bt=FAKE + 2), INVALID, "aligned"),
    (dict(out_dtype=_lib.PA_F16), UNSUPPORTED, "out_dtype"),
    (dict(scale=float("nan")), INVALID, "finite"),
    (dict(scale=float("inf")), INVALID, "finite"),
    (dict(scale=float("-inf")), INVALID, "finite"),
    (dict(window=-1), INVALID, "window"),
    (dict(maxb=8192, ws=FAKE, ws_bytes=16), INVALID, "workspace"),   # too small (NULL: library's own)
    (dict(maxb=8192, window=4096, ws=FAKE, ws_bytes=16), INVALID, "workspace"),
    (dict(alibi=FAKE + 2), INVALID, "alibi_slopes"),
])
def test_decode_rejects(L, kw, code, msg):
    assert decode(L, **kw) == code
    assert msg in _lib.last_error()


def test_decode_empty_batch_is_a_noop(L):
    assert decode(L, batch=0) == PA_OK


def decode_append(L, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, slots=FAKE, batch=2, n_q=8, k=FAKE, v=FAKE, cache=desc(),
             bt=FAKE, maxb=4, ctx=FAKE, scale=0.125, window=0, alibi=None, out=FAKE, out_dtype=_lib.PA_F32,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.pa_paged_attn_decode_append(a["q"], a["kn"], a["vn"], a["slots"], a["batch"],
                                         a["n_q"], a["k"], a["v"], a["cache"], a["bt"], a["maxb"],
                                         a["ctx"], a["scale"], a["window"], a["alibi"], a["out"], a["out_dtype"], a["ws"],
                                         a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(kn=None), INVALID, "k_new"),
    (dict(slots=None), INVALID, "slot_mapping"),
    (dict(vn=MISALIGNED), INVALID, "aligned"),
    (dict(slots=FAKE + 4), INVALID, "aligned"),
    (dict(cache=desc(bs=32)), UNSUPPORTED, "block_size"),
    (dict(n_q=5), INVALID, "multiple"),
    (dict(window=-3), INVALID, "window"),
    (dict(alibi=FAKE + 2), INVALID, "alibi_slopes"),
])
def test_decode_append_rejects(L, kw, code, msg):
    assert decode_append(L, **kw) == code
    assert msg in _lib.last_error()


def test_workspace_query(L):
    # VALU kernel (fp32 cache): 2048-token partitions, so a 2048-token context
    # needs no workspace and 4096-token contexts need (m, l, acc) for 2
    # partitions of every query head.
    f32 = _lib.PA_F32
    assert L.pa_decode_workspace_bytes(32, 32, 128, desc(nb=4096, n_kv=8, dtype=f32)) == 0
    n = L.pa_decode_workspace_bytes(32, 32, 256, desc(nb=8192, n_kv=8, dtype=f32))
    rows = 32 * 32 * 2
    assert n == 2 * rows * 4 + rows * 128 * 4
    # Matrix-core kernel (bf16, groups of 4/8/16): about 2048 waves of up to 64
    # blocks each. 32 x 8 (sequence, KV head) units over 4096 tokens fit one
    # partition of 8 waves x 32 blocks; 8 x 8 units over 32768 tokens take 4
    # partitions of 8 waves x 64 blocks.
    assert L.pa_decode_workspace_bytes(32, 32, 256, desc(nb=8192, n_kv=8)) == 0
    n = L.pa_decode_workspace_bytes(8, 64, 2048, desc(nb=16384, n_kv=8))
    rows = 8 * 64 * 4
    assert n == 2 * rows * 4 + rows * 128 * 4
    assert L.pa_decode_workspace_bytes(2, 7, 4, desc()) == 0      # invalid: 7 % 2 != 0


def test_partition_override(L):
    assert L.pa_set_decode_partition_tokens(17) == -1
    assert L.pa_set_decode_partition_tokens(-16) == -1
    prev = L.pa_set_decode_partition_tokens(256)
    try:
        assert L.pa_decode_workspace_bytes(1, 8, 64, desc()) > 0    # 1024 tokens / 256
    finally:
        assert L.pa_set_decode_partition_tokens(prev) == 256


def test_set_workspace_rejects(L):
    assert L.pa_set_workspace(None, 16) == INVALID
    assert "NULL" in _lib.last_error()
    assert L.pa_set_workspace(MISALIGNED, 1 << 20) == INVALID
    assert "aligned" in _lib.last_error()
    assert L.pa_set_workspace(None, 0) == PA_OK


def append(L, **kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, T=4, kc=FAKE, vc=FAKE, cache=desc(), stream=None)
    a.update(kw)
    return L.pa_kv_append(a["k"], a["v"], a["slots"], a["T"], a["kc"], a["vc"], a["cache"],
                          a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cache=None), INVALID),
    (dict(cache=desc(bs=32)), UNSUPPORTED),
    (dict(T=-1), INVALID),
    (dict(v=None), INVALID),
    (dict(kc=MISALIGNED), INVALID),
    (dict(slots=FAKE + 4), INVALID),
])
def test_append_rejects(L, kw, code):
    assert append(L, **kw) == code


def test_append_zero_tokens_is_a_noop(L):
    assert append(L, T=0) == PA_OK


def prefill(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=_lib.PA_BF16, B=1, S=64, n_q=8, n_kv=2, d=128,
             causal=1, scale=0.1, window=0, alibi=None, out=FAKE, out_dtype=_lib.PA_F32, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return L.pa_paged_attn_prefill(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["S"], a["n_q"],
                                   a["n_kv"], a["d"], a["causal"], a["scale"], a["window"], a["alibi"], a["out"],
                                   a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=_lib.PA_FP8_E4M3), UNSUPPORTED),
    (dict(dtype=_lib.PA_F32, d=80), UNSUPPORTED),
    (dict(dtype=_lib.PA_F32, out_dtype=_lib.PA_BF16), UNSUPPORTED),
    (dict(dtype=_lib.PA_F32, S=2**30), UNSUPPORTED),              # rows * group past an int
    (dict(dtype=_lib.PA_F32, n_q=65536, n_kv=65536), UNSUPPORTED),  # KV heads past grid y
    (dict(d=80), UNSUPPORTED),
    (dict(n_q=6, n_kv=4), INVALID),
    (dict(causal=2), INVALID),
    (dict(S=-1), INVALID),
    (dict(out=None), INVALID),
    (dict(k=MISALIGNED), INVALID),
    (dict(out_dtype=_lib.PA_F16), UNSUPPORTED),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("-inf")), INVALID),
    (dict(window=-1), INVALID),
    (dict(window=8, causal=0), INVALID),    # a window is a causal band
    (dict(alibi=FAKE + 2), INVALID),
    (dict(alibi=FAKE, causal=0), INVALID),  # the bias is defined for causal attention
    (dict(S=2**31 - 1, n_q=64, n_kv=8, B=4), UNSUPPORTED),   # 2^32 workgroups in one grid
    (dict(S=2**31 - 100), UNSUPPORTED),                       # rows too close to the int limit
])
def test_prefill_rejects(L, kw, code):
    assert prefill(L, **kw) == code


def test_prefill_workspace_bytes(L, option):
    # bf16: an f16 copy of v ([B][S][n_kv][d], 2 bytes each), then one flag byte per
    # (sequence, KV head, 64-key tile), each part rounded up to 16 bytes.
    assert L.pa_prefill_workspace_bytes(_lib.PA_BF16, 2, 4096, 8, 128) == 2 * 4096 * 8 * 128 * 2 + 1024
    assert L.pa_prefill_workspace_bytes(_lib.PA_BF16, 1, 65, 1, 64) == 65 * 64 * 2 + 16
    assert L.pa_prefill_workspace_bytes(_lib.PA_F16, 2, 4096, 8, 128) == 0
    assert L.pa_prefill_workspace_bytes(_lib.PA_BF16, 0, 4096, 8, 128) == 0
    option("prefill_stage_v", 0)
    assert L.pa_prefill_workspace_bytes(_lib.PA_BF16, 2, 4096, 8, 128) == 0


def test_prefill_rejects_small_or_misaligned_workspace(L):
    need = L.pa_prefill_workspace_bytes(_lib.PA_BF16, 1, 64, 2, 128)
    assert prefill(L, ws=FAKE, ws_bytes=need - 1) == INVALID
    assert "workspace" in _lib.last_error()
    assert prefill(L, ws=FAKE + 8, ws_bytes=need) == INVALID
    assert "aligned" in _lib.last_error()


def test_prefill_empty_is_a_noop(L):
    assert prefill(L, S=0) == PA_OK
    assert prefill(L, B=0) == PA_OK


def chunked(L, **kw):
    a = dict(q=FAKE, B=2, C=16, n_q=8, k=FAKE, v=FAKE, cache=desc(), bt=FAKE, maxb=4, ctx=FAKE,
             scale=0.125, window=0, alibi=None, out=FAKE, out_dtype=_lib.PA_F32, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return L.pa_paged_attn_chunked_prefill(a["q"], a["B"], a["C"], a["n_q"], a["k"], a["v"],
                                           a["cache"], a["bt"], a["maxb"], a["ctx"], a["scale"],
                                           a["window"], a["alibi"], a["out"], a["out_dtype"], a["ws"],
                                           a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(cache=None), INVALID, "descriptor"),
    (dict(cache=desc(dtype=_lib.PA_INT8)), UNSUPPORTED, "quantised"),
    (dict(cache=desc(dtype=_lib.PA_F32), out_dtype=_lib.PA_BF16), UNSUPPORTED, "out_dtype"),
    (dict(cache=desc(dtype=_lib.PA_F32, n_kv=8), C=2**30, n_q=64), UNSUPPORTED, "grid"),
    (dict(cache=desc(d=96)), UNSUPPORTED, "head_dim"),
    (dict(C=-1), INVALID, "chunk_len"),
    (dict(n_q=7), INVALID, "multiple"),
    (dict(scale=float("inf")), INVALID, "finite"),
    (dict(q=None), INVALID, "NULL"),
    (dict(out=MISALIGNED), INVALID, "aligned"),
    (dict(ctx=FAKE + 2), INVALID, "aligned"),
    (dict(out_dtype=_lib.PA_F16), UNSUPPORTED, "out_dtype"),
    (dict(window=-1), INVALID, "window"),
    (dict(alibi=FAKE + 2), INVALID, "alibi_slopes"),
    (dict(C=2**31 - 1, n_q=64, cache=desc(n_kv=8), B=4), UNSUPPORTED, "exceeds one launch"),
])
def test_chunked_prefill_rejects(L, kw, code, msg):
    assert chunked(L, **kw) == code
    assert msg in _lib.last_error()


def test_f32_paths_take_no_workspace(L):
    f32 = desc(nb=4096, n_kv=8, dtype=_lib.PA_F32)
    assert L.pa_prefill_workspace_bytes(_lib.PA_F32, 2, 4096, 8, 128) == 0
    assert L.pa_chunked_prefill_workspace_bytes(2, 256, f32) == 0
    assert L.pa_decode_multi_workspace_bytes(4, 4, 64, 256, f32) == 0


def test_chunked_prefill_empty_is_a_noop(L):
    assert chunked(L, C=0) == PA_OK
    assert chunked(L, B=0) == PA_OK


def test_chunked_prefill_workspace(L, option):
    # bf16: an f16 copy of the V blocks the call may read ([B][max_blocks][n_kv][16][d]),
    # then one flag byte per (sequence, KV head, block), each part rounded up to 16 bytes;
    # nothing past 256 MiB, nothing for f16 caches or with PA_PREFILL_STAGE_V=0.
    assert L.pa_chunked_prefill_workspace_bytes(2, 256, desc(n_kv=8)) == 2 * 256 * 8 * 16 * 128 * 2 + 4096
    assert L.pa_chunked_prefill_workspace_bytes(1, 3, desc(n_kv=1, d=64)) == 3 * 16 * 64 * 2 + 16
    assert L.pa_chunked_prefill_workspace_bytes(64, 8192, desc(n_kv=8)) == 0
    assert L.pa_chunked_prefill_workspace_bytes(2, 256, desc(n_kv=8, dtype=_lib.PA_F16)) == 0
    assert L.pa_chunked_prefill_workspace_bytes(0, 256, desc()) == 0
    need = L.pa_chunked_prefill_workspace_bytes(2, 4, desc())
    assert chunked(L, ws=FAKE, ws_bytes=need - 1) == INVALID
    assert "workspace" in _lib.last_error()
    assert chunked(L, ws=FAKE + 8, ws_bytes=need) == INVALID
    assert "aligned" in _lib.last_error()
    option("prefill_stage_v", 0)
    assert L.pa_chunked_prefill_workspace_bytes(2, 256, desc(n_kv=8)) == 0


def multi(L, **kw):
    a = dict(q=FAKE, B=2, R=4, n_q=8, k=FAKE, v=FAKE, cache=desc(), bt=FAKE, maxb=4, ctx=FAKE,
             scale=0.125, window=0, alibi=None, out=FAKE, out_dtype=_lib.PA_F32, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.pa_paged_attn_decode_multi(a["q"], a["B"], a["R"], a["n_q"], a["k"], a["v"], a["cache"],
                                        a["bt"], a["maxb"], a["ctx"], a["scale"], a["window"], a["alibi"], a["out"],
                                        a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(cache=None), INVALID, "descriptor"),
    (dict(cache=desc(dtype=_lib.PA_FP8_E4M3)), UNSUPPORTED, "quantised"),
    (dict(cache=desc(dtype=_lib.PA_F32), out_dtype=_lib.PA_F16), UNSUPPORTED, "out_dtype"),
    (dict(cache=desc(dtype=_lib.PA_F32), R=2**29, n_q=64), UNSUPPORTED, "grid"),
    (dict(R=0), INVALID, "q_rows"),
    (dict(n_q=7), INVALID, "multiple"),
    (dict(scale=float("nan")), INVALID, "finite"),
    (dict(v=None), INVALID, "NULL"),
    (dict(q=MISALIGNED), INVALID, "aligned"),
    (dict(maxb=8192, ws=FAKE, ws_bytes=16), INVALID, "workspace"),
    (dict(maxb=8192, window=4096, ws=FAKE, ws_bytes=16), INVALID, "workspace"),
    (dict(window=-1), INVALID, "window"),
    (dict(alibi=FAKE + 2), INVALID, "alibi_slopes"),
])
def test_decode_multi_rejects(L, kw, code, msg):
    assert multi(L, **kw) == code
    assert msg in _lib.last_error()


def _partials(rows):
    return 2 * rows * 4 + rows * 128 * 4   # m and l (fp32 each), then acc [rows][128]


def test_decode_multi_workspace_query(L, option):
    # Multi-row kernel (G * q_rows = 8 * 4 = 32 (head, row) pairs): 2048-token partitions,
    # so 4096-token contexts need (m, l, acc) for 2 partitions of every (sequence, row, head).
    assert L.pa_decode_multi_workspace_bytes(4, 4, 64, 128, desc(nb=4096, n_kv=8)) == 0
    assert L.pa_decode_multi_workspace_bytes(4, 4, 64, 256, desc(nb=4096, n_kv=8)) == _partials(4 * 4 * 64 * 2)
    # 16 pairs go to the matrix-core decode kernel: 8-wave workgroups over 32
    # (sequence, KV head) units take 4 partitions of a 128-block table ...
    assert L.pa_decode_multi_workspace_bytes(4, 4, 32, 128, desc(nb=4096, n_kv=8)) == _partials(4 * 4 * 32 * 4)
    # ... unless that kernel is turned off.
    option("decode_matrix_cores", 0)
    assert L.pa_decode_multi_workspace_bytes(4, 4, 32, 128, desc(nb=4096, n_kv=8)) == 0
    assert L.pa_decode_multi_workspace_bytes(4, 4, 32, 256, desc(nb=4096, n_kv=8)) == _partials(4 * 4 * 32 * 2)
    assert L.pa_decode_multi_workspace_bytes(4, 0, 32, 256, desc(nb=4096, n_kv=8)) == 0
    assert multi(L, B=0) == PA_OK


# ---- quantised cache entry points --------------------------------------------------------

FP8, INT8 = _lib.PA_FP8_E4M3, _lib.PA_INT8


def decode_quant(L, **kw):
    a = dict(q=FAKE, q_dtype=_lib.PA_BF16, batch=2, n_q=8, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE,
             cache=desc(dtype=FP8), bt=FAKE, maxb=4, ctx=FAKE, scale=0.125, window=0, alibi=None, out=FAKE,
             out_dtype=_lib.PA_F32, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.pa_paged_attn_decode_quant(a["q"], a["q_dtype"], a["batch"], a["n_q"], a["k"], a["v"],
                                        a["ks"], a["vs"], a["cache"], a["bt"], a["maxb"], a["ctx"],
                                        a["scale"], a["window"], a["alibi"], a["out"], a["out_dtype"], a["ws"],
                                        a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(cache=desc(dtype=_lib.PA_BF16)), INVALID, "PA_FP8_E4M3"),
    (dict(q_dtype=_lib.PA_F32), UNSUPPORTED, "q must be"),
    (dict(out_dtype=_lib.PA_F16), UNSUPPORTED, "out_dtype"),
    (dict(ks=None), INVALID, "NULL"),
    (dict(vs=FAKE + 4), INVALID, "aligned"),
    (dict(cache=desc(dtype=INT8, d=96)), UNSUPPORTED, "head_dim"),
    (dict(n_q=7), INVALID, "multiple"),
    (dict(scale=float("nan")), INVALID, "finite"),
    (dict(window=-2), INVALID, "window"),
    (dict(alibi=FAKE + 2), INVALID, "alibi_slopes"),
])
def test_decode_quant_rejects(L, kw, code, msg):
    assert decode_quant(L, **kw) == code
    assert msg in _lib.last_error()


def rows_quant(L, name, **kw):
    a = dict(q=FAKE, q_dtype=_lib.PA_BF16, batch=2, rows=4, n_q=8, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE,
             cache=desc(dtype=FP8), bt=FAKE, maxb=4, ctx=FAKE, scale=0.125, window=0, alibi=None, out=FAKE,
             out_dtype=_lib.PA_F32, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return getattr(L, name)(a["q"], a["q_dtype"], a["batch"], a["rows"], a["n_q"], a["k"], a["v"], a["ks"],
                            a["vs"], a["cache"], a["bt"], a["maxb"], a["ctx"], a["scale"], a["window"], a["alibi"],
                            a["out"], a["out_dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("name", ["pa_paged_attn_decode_multi_quant", "pa_paged_attn_chunked_prefill_quant"])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(cache=desc(dtype=_lib.PA_BF16)), INVALID, "PA_FP8_E4M3"),
    (dict(q_dtype=_lib.PA_F32), UNSUPPORTED, "q must be"),
    (dict(out_dtype=_lib.PA_F16), UNSUPPORTED, "out_dtype"),
    (dict(rows=-1), INVALID, "must be positive"),
    (dict(ks=None), INVALID, "NULL"),
    (dict(cache=desc(dtype=INT8, d=96)), UNSUPPORTED, "head_dim"),
    (dict(n_q=7), INVALID, "multiple"),
    (dict(scale=float("inf")), INVALID, "finite"),
    (dict(window=-2), INVALID, "window"),
    (dict(rows=2**24, n_q=64, cache=desc(dtype=FP8, n_kv=8)), UNSUPPORTED, "grid"),
    (dict(maxb=8192, ws=FAKE, ws_bytes=16), INVALID, "workspace"),
])
def test_rows_quant_rejects(L, name, kw, code, msg):
    if name.endswith("chunked_prefill_quant") and kw.get("rows") == -1:
        msg = "chunk_len"
    assert rows_quant(L, name, **kw) == code
    assert msg in _lib.last_error()


def test_rows_quant_empty_and_workspace_query(L):
    assert rows_quant(L, "pa_paged_attn_chunked_prefill_quant", rows=0) == PA_OK
    assert rows_quant(L, "pa_paged_attn_decode_multi_quant", batch=0) == PA_OK
    # 8 KV heads x 4 rows x G = 8: 32 pairs per KV head in two slices of 16 columns, a
    # 128-block table: (m, l, acc) for every (sequence, row, head) and partition, as the
    # single-row quantised decode of 32 heads per KV head would need.
    q = L.pa_decode_multi_workspace_bytes(4, 4, 64, 128, desc(nb=4096, n_kv=8, dtype=FP8))
    one = L.pa_decode_workspace_bytes(4, 256, 128, desc(nb=4096, n_kv=8, dtype=FP8))
    assert q == one and q > 0


def decode_quant_append(L, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, q_dtype=_lib.PA_BF16, slots=FAKE, batch=2, n_q=8, k=FAKE, v=FAKE,
             ks=FAKE, vs=FAKE, cache=_lib.CacheDesc(64, 16, 2, 128, _lib.PA_FP8_E4M3), bt=FAKE, maxb=4,
             ctx=FAKE, scale=0.1, window=0, alibi=None, out=FAKE, out_dtype=_lib.PA_F32, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    return L.pa_paged_attn_decode_quant_append(
        a["q"], a["kn"], a["vn"], a["q_dtype"], a["slots"], a["batch"], a["n_q"], a["k"], a["v"], a["ks"],
        a["vs"], ctypes.byref(a["cache"]), a["bt"], a["maxb"], a["ctx"], a["scale"], a["window"], a["alibi"], a["out"],
        a["out_dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(kn=None), INVALID, "k_new"),
    (dict(slots=None), INVALID, "slot_mapping"),
    (dict(vn=FAKE + 4), INVALID, "aligned"),
    (dict(slots=FAKE + 4), INVALID, "8-byte"),
    (dict(cache=_lib.CacheDesc(64, 16, 2, 128, _lib.PA_BF16)), INVALID, "PA_FP8_E4M3"),
    (dict(q_dtype=_lib.PA_F32), UNSUPPORTED, "bf16 or f16"),
    (dict(window=-1), INVALID, "window"),
    (dict(alibi=FAKE + 2), INVALID, "alibi_slopes"),
])
def test_decode_quant_append_rejects(L, kw, code, msg):
    assert decode_quant_append(L, **kw) == code
    assert msg in _lib.last_error()


def test_decode_quant_append_empty_batch_is_a_noop(L):
    assert decode_quant_append(L, batch=0) == PA_OK


@pytest.mark.parametrize("dt", [FP8, INT8, _lib.PA_FP8_E4M3_PER_CHANNEL, _lib.PA_INT8_PER_CHANNEL])
def test_quantised_cache_refused_elsewhere(L, dt):
    # The f32/bf16/f16 entry points do not take a quantised cache description.
    assert decode(L, cache=desc(dtype=dt)) == UNSUPPORTED
    assert "quantised" in _lib.last_error()
    assert L.pa_kv_append(FAKE, FAKE, FAKE, 4, FAKE, FAKE, desc(dtype=dt), None) == UNSUPPORTED
    assert chunked(L, cache=desc(dtype=dt)) == UNSUPPORTED
    assert multi(L, cache=desc(dtype=dt)) == UNSUPPORTED


def test_per_channel_caches_take_the_quantised_checks(L):
    for dt in (_lib.PA_FP8_E4M3_PER_CHANNEL, _lib.PA_INT8_PER_CHANNEL):
        assert append_quant(L, cache=desc(dtype=dt), ks=FAKE + 4) == INVALID
        assert "aligned" in _lib.last_error()
        assert decode_quant(L, cache=desc(dtype=dt), q_dtype=_lib.PA_F32) == UNSUPPORTED
        assert rows_quant(L, "pa_paged_attn_decode_multi_quant", cache=desc(dtype=dt), vs=None) == INVALID
        assert append_quant(L, cache=desc(dtype=dt), T=0) == PA_OK
    assert append_quant(L, cache=desc(dtype=7)) != PA_OK     # past the last dtype


def append_quant(L, **kw):
    a = dict(k=FAKE, v=FAKE, src=_lib.PA_BF16, slots=FAKE, T=4, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE,
             cache=desc(dtype=FP8), stream=None)
    a.update(kw)
    return L.pa_kv_append_quant(a["k"], a["v"], a["src"], a["slots"], a["T"], a["kc"], a["vc"],
                                a["ks"], a["vs"], a["cache"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(cache=desc(dtype=_lib.PA_F16)), INVALID, "PA_FP8_E4M3"),
    (dict(src=FP8), UNSUPPORTED, "f32, bf16 or f16"),
    (dict(T=-1), INVALID, "num_tokens"),
    (dict(ks=None), INVALID, "NULL"),
    (dict(slots=FAKE + 4), INVALID, "8-byte"),
    (dict(kc=MISALIGNED), INVALID, "aligned"),
])
def test_append_quant_rejects(L, kw, code, msg):
    assert append_quant(L, **kw) == code
    assert msg in _lib.last_error()


def test_append_quant_no_tokens_is_a_noop(L):
    assert append_quant(L, T=0) == PA_OK


def test_quant_workspace_query(L):
    # Same plan as the bf16 matrix-core decode: one partition for 32 x 8 units of
    # 4096 tokens, four of 8 x 64 blocks for 8 x 8 units of 32768 tokens.
    assert L.pa_decode_workspace_bytes(32, 32, 256, desc(nb=8192, n_kv=8, dtype=FP8)) == 0
    rows = 8 * 64 * 4
    assert L.pa_decode_workspace_bytes(8, 64, 2048, desc(nb=16384, n_kv=8, dtype=INT8)) == \
        2 * rows * 4 + rows * 128 * 4
