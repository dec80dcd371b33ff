"""MI355X (gfx950) paged GQA attention: Python binding of the C-ABI library.

The functions here have the names of the library's entry points and only
marshal arguments: they check that tensors are contiguous device tensors of
the right type, read sizes from shapes, and pass raw pointers and the current
HIP stream to ``libpagedattn.so``. Every step of the computation runs in the
library's HIP kernels; there is no fallback implementation.

Layouts (see include/pagedattn.h):
  q            [B][n_q][d]                 (decode)
  k/v caches   [num_blocks][n_kv][16][d]
  block_table  int32 [B][max_blocks_per_seq]
  context_lens int32 [B]
  slot_mapping int64 [T]
  prefill q    [B][S][n_q][d], k/v [B][S][n_kv][d]
  quantised caches: codes uint8 (FP8 E4M3 bit patterns; torch.float8_e4m3fn views
  are accepted too) or int8 [num_blocks][n_kv][16][d], scales float32
  [num_blocks][n_kv][16]
  alibi_slopes float32 [n_q], optional on every attention call: query head h adds
  -alibi_slopes[h] * (query position - key position) to each score
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import CacheDesc, LibraryNotBuilt

__all__ = ["kv_append", "paged_attn_decode", "paged_attn_decode_noalloc", "paged_attn_decode_append", "paged_attn_prefill",
           "paged_attn_chunked_prefill", "paged_attn_decode_multi", "kv_append_quant",
           "paged_attn_decode_quant", "paged_attn_decode_quant_append", "quant_decode_workspace_bytes",
           "paged_attn_decode_multi_quant", "paged_attn_chunked_prefill_quant",
           "prefill_workspace_bytes", "chunked_prefill_workspace_bytes",
           "decode_workspace_bytes", "set_workspace",
           "set_decode_partition_tokens", "set_option", "get_option", "library_version", "LibraryNotBuilt", "PagedAttnError"]

_DTYPE = {torch.float32: _lib.PA_F32, torch.bfloat16: _lib.PA_BF16, torch.float16: _lib.PA_F16}


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed ({code}): {_lib.last_error()}")
        self.code = code


def _check(fn: str, code: int) -> None:
    if code != _lib.PA_OK:
        raise PagedAttnError(fn, code)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t.data_ptr()


def _torch_stream(t: torch.Tensor, stream):
    """The stream a call enqueues on: ``stream``, else the current stream of t's device."""
    return stream if stream is not None else torch.cuda.current_stream(t.device)


def _stream(t: torch.Tensor, stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(_torch_stream(t, stream).cuda_stream)


def _alloc(shape, dtype, like: torch.Tensor, stream) -> torch.Tensor:
    """An output or scratch tensor owned by the stream the kernels run on, so that the
    caching allocator does not hand its memory to other work before they finish."""
    with torch.cuda.stream(_torch_stream(like, stream)):
        return torch.empty(shape, dtype=dtype, device=like.device)


def _alibi_arg(alibi_slopes, n_q: int):
    """Device pointer of ALiBi slopes (float32 [n_q] on the GPU), or None for no bias."""
    if alibi_slopes is None:
        return None
    if alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (n_q,):
        raise ValueError(f"alibi_slopes must be float32 [{n_q}]")
    return _dev(alibi_slopes, "alibi_slopes", torch.float32)


def _workspace_args(workspace):
    """(pointer, bytes) of an optional device workspace; (None, 0) for none."""
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def _cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    if k_cache.dim() != 4:
        raise ValueError("caches must be [num_blocks][n_kv][block_size][head_dim]")
    if k_cache.dtype not in _DTYPE:
        raise TypeError(f"unsupported cache dtype {k_cache.dtype}")
    nb, n_kv, bs, d = k_cache.shape
    return CacheDesc(nb, bs, n_kv, d, _DTYPE[k_cache.dtype])


def library_version() -> int:
    return int(_lib.load().pa_version())


def set_decode_partition_tokens(tokens: int) -> int:
    """Override the decode partition size (tokens); 0 restores the built-in choice."""
    prev = _lib.load().pa_set_decode_partition_tokens(int(tokens))
    if prev < 0:
        raise ValueError(f"invalid partition size {tokens}")
    return int(prev)


def set_option(name: str, value: int) -> int:
    """Set a kernel-choice option (``_lib.OPTIONS`` names them); returns the previous value.

    decode_matrix_cores (0/1), decode_ring (1/2), decode_waves (0 = planner's
    choice, 1..8), prefill_stage_v (0/1), validate (0/1). Each starts from its
    environment variable, read once by the library.
    """
    if name not in _lib.OPTIONS:
        raise ValueError(f"unknown option {name!r} (known: {sorted(_lib.OPTIONS)})")
    prev = _lib.load().pa_set_option(_lib.OPTIONS[name][0], int(value))
    if prev < 0:
        raise ValueError(f"option {name}: value {value} out of range")
    return int(prev)


def get_option(name: str) -> int:
    """Current value of a kernel-choice option."""
    if name not in _lib.OPTIONS:
        raise ValueError(f"unknown option {name!r} (known: {sorted(_lib.OPTIONS)})")
    return int(_lib.load().pa_get_option(_lib.OPTIONS[name][0]))


def kv_append(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
              k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Write k/v rows [T][n_kv][d] into the caches at ``slot_mapping`` (int64 [T])."""
    L = _lib.load()
    desc = _cache_desc(k_cache)
    if v_cache.shape != k_cache.shape or k.shape != v.shape:
        raise ValueError("k/v or cache shapes differ")
    if k.dim() != 3 or k.shape[1:] != k_cache.shape[1:2] + k_cache.shape[3:]:
        raise ValueError("k and v must be [T][n_kv][head_dim] matching the cache")
    T = k.shape[0]
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    dt = k_cache.dtype
    _check("pa_kv_append", L.pa_kv_append(
        _dev(k, "k", dt), _dev(v, "v", dt), _dev(slot_mapping, "slot_mapping", torch.int64), T,
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt), ctypes.byref(desc),
        _stream(k_cache, stream)))


def set_workspace(workspace: torch.Tensor | None) -> None:
    """Default decode workspace for calls made with ``workspace=None`` at the C ABI
    (the binding below always passes one it allocated); None clears it."""
    L = _lib.load()
    if workspace is None:
        _check("pa_set_workspace", L.pa_set_workspace(None, 0))
    else:
        _check("pa_set_workspace", L.pa_set_workspace(_dev(workspace, "workspace"),
                                                      workspace.numel() * workspace.element_size()))


def decode_workspace_bytes(batch: int, n_q: int, max_blocks_per_seq: int,
                           k_cache: torch.Tensor) -> int:
    desc = _cache_desc(k_cache)
    return int(_lib.load().pa_decode_workspace_bytes(batch, n_q, max_blocks_per_seq,
                                                     ctypes.byref(desc)))


def paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                      workspace: torch.Tensor | None = None, stream=None,
                      window: int = 0,
        alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention of q [B][n_q][d] over the paged caches; returns out [B][n_q][d].
    window W > 0 restricts each sequence to its last W positions."""
    L = _lib.load()
    desc = _cache_desc(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    B, n_q, d = q.shape
    if d != k_cache.shape[3]:
        raise ValueError("q head_dim differs from the cache")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    maxb = block_table.shape[1]
    if out is None:
        out = _alloc((B, n_q, d), out_dtype, q, stream)
    if out.shape != (B, n_q, d) or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][n_q][d] in a supported dtype")
    if workspace is None:
        need = int(L.pa_decode_workspace_bytes(B, n_q, maxb, ctypes.byref(desc)))
        if need:
            workspace = _alloc(need, torch.uint8, q, stream)
    ws_ptr, ws_bytes = _workspace_args(workspace)
    dt = k_cache.dtype
    _check("pa_paged_attn_decode", L.pa_paged_attn_decode(
        _dev(q, "q", dt), B, n_q, _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        ctypes.byref(desc), _dev(block_table, "block_table", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"),
        _DTYPE[out.dtype], ws_ptr, ws_bytes, _stream(q, stream)))
    return out


def paged_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                              out: torch.Tensor, stream=None, window: int = 0,
                              alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """paged_attn_decode into the caller's ``out`` [B][n_q][d] with no allocation at all:
    split-context partials go to the library's fixed per-GPU scratch array."""
    L = _lib.load()
    desc = _cache_desc(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    B, n_q, d = q.shape
    if d != k_cache.shape[3]:
        raise ValueError("q head_dim differs from the cache")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    if out.shape != (B, n_q, d) or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][n_q][d] in a supported dtype")
    dt = k_cache.dtype
    _check("pa_paged_attn_decode_noalloc", L.pa_paged_attn_decode_noalloc(
        _dev(q, "q", dt), B, n_q, _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        ctypes.byref(desc), _dev(block_table, "block_table", torch.int32), block_table.shape[1],
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"), _DTYPE[out.dtype], _stream(q, stream)))
    return out


def paged_attn_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, block_table: torch.Tensor,
                             context_lens: torch.Tensor, scale: float,
                             out: torch.Tensor | None = None,
                             out_dtype: torch.dtype = torch.float32,
                             workspace: torch.Tensor | None = None, stream=None,
                             window: int = 0,
        alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one launch: write k_new/v_new [B][n_kv][d] at slot_mapping [B],
    then attend with q [B][n_q][d] over the caches; returns out [B][n_q][d].
    window W > 0 restricts each sequence to its last W positions."""
    L = _lib.load()
    desc = _cache_desc(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    B, n_q, d = q.shape
    if d != k_cache.shape[3]:
        raise ValueError("q head_dim differs from the cache")
    if k_new.shape != (B, k_cache.shape[1], d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B][n_kv][head_dim]")
    if slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be [B]")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    maxb = block_table.shape[1]
    if out is None:
        out = _alloc((B, n_q, d), out_dtype, q, stream)
    if out.shape != (B, n_q, d) or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][n_q][d] in a supported dtype")
    if workspace is None:
        need = int(L.pa_decode_workspace_bytes(B, n_q, maxb, ctypes.byref(desc)))
        if need:
            workspace = _alloc(need, torch.uint8, q, stream)
    ws_ptr, ws_bytes = _workspace_args(workspace)
    dt = k_cache.dtype
    _check("pa_paged_attn_decode_append", L.pa_paged_attn_decode_append(
        _dev(q, "q", dt), _dev(k_new, "k_new", dt), _dev(v_new, "v_new", dt),
        _dev(slot_mapping, "slot_mapping", torch.int64), B, n_q, _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), ctypes.byref(desc),
        _dev(block_table, "block_table", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"),
        _DTYPE[out.dtype], ws_ptr, ws_bytes, _stream(q, stream)))
    return out


def prefill_workspace_bytes(dtype: torch.dtype, batch: int, seq_len: int, n_kv: int,
                            head_dim: int) -> int:
    """Bytes of device workspace a prefill with these sizes uses (0: none)."""
    if dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {dtype}")
    return int(_lib.load().pa_prefill_workspace_bytes(_DTYPE[dtype], batch, seq_len, n_kv, head_dim))


def paged_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool,
                       scale: float, out: torch.Tensor | None = None,
                       out_dtype: torch.dtype = torch.float32, stream=None,
                       window: int = 0, workspace: torch.Tensor | None = None,
                       alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """Attention of a prompt over itself: q [B][S][n_q][d], k/v [B][S][n_kv][d].
    window W > 0 (causal only) restricts row i to keys i - W + 1 .. i. workspace:
    a device buffer of at least prefill_workspace_bytes(...) bytes, or None to
    allocate one here."""
    L = _lib.load()
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B][S][n_q][d] and k, v [B][S][n_kv][d]")
    B, S, n_q, d = q.shape
    if k.shape[0] != B or k.shape[1] != S or k.shape[3] != d:
        raise ValueError("k/v batch, length or head_dim differ from q")
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if out is None:
        out = _alloc((B, S, n_q, d), out_dtype, q, stream)
    if out.shape != q.shape or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][S][n_q][d] in a supported dtype")
    dt = q.dtype
    if workspace is None:
        need = int(L.pa_prefill_workspace_bytes(_DTYPE[dt], B, S, k.shape[2], d))
        if need:
            workspace = _alloc(need, torch.uint8, q, stream)
    _check("pa_paged_attn_prefill", L.pa_paged_attn_prefill(
        _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt), _DTYPE[dt], B, S, n_q, k.shape[2],
        d, int(bool(causal)), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"), _DTYPE[out.dtype],
        *_workspace_args(workspace), _stream(q, stream)))
    return out


def chunked_prefill_workspace_bytes(batch: int, max_blocks_per_seq: int,
                                    k_cache: torch.Tensor) -> int:
    """Bytes of device workspace a chunked prefill with these sizes uses (0: none)."""
    desc = _cache_desc(k_cache)
    return int(_lib.load().pa_chunked_prefill_workspace_bytes(batch, max_blocks_per_seq,
                                                              ctypes.byref(desc)))


def paged_attn_chunked_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                               out: torch.Tensor | None = None,
                               out_dtype: torch.dtype = torch.float32, stream=None,
                               window: int = 0,
                               alibi_slopes: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """A prompt chunk q [B][C][n_q][d] attends to its paged prefix and causally to itself;
    row i of sequence b is position context_lens[b] - C + i. Returns out [B][C][n_q][d].
    window W > 0 restricts the row at position p to positions p - W + 1 .. p. workspace:
    a device buffer of at least chunked_prefill_workspace_bytes(...) bytes, or None to
    allocate one here."""
    L = _lib.load()
    desc = _cache_desc(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if q.dim() != 4 or q.shape[3] != k_cache.shape[3]:
        raise ValueError("q must be [B][chunk_len][n_q][head_dim] matching the cache")
    B, C, n_q, d = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    maxb = block_table.shape[1]
    if out is None:
        out = _alloc((B, C, n_q, d), out_dtype, q, stream)
    if out.shape != q.shape or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][chunk_len][n_q][d] in a supported dtype")
    if workspace is None and B > 0 and C > 0:
        need = int(L.pa_chunked_prefill_workspace_bytes(B, maxb, ctypes.byref(desc)))
        if need:
            workspace = _alloc(need, torch.uint8, q, stream)
    dt = k_cache.dtype
    _check("pa_paged_attn_chunked_prefill", L.pa_paged_attn_chunked_prefill(
        _dev(q, "q", dt), B, C, n_q, _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        ctypes.byref(desc), _dev(block_table, "block_table", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"),
        _DTYPE[out.dtype], *_workspace_args(workspace), _stream(q, stream)))
    return out


def paged_attn_decode_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                            out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                            workspace: torch.Tensor | None = None, stream=None,
                            window: int = 0,
        alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """q_rows new rows per sequence, q [B][q_rows][n_q][d]; row r of sequence b is position
    context_lens[b] - q_rows + r. Returns out [B][q_rows][n_q][d]. window W > 0 restricts
    the row at position p to positions p - W + 1 .. p."""
    L = _lib.load()
    desc = _cache_desc(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if q.dim() != 4 or q.shape[3] != k_cache.shape[3]:
        raise ValueError("q must be [B][q_rows][n_q][head_dim] matching the cache")
    B, R, n_q, d = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    maxb = block_table.shape[1]
    if out is None:
        out = _alloc((B, R, n_q, d), out_dtype, q, stream)
    if out.shape != q.shape or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][q_rows][n_q][d] in a supported dtype")
    need = int(L.pa_decode_multi_workspace_bytes(B, R, n_q, maxb, ctypes.byref(desc)))
    if need and workspace is None:
        workspace = _alloc(need, torch.uint8, q, stream)
    ws_ptr, ws_bytes = _workspace_args(workspace)
    dt = k_cache.dtype
    _check("pa_paged_attn_decode_multi", L.pa_paged_attn_decode_multi(
        _dev(q, "q", dt), B, R, n_q, _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt),
        ctypes.byref(desc), _dev(block_table, "block_table", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"),
        _DTYPE[out.dtype], ws_ptr, ws_bytes, _stream(q, stream)))
    return out


# ---- quantised cache (one-byte codes + one fp32 scale per row) ------------------------------

# Quantised cache formats: codes with one scale per row ("fp8", "int8"), or with fixed
# scales per (KV head, channel) ("fp8_per_channel", "int8_per_channel").
_QFMT = {"fp8": _lib.PA_FP8_E4M3, "int8": _lib.PA_INT8, "fp8_per_channel": _lib.PA_FP8_E4M3_PER_CHANNEL,
         "int8_per_channel": _lib.PA_INT8_PER_CHANNEL}
_FP8_CODES = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
_QCODE = {"fp8": _FP8_CODES, "int8": (torch.int8,), "fp8_per_channel": _FP8_CODES,
          "int8_per_channel": (torch.int8,)}


def _quant_desc(k_cache: torch.Tensor, fmt: str) -> CacheDesc:
    if fmt not in _QFMT:
        raise ValueError(f"fmt must be one of {sorted(_QFMT)} (got {fmt!r})")
    if k_cache.dim() != 4:
        raise ValueError("code pools must be [num_blocks][n_kv][block_size][head_dim]")
    if k_cache.dtype not in _QCODE[fmt]:
        raise TypeError(f"{fmt} code pools must be {_QCODE[fmt]} (got {k_cache.dtype})")
    nb, n_kv, bs, d = k_cache.shape
    return CacheDesc(nb, bs, n_kv, d, _QFMT[fmt])


def _check_scales(k_cache, k_scale, v_scale, fmt="fp8"):
    per_channel = fmt.endswith("_per_channel")
    want = (k_cache.shape[1], k_cache.shape[3]) if per_channel else tuple(k_cache.shape[:3])
    what = "[n_kv][head_dim]" if per_channel else "[num_blocks][n_kv][block_size]"
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if tuple(t.shape) != tuple(want):
            raise ValueError(f"{name} must be {what} = {list(want)}")


def kv_append_quant(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                    v_scale: torch.Tensor, fmt: str, stream=None) -> None:
    """Quantise k/v rows [T][n_kv][d] (f32, bf16 or f16) into the code pools at ``slot_mapping``
    (int64 [T]). ``fmt`` 'fp8' or 'int8': one scale per row, written to the float32 scale pools
    [num_blocks][n_kv][block_size]; 'fp8_per_channel' or 'int8_per_channel': k_scale / v_scale
    are the fixed float32 channel scales [n_kv][d], only read."""
    L = _lib.load()
    desc = _quant_desc(k_cache, fmt)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype or k.shape != v.shape:
        raise ValueError("k/v or cache shapes differ")
    if k.dim() != 3 or k.shape[1:] != k_cache.shape[1:2] + k_cache.shape[3:]:
        raise ValueError("k and v must be [T][n_kv][head_dim] matching the cache")
    if k.dtype not in _DTYPE or v.dtype != k.dtype:
        raise TypeError("k and v must share one of float32, bfloat16, float16")
    _check_scales(k_cache, k_scale, v_scale, fmt)
    T = k.shape[0]
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    _check("pa_kv_append_quant", L.pa_kv_append_quant(
        _dev(k, "k"), _dev(v, "v"), _DTYPE[k.dtype], _dev(slot_mapping, "slot_mapping", torch.int64), T,
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), ctypes.byref(desc), _stream(k_cache, stream)))


def quant_decode_workspace_bytes(batch: int, n_q: int, max_blocks_per_seq: int,
                                 k_cache: torch.Tensor, fmt: str) -> int:
    desc = _quant_desc(k_cache, fmt)
    return int(_lib.load().pa_decode_workspace_bytes(batch, n_q, max_blocks_per_seq,
                                                     ctypes.byref(desc)))


def paged_attn_decode_quant(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            k_scale: torch.Tensor, v_scale: torch.Tensor, fmt: str,
                            block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                            out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                            workspace: torch.Tensor | None = None, stream=None,
                            window: int = 0,
        alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention of q [B][n_q][d] (bf16 or f16) over a quantised paged cache (codes
    and per-row scales); returns out [B][n_q][d] (float32 or q's dtype)."""
    L = _lib.load()
    desc = _quant_desc(k_cache, fmt)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache differ")
    _check_scales(k_cache, k_scale, v_scale, fmt)
    B, n_q, d = q.shape
    if d != k_cache.shape[3]:
        raise ValueError("q head_dim differs from the cache")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    maxb = block_table.shape[1]
    if out is None:
        out = _alloc((B, n_q, d), out_dtype, q, stream)
    if out.shape != (B, n_q, d) or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][n_q][d] in a supported dtype")
    if workspace is None:
        need = int(L.pa_decode_workspace_bytes(B, n_q, maxb, ctypes.byref(desc)))
        if need:
            workspace = _alloc(need, torch.uint8, q, stream)
    ws_ptr, ws_bytes = _workspace_args(workspace)
    _check("pa_paged_attn_decode_quant", L.pa_paged_attn_decode_quant(
        _dev(q, "q"), _DTYPE[q.dtype], B, n_q, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        ctypes.byref(desc), _dev(block_table, "block_table", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"),
        _DTYPE[out.dtype], ws_ptr, ws_bytes, _stream(q, stream)))
    return out


def _rows_quant(fn_name: str, q, k_cache, v_cache, k_scale, v_scale, fmt, block_table, context_lens, scale,
                out, out_dtype, workspace, stream, window, alibi_slopes):
    L = _lib.load()
    desc = _quant_desc(k_cache, fmt)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache differ")
    _check_scales(k_cache, k_scale, v_scale, fmt)
    if q.dim() != 4 or q.shape[3] != k_cache.shape[3]:
        raise ValueError("q must be [B][rows][n_q][head_dim] matching the cache")
    B, R, n_q, d = q.shape
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    maxb = block_table.shape[1]
    if out is None:
        out = _alloc((B, R, n_q, d), out_dtype, q, stream)
    if out.shape != q.shape or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][rows][n_q][d] in a supported dtype")
    if workspace is None and B > 0 and R > 0:
        need = int(L.pa_decode_multi_workspace_bytes(B, R, n_q, maxb, ctypes.byref(desc)))
        if need:
            workspace = _alloc(need, torch.uint8, q, stream)
    ws_ptr, ws_bytes = _workspace_args(workspace)
    _check(fn_name, getattr(L, fn_name)(
        _dev(q, "q"), _DTYPE[q.dtype], B, R, n_q, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        ctypes.byref(desc), _dev(block_table, "block_table", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"), _DTYPE[out.dtype], ws_ptr, ws_bytes, _stream(q, stream)))
    return out


def paged_attn_decode_multi_quant(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  k_scale: torch.Tensor, v_scale: torch.Tensor, fmt: str,
                                  block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                  out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                                  workspace: torch.Tensor | None = None, stream=None, window: int = 0,
                                  alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """q_rows query rows per sequence, q [B][q_rows][n_q][d] (bf16 or f16), over a quantised
    paged cache already holding the rows' own K/V; returns out [B][q_rows][n_q][d]."""
    return _rows_quant("pa_paged_attn_decode_multi_quant", q, k_cache, v_cache, k_scale, v_scale, fmt,
                       block_table, context_lens, scale, out, out_dtype, workspace, stream, window, alibi_slopes)


def paged_attn_chunked_prefill_quant(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                     k_scale: torch.Tensor, v_scale: torch.Tensor, fmt: str,
                                     block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                     out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                                     workspace: torch.Tensor | None = None, stream=None, window: int = 0,
                                     alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """A prompt chunk q [B][chunk_len][n_q][d] (bf16 or f16) over a quantised paged cache already
    holding the chunk's own K/V; returns out [B][chunk_len][n_q][d]."""
    return _rows_quant("pa_paged_attn_chunked_prefill_quant", q, k_cache, v_cache, k_scale, v_scale, fmt,
                       block_table, context_lens, scale, out, out_dtype, workspace, stream, window, alibi_slopes)


def paged_attn_decode_quant_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                   slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                                   fmt: str, block_table: torch.Tensor, context_lens: torch.Tensor,
                                   scale: float, out: torch.Tensor | None = None,
                                   out_dtype: torch.dtype = torch.float32,
                                   workspace: torch.Tensor | None = None, stream=None,
                                   window: int = 0,
        alibi_slopes: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step over a quantised cache in one launch: quantise and write
    k_new/v_new [B][n_kv][d] (q's dtype) at slot_mapping [B], then attend with q
    [B][n_q][d]; returns out [B][n_q][d]."""
    L = _lib.load()
    desc = _quant_desc(k_cache, fmt)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache differ")
    _check_scales(k_cache, k_scale, v_scale, fmt)
    B, n_q, d = q.shape
    if d != k_cache.shape[3]:
        raise ValueError("q head_dim differs from the cache")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    n_kv = k_cache.shape[1]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.shape != (B, n_kv, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B][n_kv][d] in q's dtype")
    if slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be [B]")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B][max_blocks] and context_lens [B]")
    maxb = block_table.shape[1]
    if out is None:
        out = _alloc((B, n_q, d), out_dtype, q, stream)
    if out.shape != (B, n_q, d) or out.dtype not in _DTYPE:
        raise ValueError("out must be [B][n_q][d] in a supported dtype")
    if workspace is None:
        need = int(L.pa_decode_workspace_bytes(B, n_q, maxb, ctypes.byref(desc)))
        if need:
            workspace = _alloc(need, torch.uint8, q, stream)
    ws_ptr, ws_bytes = _workspace_args(workspace)
    _check("pa_paged_attn_decode_quant_append", L.pa_paged_attn_decode_quant_append(
        _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _DTYPE[q.dtype],
        _dev(slot_mapping, "slot_mapping", torch.int64), B, n_q, _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), ctypes.byref(desc),
        _dev(block_table, "block_table", torch.int32), maxb,
        _dev(context_lens, "context_lens", torch.int32), float(scale), int(window),
        _alibi_arg(alibi_slopes, n_q), _dev(out, "out"),
        _DTYPE[out.dtype], ws_ptr, ws_bytes, _stream(q, stream)))
    return out
