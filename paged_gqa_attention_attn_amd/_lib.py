"""ctypes loader for ``libpagedattn.so`` (the gfx950 HIP library behind include/pagedattn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libpagedattn.so"

PA_F32, PA_BF16, PA_F16, PA_FP8_E4M3, PA_INT8 = 0, 1, 2, 3, 4
PA_FP8_E4M3_PER_CHANNEL, PA_INT8_PER_CHANNEL = 5, 6
PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP = 0, -1, -2, -3

# pa_option: name -> (value, environment variable giving its initial value)
OPTIONS = {"decode_matrix_cores": (0, "PA_DECODE_MFMA"), "decode_ring": (1, "PA_DECODE_RING"),
           "decode_waves": (2, "PA_DECODE_WAVES"), "prefill_stage_v": (3, "PA_PREFILL_STAGE_V"),
           "validate": (4, "PA_VALIDATE")}

EXPORTS = (
    "pa_kv_append",
    "pa_decode_workspace_bytes",
    "pa_paged_attn_decode",
    "pa_paged_attn_decode_noalloc",
    "pa_paged_attn_decode_append",
    "pa_decode_multi_workspace_bytes",
    "pa_paged_attn_decode_multi",
    "pa_prefill_workspace_bytes",
    "pa_paged_attn_prefill",
    "pa_chunked_prefill_workspace_bytes",
    "pa_paged_attn_chunked_prefill",
    "pa_kv_append_quant",
    "pa_paged_attn_decode_quant",
    "pa_paged_attn_decode_quant_append",
    "pa_paged_attn_decode_multi_quant",
    "pa_paged_attn_chunked_prefill_quant",
    "pa_set_decode_partition_tokens",
    "pa_set_option",
    "pa_get_option",
    "pa_set_workspace",
    "pa_last_error",
    "pa_version",
)


class CacheDesc(ctypes.Structure):
    """Mirror of ``pa_cache_desc``."""

    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int),
    ]


class LibraryNotBuilt(RuntimeError):
    pass


_lib: ctypes.CDLL | None = None


def load(path: Path | str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the shared library."""
    global _lib
    if _lib is not None:
        return _lib
    path = Path(path)
    if not path.exists():
        raise LibraryNotBuilt(
            f"{path} does not exist: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(str(path))
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cd = ctypes.POINTER(CacheDesc)
    L.pa_kv_append.argtypes = [vp, vp, vp, i32, vp, vp, cd, vp]
    L.pa_kv_append.restype = ctypes.c_int
    L.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, cd]
    L.pa_decode_workspace_bytes.restype = sz
    L.pa_paged_attn_decode.argtypes = [vp, i32, i32, vp, vp, cd, vp, i32, vp, ctypes.c_float, i32, vp,
                                       vp, ctypes.c_int, vp, sz, vp]
    L.pa_paged_attn_decode.restype = ctypes.c_int
    L.pa_paged_attn_decode_noalloc.argtypes = [vp, i32, i32, vp, vp, cd, vp, i32, vp, ctypes.c_float, i32,
                                               vp, vp, ctypes.c_int, vp]
    L.pa_paged_attn_decode_noalloc.restype = ctypes.c_int
    L.pa_paged_attn_decode_append.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, cd, vp, i32, vp,
                                              ctypes.c_float, i32, vp, vp, ctypes.c_int, vp, sz, vp]
    L.pa_paged_attn_decode_append.restype = ctypes.c_int
    L.pa_decode_multi_workspace_bytes.argtypes = [i32, i32, i32, i32, cd]
    L.pa_decode_multi_workspace_bytes.restype = sz
    L.pa_paged_attn_decode_multi.argtypes = [vp, i32, i32, i32, vp, vp, cd, vp, i32, vp,
                                             ctypes.c_float, i32, vp, vp, ctypes.c_int, vp, sz, vp]
    L.pa_paged_attn_decode_multi.restype = ctypes.c_int
    L.pa_prefill_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32]
    L.pa_prefill_workspace_bytes.restype = sz
    L.pa_paged_attn_prefill.argtypes = [vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_float, i32, vp, vp, ctypes.c_int, vp, sz, vp]
    L.pa_paged_attn_prefill.restype = ctypes.c_int
    L.pa_chunked_prefill_workspace_bytes.argtypes = [i32, i32, cd]
    L.pa_chunked_prefill_workspace_bytes.restype = sz
    L.pa_paged_attn_chunked_prefill.argtypes = [vp, i32, i32, i32, vp, vp, cd, vp, i32, vp,
                                                ctypes.c_float, i32, vp, vp, ctypes.c_int, vp, sz, vp]
    L.pa_paged_attn_chunked_prefill.restype = ctypes.c_int
    L.pa_kv_append_quant.argtypes = [vp, vp, ctypes.c_int, vp, i32, vp, vp, vp, vp, cd, vp]
    L.pa_kv_append_quant.restype = ctypes.c_int
    L.pa_paged_attn_decode_quant.argtypes = [vp, ctypes.c_int, i32, i32, vp, vp, vp, vp, cd, vp, i32, vp,
                                             ctypes.c_float, i32, vp, vp, ctypes.c_int, vp, sz, vp]
    L.pa_paged_attn_decode_quant.restype = ctypes.c_int
    L.pa_paged_attn_decode_quant_append.argtypes = [vp, vp, vp, ctypes.c_int, vp, i32, i32, vp, vp, vp, vp,
                                                    cd, vp, i32, vp, ctypes.c_float, i32, vp, vp,
                                                    ctypes.c_int, vp, sz, vp]
    L.pa_paged_attn_decode_quant_append.restype = ctypes.c_int
    for name in ("pa_paged_attn_decode_multi_quant", "pa_paged_attn_chunked_prefill_quant"):
        fn = getattr(L, name)
        fn.argtypes = [vp, ctypes.c_int, i32, i32, i32, vp, vp, vp, vp, cd, vp, i32, vp, ctypes.c_float, i32, vp,
                       vp, ctypes.c_int, vp, sz, vp]
        fn.restype = ctypes.c_int
    L.pa_set_decode_partition_tokens.argtypes = [i32]
    L.pa_set_decode_partition_tokens.restype = i32
    L.pa_set_option.argtypes = [i32, i32]
    L.pa_set_option.restype = i32
    L.pa_get_option.argtypes = [i32]
    L.pa_get_option.restype = i32
    L.pa_set_workspace.argtypes = [vp, sz]
    L.pa_set_workspace.restype = ctypes.c_int
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_version.argtypes = []
    L.pa_version.restype = i32
    _lib = L
    return L


def last_error() -> str:
    return load().pa_last_error().decode(errors="replace")
