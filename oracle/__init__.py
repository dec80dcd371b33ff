"""CPU fp64 oracle for paged GQA attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library
(``paged_gqa_attention_attn_amd``) never imports it, and it imports nothing
from there: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over output rows);
this module only compiles it with gcc, loads it with ctypes and converts numpy
arrays of stored bit patterns to pointers. Every function cites, in
``oracle.c``, the page passage it follows.

Arrays are passed as numpy arrays holding the exact stored values:
``float32`` for fp32, ``uint16`` bit patterns for bf16 and fp16, and one-byte
codes for a quantised cache (``uint8`` for FP8 E4M3, ``int8`` for INT8) with
its ``float32`` per-row scales.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "oracle.c"
LIB_PATH = _HERE / "liboracle.so"

DTYPE_CODES = {"f32": 0, "bf16": 1, "f16": 2, "fp8": 3, "int8": 4}
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1, "int8": 1}
QUANTISED = ("fp8", "int8")
_STORED = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "fp8": np.uint8, "int8": np.int8}


def compile_library(source: Path = SOURCE, out: Path = LIB_PATH, extra_flags=()) -> Path:
    """Compile ``source`` into a shared library with gcc (OpenMP on)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, str(source), "-o", str(out), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def build() -> Path:
    """Always recompile the oracle library in-tree."""
    return compile_library()


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle arrays must be C-contiguous")
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_stored(a: np.ndarray, dtype: str, name: str) -> None:
    want = _STORED[dtype]
    if a.dtype != want:
        raise TypeError(f"{name}: dtype {dtype} is passed as {np.dtype(want).name}, got {a.dtype}")


def _slopes(alibi, n_q: int):
    """ALiBi slopes as a contiguous float32 [n_q] array, or None."""
    if alibi is None:
        return None
    a = np.ascontiguousarray(alibi, dtype=np.float32)
    if a.shape != (n_q,):
        raise ValueError("alibi slopes must be [n_q]")
    return a


class Oracle:
    """ctypes view of one compiled oracle library (the default one, or a test variant)."""

    def __init__(self, lib_path: Path | str = LIB_PATH):
        lib_path = Path(lib_path)
        if not lib_path.exists():
            raise FileNotFoundError(f"{lib_path} is not built; call oracle.build()")
        self.lib = ctypes.CDLL(str(lib_path))
        L = self.lib
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_upcast.argtypes = [vp, ctypes.c_int, i64, vp]
        L.oracle_upcast.restype = ctypes.c_int
        L.oracle_kv_append.argtypes = [vp, vp, vp, i64, i32, i32, i32, i64, i32, vp, vp]
        L.oracle_kv_append.restype = i64
        L.oracle_decode.argtypes = [vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i64, i32,
                                    vp, i32, vp, f64, i32, vp, vp, i64, vp, i32]
        L.oracle_decode.restype = ctypes.c_int
        L.oracle_decode_ex.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp, i32, i32, i32,
                                       i32, i64, i32, vp, i32, vp, f64, i32, vp, vp, i64, vp, i32]
        L.oracle_decode_ex.restype = ctypes.c_int
        L.oracle_encode_fp8_e4m3.argtypes = [vp, i64, vp]
        L.oracle_encode_fp8_e4m3.restype = ctypes.c_int
        L.oracle_quantize_rows.argtypes = [vp, ctypes.c_int, i64, i32, ctypes.c_int, vp, vp]
        L.oracle_quantize_rows.restype = ctypes.c_int
        L.oracle_kv_append_quant.argtypes = [vp, vp, ctypes.c_int, vp, i64, i32, i32, ctypes.c_int,
                                             i64, i32, vp, vp, vp, vp]
        L.oracle_kv_append_quant.restype = i64
        L.oracle_decode_channel.argtypes = L.oracle_decode_ex.argtypes
        L.oracle_decode_channel.restype = ctypes.c_int
        L.oracle_quantize_channels.argtypes = [vp, ctypes.c_int, i64, i32, i32, ctypes.c_int, vp, vp]
        L.oracle_quantize_channels.restype = ctypes.c_int
        L.oracle_kv_append_quant_channel.argtypes = [vp, vp, ctypes.c_int, vp, i64, i32, i32, ctypes.c_int,
                                                     i64, i32, vp, vp, vp, vp]
        L.oracle_kv_append_quant_channel.restype = i64
        L.oracle_prefill.argtypes = [vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32, i32, f64,
                                     i32, vp, vp, i64, vp, i32]
        L.oracle_prefill.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = ctypes.c_int

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    # -- exact widening ------------------------------------------------------
    def upcast(self, a: np.ndarray, dtype: str) -> np.ndarray:
        _check_stored(a, dtype, "a")
        a = np.ascontiguousarray(a)
        out = np.empty(a.shape, dtype=np.float64)
        rc = self.lib.oracle_upcast(_ptr(a), DTYPE_CODES[dtype], a.size, _ptr(out))
        if rc != 0:
            raise ValueError("oracle_upcast rejected its arguments")
        return out

    # -- slot-mapped cache write (in place on the pools) ---------------------
    def kv_append(self, k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                  k_pool: np.ndarray, v_pool: np.ndarray) -> int:
        """k, v: [T][n_kv][d]; pools: [num_blocks][n_kv][bs][d]; slots int64 [T]."""
        T, n_kv, d = k.shape
        nb, n_kv2, bs, d2 = k_pool.shape
        if v.shape != k.shape or v_pool.shape != k_pool.shape or n_kv2 != n_kv or d2 != d:
            raise ValueError("shape mismatch")
        if not (k.dtype == v.dtype == k_pool.dtype == v_pool.dtype):
            raise TypeError("k, v and pools must share one dtype")
        slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        if slots.shape != (T,):
            raise ValueError("slot_mapping must have one entry per token")
        n = self.lib.oracle_kv_append(_ptr(np.ascontiguousarray(k)), _ptr(np.ascontiguousarray(v)),
                                      _ptr(slots), T, n_kv, d, k.dtype.itemsize, nb, bs,
                                      _ptr(k_pool), _ptr(v_pool))
        if n < 0:
            raise ValueError("oracle_kv_append rejected its arguments (slot out of range?)")
        return int(n)

    # -- per-token quantisation (fp32 steps) -----------------------------------
    def encode_fp8(self, y: np.ndarray) -> np.ndarray:
        """Nearest OCP E4M3 code (ties to even) of each float32 y, |y| <= 448."""
        y = np.ascontiguousarray(y, dtype=np.float32)
        out = np.empty(y.shape, dtype=np.uint8)
        if self.lib.oracle_encode_fp8_e4m3(_ptr(y), y.size, _ptr(out)) != 0:
            raise ValueError("oracle_encode_fp8_e4m3: values must be finite with |y| <= 448")
        return out

    def quantize_rows(self, x: np.ndarray, src_dtype: str, fmt: str):
        """Rows x [..., d] (stored values of src_dtype) -> (codes [..., d], scales [...])."""
        _check_stored(x, src_dtype, "x")
        x = np.ascontiguousarray(x)
        d = x.shape[-1]
        codes = np.empty(x.shape, dtype=_STORED[fmt])
        scales = np.empty(x.shape[:-1], dtype=np.float32)
        rc = self.lib.oracle_quantize_rows(_ptr(x), DTYPE_CODES[src_dtype], x.size // d, d,
                                           DTYPE_CODES[fmt], _ptr(codes), _ptr(scales))
        if rc != 0:
            raise ValueError("oracle_quantize_rows rejected its arguments")
        return codes, scales

    def quantize_channels(self, x: np.ndarray, src_dtype: str, fmt: str, scales: np.ndarray) -> np.ndarray:
        """Rows x [..., n_kv, d] (stored values of src_dtype) -> codes [..., n_kv, d] with the
        fixed per-channel scales [n_kv][d] (float32)."""
        _check_stored(x, src_dtype, "x")
        x = np.ascontiguousarray(x)
        n_kv, d = x.shape[-2:]
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        if scales.shape != (n_kv, d):
            raise ValueError("scales must be [n_kv][d]")
        codes = np.empty(x.shape, dtype=_STORED[fmt])
        rc = self.lib.oracle_quantize_channels(_ptr(x), DTYPE_CODES[src_dtype], x.size // (n_kv * d), n_kv, d,
                                               DTYPE_CODES[fmt], _ptr(scales), _ptr(codes))
        if rc != 0:
            raise ValueError("oracle_quantize_channels rejected its arguments")
        return codes

    def kv_append_quant_channel(self, k: np.ndarray, v: np.ndarray, src_dtype: str, slot_mapping: np.ndarray,
                                k_pool: np.ndarray, v_pool: np.ndarray, k_chan: np.ndarray, v_chan: np.ndarray,
                                fmt: str) -> int:
        """Quantise k, v [T][n_kv][d] with the fixed channel scales k_chan / v_chan [n_kv][d] into the
        code pools [nb][n_kv][bs][d] (in place) at slot_mapping [T]."""
        _check_stored(k, src_dtype, "k")
        _check_stored(v, src_dtype, "v")
        for name, a in (("k_pool", k_pool), ("v_pool", v_pool)):
            _check_stored(a, fmt, name)
        T, n_kv, d = k.shape
        nb, n_kv2, bs, d2 = k_pool.shape
        if v.shape != k.shape or v_pool.shape != k_pool.shape or n_kv2 != n_kv or d2 != d:
            raise ValueError("shape mismatch")
        kc = np.ascontiguousarray(k_chan, dtype=np.float32)
        vc = np.ascontiguousarray(v_chan, dtype=np.float32)
        if kc.shape != (n_kv, d) or vc.shape != (n_kv, d):
            raise ValueError("channel scales must be [n_kv][d]")
        slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        if slots.shape != (T,):
            raise ValueError("slot_mapping must have one entry per token")
        n = self.lib.oracle_kv_append_quant_channel(_ptr(np.ascontiguousarray(k)), _ptr(np.ascontiguousarray(v)),
                                                    DTYPE_CODES[src_dtype], _ptr(slots), T, n_kv, d,
                                                    DTYPE_CODES[fmt], nb, bs, _ptr(k_pool), _ptr(v_pool),
                                                    _ptr(kc), _ptr(vc))
        if n < 0:
            raise ValueError("oracle_kv_append_quant_channel rejected its arguments (slot out of range?)")
        return int(n)

    def kv_append_quant(self, k: np.ndarray, v: np.ndarray, src_dtype: str,
                        slot_mapping: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                        k_scale: np.ndarray, v_scale: np.ndarray, fmt: str) -> int:
        """Quantise k, v [T][n_kv][d] per row into code pools [nb][n_kv][bs][d] and scale
        pools [nb][n_kv][bs] (in place) at slot_mapping [T]."""
        _check_stored(k, src_dtype, "k")
        _check_stored(v, src_dtype, "v")
        for name, a in (("k_pool", k_pool), ("v_pool", v_pool)):
            _check_stored(a, fmt, name)
        T, n_kv, d = k.shape
        nb, n_kv2, bs, d2 = k_pool.shape
        if (v.shape != k.shape or v_pool.shape != k_pool.shape or n_kv2 != n_kv or d2 != d
                or k_scale.shape != (nb, n_kv, bs) or v_scale.shape != k_scale.shape):
            raise ValueError("shape mismatch")
        if k_scale.dtype != np.float32 or v_scale.dtype != np.float32:
            raise TypeError("scales are float32")
        slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        if slots.shape != (T,):
            raise ValueError("slot_mapping must have one entry per token")
        n = self.lib.oracle_kv_append_quant(_ptr(np.ascontiguousarray(k)), _ptr(np.ascontiguousarray(v)),
                                            DTYPE_CODES[src_dtype], _ptr(slots), T, n_kv, d,
                                            DTYPE_CODES[fmt], nb, bs, _ptr(k_pool), _ptr(v_pool),
                                            _ptr(k_scale), _ptr(v_scale))
        if n < 0:
            raise ValueError("oracle_kv_append_quant rejected its arguments (slot out of range?)")
        return int(n)

    # -- decode over the paged cache -------------------------------------------
    def decode(self, q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, dtype: str,
               block_table: np.ndarray, context_lens: np.ndarray, scale: float,
               sel: np.ndarray | None = None, n_threads: int = 0, window: int = 0,
               q_dtype: str | None = None, k_scale: np.ndarray | None = None,
               v_scale: np.ndarray | None = None, alibi: np.ndarray | None = None,
               scale_mode: str = "token") -> np.ndarray:
        """q [B][n_q][d]; pools [nb][n_kv][bs][d]; returns fp64 [B][n_q][d] or [len(sel)][d].

        ``window`` W > 0 keeps only the last W positions of each context. For a quantised
        cache (``dtype`` "fp8" or "int8") pass ``q_dtype`` and the scales: [nb][n_kv][bs] per
        token (``scale_mode`` "token"), or [n_kv][d] per channel (``scale_mode`` "channel").
        ``alibi``: float32 [n_q] slopes m_h; the score of position t gets -m_h (ctx - 1 - t)."""
        q_dtype = q_dtype or dtype
        _check_stored(q, q_dtype, "q")
        for name, a in (("k_pool", k_pool), ("v_pool", v_pool)):
            _check_stored(a, dtype, name)
        if scale_mode not in ("token", "channel"):
            raise ValueError("scale_mode is 'token' or 'channel'")
        per_channel = scale_mode == "channel"
        if dtype in QUANTISED:
            want = (k_pool.shape[1], k_pool.shape[3]) if per_channel else k_pool.shape[:3]
            for name, a in (("k_scale", k_scale), ("v_scale", v_scale)):
                if a is None or a.dtype != np.float32 or a.shape != want:
                    raise ValueError(f"{name} must be float32 {'[n_kv][d]' if per_channel else '[nb][n_kv][bs]'}")
            k_scale, v_scale = np.ascontiguousarray(k_scale), np.ascontiguousarray(v_scale)
        elif per_channel:
            raise ValueError("per-channel scales need a quantised cache")
        B, n_q, d = q.shape
        nb, n_kv, bs, d2 = k_pool.shape
        if d2 != d or v_pool.shape != k_pool.shape:
            raise ValueError("shape mismatch")
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if bt.ndim != 2 or bt.shape[0] != B:
            raise ValueError("block_table must be [B][max_blocks_per_seq]")
        ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
        if ctx.shape != (B,):
            raise ValueError("context_lens must be [B]")
        alibi = _slopes(alibi, n_q)
        if sel is not None:
            sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 2)
            out = np.empty((sel.shape[0], d), dtype=np.float64)
        else:
            out = np.empty((B, n_q, d), dtype=np.float64)
        fn = self.lib.oracle_decode_channel if per_channel else self.lib.oracle_decode_ex
        rc = fn(_ptr(np.ascontiguousarray(q)), DTYPE_CODES[q_dtype],
                                       _ptr(np.ascontiguousarray(k_pool)),
                                       _ptr(np.ascontiguousarray(v_pool)), DTYPE_CODES[dtype],
                                       _ptr(k_scale), _ptr(v_scale), B, n_q, n_kv, d, nb, bs,
                                       _ptr(bt), bt.shape[1], _ptr(ctx), float(scale), int(window),
                                       _ptr(alibi), _ptr(sel), 0 if sel is None else sel.shape[0],
                                       _ptr(out), n_threads)
        if rc != 0:
            raise ValueError("oracle_decode rejected its arguments")
        return out

    # -- prefill over contiguous Q/K/V ---------------------------------------
    def prefill(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: str, causal: bool,
                scale: float, sel: np.ndarray | None = None, n_threads: int = 0,
                window: int = 0, alibi: np.ndarray | None = None) -> np.ndarray:
        """q [B][S][n_q][d], k/v [B][S][n_kv][d]; returns fp64 [B][S][n_q][d] or [len(sel)][d].

        ``sel`` rows are (b, h, i) triples. ``alibi`` (causal only): float32 [n_q] slopes
        m_h; the score of row i and key j gets -m_h (i - j).
        """
        for name, a in (("q", q), ("k", k), ("v", v)):
            _check_stored(a, dtype, name)
        B, S, n_q, d = q.shape
        n_kv = k.shape[2]
        if k.shape != (B, S, n_kv, d) or v.shape != k.shape:
            raise ValueError("shape mismatch")
        alibi = _slopes(alibi, n_q)
        if sel is not None:
            sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 3)
            out = np.empty((sel.shape[0], d), dtype=np.float64)
        else:
            out = np.empty((B, S, n_q, d), dtype=np.float64)
        rc = self.lib.oracle_prefill(_ptr(np.ascontiguousarray(q)), _ptr(np.ascontiguousarray(k)),
                                     _ptr(np.ascontiguousarray(v)), DTYPE_CODES[dtype], B, S, n_q,
                                     n_kv, d, int(bool(causal)), float(scale), int(window), _ptr(alibi),
                                     _ptr(sel), 0 if sel is None else sel.shape[0], _ptr(out), n_threads)
        if rc != 0:
            raise ValueError("oracle_prefill rejected its arguments")
        return out


    # -- a prompt chunk over its paged prefix ---------------------------------
    def chunked_prefill(self, q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, dtype: str,
                        block_table: np.ndarray, context_lens: np.ndarray, scale: float,
                        sel: np.ndarray | None = None, n_threads: int = 0,
                        window: int = 0, **quant) -> np.ndarray:
        """q [B][C][n_q][d]; row i of sequence b is position ctx_b - C + i and attends to
        positions 0 .. that position (the causal mask of the prefill pages, aligned at the
        bottom right as chunked prefill keeps the formula unchanged). Each row is the
        decode definition over the first ctx_b - C + i + 1 positions, so this runs
        oracle_decode with one pseudo-sequence per (b, i); rows at negative positions are
        zero. With ``window`` W > 0 a row sees only the last W of its positions (the sliding
        window applies per row); ``alibi`` slopes bias each row by its own position. Returns
        fp64 [B][C][n_q][d], or [len(sel)][d] for (b, i, h)."""
        B, C, n_q, d = q.shape
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        ctx = np.ascontiguousarray(context_lens, dtype=np.int64)
        rows_ctx = (ctx[:, None] - C + np.arange(C)[None, :] + 1).clip(min=0).astype(np.int32)
        q2 = np.ascontiguousarray(q).reshape(B * C, n_q, d)
        bt2 = np.repeat(bt, C, axis=0)
        if sel is not None:
            sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 3)
            sel2 = np.stack([sel[:, 0] * C + sel[:, 1], sel[:, 2]], axis=1)
            return self.decode(q2, k_pool, v_pool, dtype, bt2, rows_ctx.reshape(-1), scale,
                               sel=sel2, n_threads=n_threads, window=window, **quant)
        out = self.decode(q2, k_pool, v_pool, dtype, bt2, rows_ctx.reshape(-1), scale,
                          n_threads=n_threads, window=window, **quant)
        return out.reshape(B, C, n_q, d)


_default: Oracle | None = None


def get() -> Oracle:
    """The in-tree oracle library, compiled on first use if it is missing. PA_ORACLE_LIB in
    the environment names another build of the same source to load instead (the
    sanitizer test runs the pins against an AddressSanitizer build this way)."""
    global _default
    if _default is None:
        override = os.environ.get("PA_ORACLE_LIB")
        if override:
            _default = Oracle(override)
        else:
            if not LIB_PATH.exists():
                build()
            _default = Oracle(LIB_PATH)
    return _default


def decode(*args, **kwargs):
    return get().decode(*args, **kwargs)


def prefill(*args, **kwargs):
    return get().prefill(*args, **kwargs)


def chunked_prefill(*args, **kwargs):
    return get().chunked_prefill(*args, **kwargs)


def kv_append(*args, **kwargs):
    return get().kv_append(*args, **kwargs)


def upcast(*args, **kwargs):
    return get().upcast(*args, **kwargs)


def encode_fp8(*args, **kwargs):
    return get().encode_fp8(*args, **kwargs)


def quantize_rows(*args, **kwargs):
    return get().quantize_rows(*args, **kwargs)


def kv_append_quant(*args, **kwargs):
    return get().kv_append_quant(*args, **kwargs)


def quantize_channels(*args, **kwargs):
    return get().quantize_channels(*args, **kwargs)


def kv_append_quant_channel(*args, **kwargs):
    return get().kv_append_quant_channel(*args, **kwargs)


def max_threads() -> int:
    return get().max_threads()


__all__ = ["Oracle", "build", "compile_library", "get", "decode", "prefill", "kv_append",
           "upcast", "encode_fp8", "quantize_rows", "kv_append_quant", "quantize_channels",
           "kv_append_quant_channel", "max_threads",
           "DTYPE_CODES", "ELEM_BYTES", "QUANTISED", "LIB_PATH", "SOURCE"]
