"""Helpers for the GPU parity tests: device/CPU conversion, oracle runs, tolerances.

Tolerances (written in each test through ``assert_parity``): for bf16/fp16
inputs max |gpu - oracle| <= 2e-3 and max |gpu - oracle| / max |oracle| <= 1e-2;
for fp32 inputs both bounds are 1e-5.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = {"bf16": (2e-3, 1e-2), "f16": (2e-3, 1e-2), "f32": (1e-5, 1e-5)}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def stored_np(t: torch.Tensor) -> np.ndarray:
    """Exact stored bits of a tensor as the oracle takes them (float32 or uint16 view)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    a = a.detach().to("cpu").contiguous()
    b = b.detach().to("cpu").contiguous()
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    iv = {4: torch.int32, 2: torch.int16, 8: torch.int64, 1: torch.uint8}[a.element_size()]
    return torch.equal(a.view(iv), b.view(iv))


def assert_parity(got, want, dtype: str, what: str, tol=None) -> dict:
    atol, rtol = tol or TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    assert np.isfinite(want).all(), f"{what}: oracle produced non-finite values"
    assert np.isfinite(got).all(), f"{what}: GPU produced non-finite values"
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    ref = float(np.abs(want).max()) if want.size else 0.0
    rel = max_abs / ref if ref > 0 else max_abs
    stats = dict(max_abs=max_abs, rel=rel)
    assert max_abs <= atol, f"{what}: max abs err {max_abs:.3e} > {atol:.1e}"
    assert rel <= rtol, f"{what}: norm-wise rel err {rel:.3e} > {rtol:.1e}"
    return stats


def oracle_step(case, sel=None):
    """The oracle's version of one decode step: append the new tokens, then attend.

    Returns (k_pool_after, v_pool_after, out) with pools as stored bits.
    """
    kp = stored_np(case.k_pool).copy()
    vp = stored_np(case.v_pool).copy()
    oracle.kv_append(stored_np(case.new_k), stored_np(case.new_v), case.slot_mapping.cpu().numpy(),
                     kp, vp)
    out = oracle.decode(stored_np(case.q), kp, vp, case.dtype, case.block_table.cpu().numpy(),
                        case.context_lens.cpu().numpy(), case.scale, sel=sel)
    return kp, vp, out


def oracle_pools(case, k_new=None, v_new=None):
    """The oracle's own append of a case's new tokens (a decode case's new_k / new_v /
    slot_mapping, or a chunk case's chunk_k / chunk_v / chunk_slots; ``k_new`` / ``v_new``
    replace the generator's rows when a test edits them) on host copies of the
    generator's pools. Tests that append on the GPU hand the oracle these pools, never the
    GPU's: no oracle input comes from the HIP path. Returns (k_pool, v_pool) as stored bits."""
    kp = stored_np(case.k_pool).copy()
    vp = stored_np(case.v_pool).copy()
    if hasattr(case, "chunk_k"):
        k, v, slots = case.chunk_k, case.chunk_v, case.chunk_slots
    else:
        k, v, slots = case.new_k, case.new_v, case.slot_mapping
    k = k if k_new is None else k_new
    v = v if v_new is None else v_new
    oracle.kv_append(stored_np(k), stored_np(v), slots.cpu().numpy(), kp, vp)
    return kp, vp


def nan_out(shape, dtype=torch.float32, device="cuda") -> torch.Tensor:
    """An output buffer filled with NaN, so that any element a kernel never writes
    fails the parity check (torch.empty may hand back finite leftovers)."""
    return torch.full(tuple(shape), float("nan"), dtype=dtype, device=device)


def gpu_step(pa, case, out_dtype=torch.float32):
    """The GPU path of one decode step on copies of the pools: kv_append then decode,
    into a NaN-filled output."""
    kp = case.k_pool.clone()
    vp = case.v_pool.clone()
    pa.kv_append(case.new_k, case.new_v, case.slot_mapping, kp, vp)
    out = nan_out((case.batch, case.n_q, case.head_dim), out_dtype)
    pa.paged_attn_decode(case.q, kp, vp, case.block_table, case.context_lens, case.scale, out=out)
    torch.cuda.synchronize()
    return kp, vp, out
