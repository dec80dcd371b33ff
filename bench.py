#!/usr/bin/env python3
"""Benchmark of the paged GQA attention hot path on one MI355X.

Default workload (the headline metric): the LLaMA-3-8B-shaped decode step --
B=32 sequences, n_q=32, n_kv=8, d=128, every context 2048 tokens, bf16 cache
in 16-token blocks scattered by a seeded permutation. One step = kv_append of
the 32 new tokens + paged decode attention over the 2048-token contexts.

Other workloads (``--workload``): the 70B-shaped long-context decode
(B=8, n_q=64, ctx 32768), the variable-length batch with a shared prefix, the
tiny fp32 case, the causal prefill + cache write + first decode step, chunked
prefill over a paged prefix, multi-row (speculative) decode, and sliding-window
decode (the 8B shape over 16384-token contexts, window 4096), and the 8B shape over an
FP8 E4M3 or INT8 cache (codes + one fp32 scale per row).

Timing: ``--warmup`` untimed steps, then exactly ``--steps`` timed steps between
two ``torch.cuda.synchronize()`` calls. Steps rotate over ``--sets``
independent input sets so the 256 MB Infinity Cache cannot keep one step's
K/V for the next. The dominant kernel call is also bracketed with HIP events
recorded on the stream it is launched on; its average duration gives the
roofline figure.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import re
import sys
import time
from pathlib import Path

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

WORKLOADS = {
    "decode_8b": 2,
    "decode_varlen": 3,
    "decode_70b_longctx": 4,
    "decode_tiny_fp32": 1,
    "prefill_then_decode": 5,
    "chunked_prefill": 6,
    "decode_multi_8b": 7,
    "decode_window_8b": 8,
    "decode_8b_fp8": 9,
    "decode_8b_int8": 10,
    "copy_calibration": 0,
}

ROOT = Path(__file__).resolve().parent
CSRC = ROOT / "paged_gqa_attention_attn_amd" / "csrc"
# Sources that determine each profiled kernel's code (their hash dates a counter summary).
KERNEL_SOURCES = {
    "decode": ["decode.hip", "decode_mfma.hip", "mfma.h", "common.h", "launch.h", "api.hip"],
    "prefill": ["prefill.hip", "mfma.h", "common.h", "launch.h", "api.hip"],
    "decode_multi": ["decode_multi.hip", "decode.hip", "decode_mfma.hip", "mfma.h", "common.h", "launch.h", "api.hip"],
    "decode_quant": ["decode_quant.hip", "decode.hip", "quant.h", "mfma.h", "common.h", "launch.h", "api.hip"],
}


_SPIN_CYCLES_PER_US = None


def time_launches(launch, n: int) -> float:
    """Average duration in ms of ``launch(i)`` for i < n, run back to back on the current
    stream between two events. A spin kernel enqueued first keeps the GPU busy while the
    host enqueues the n launches, so the events see the launches themselves and not the
    host's enqueue latency."""
    import torch
    global _SPIN_CYCLES_PER_US
    stream = torch.cuda.current_stream()
    if _SPIN_CYCLES_PER_US is None:      # the spin's counter rate, measured once
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        torch.cuda._sleep(1_000_000)
        b.record(stream)
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_US = 1_000_000 / max(a.elapsed_time(b) * 1e3, 1.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int((2000 + 200 * n) * _SPIN_CYCLES_PER_US))   # 200 us of host time per launch
    e0.record(stream)
    for i in range(n):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _code_only(text: str) -> str:
    """Source text without comments and blank lines: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash(kind: str) -> str:
    """Hash of the code (comments and blank lines dropped) of the sources that make up a
    profiled kernel: a counter summary carries it, and is used only while it matches."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        h.update(_code_only((CSRC / name).read_text()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    f = ROOT / "profiles" / f"{workload}_traffic.json"
    if not f.exists():
        return None
    rec = json.loads(f.read_text())
    if rec.get("source_hash") != source_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="decode_8b")
    p.add_argument("--sets", type=int, default=4, help="independent input sets rotated per step")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample (0 disables it)")
    p.add_argument("--partition-tokens", type=int, default=0,
                   help="decode partition size override (0: library default)")
    p.add_argument("--alibi", action="store_true",
                   help="decode and prefill workloads: add the ALiBi bias with geometric slopes")
    p.add_argument("--unfused", action="store_true",
                   help="decode step as two launches (kv_append, then decode) instead of one")
    p.add_argument("--no-sub-records", action="store_true",
                   help="default workload only: skip the sub-records of the other workloads")
    p.add_argument("--sub-cpu-seconds", type=float, default=3.0,
                   help="target CPU time of each sub-record's oracle baseline")
    return p.parse_args(argv)


def _stored(t):
    import numpy as np
    import torch
    t = t.detach().to("cpu").contiguous()
    return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)


def host_cpu_model() -> str:
    """Model name of the host CPU, from /proc/cpuinfo."""
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_record(value, unit, sample, one_value, one_sample, digits=6):
    import oracle
    return {
        "value": round(value, digits), "unit": unit, "cores": oracle.max_threads(), "kind": "oracle",
        "sample": sample,
        "one_thread": {"value": round(one_value, digits), "unit": unit, "cores": 1, "sample": one_sample},
        "host_cpu": host_cpu_model(),
    }


def cpu_baseline_decode(case, target_s: float, window: int = 0, alibi=None, quant=None):
    """Time the CPU oracle on whole sequences of one input set (all query heads), on
    all host threads and on one. ``quant``: (codes fmt, q dtype, k_scale, v_scale)."""
    import numpy as np

    import oracle
    from paged_gqa_attention_attn_amd import accounting as acc

    if quant is None:
        kp, vp = _stored(case.k_pool), _stored(case.v_pool)
        kw = {}
        dtype = case.dtype
    else:
        dtype, q_dtype, ks, vs = quant
        kp, vp = case.k_pool.cpu().contiguous().numpy(), case.v_pool.cpu().contiguous().numpy()
        kw = dict(q_dtype=q_dtype, k_scale=ks, v_scale=vs)
    q = _stored(case.q)
    bt = case.block_table.cpu().numpy()
    ctx = case.context_lens.cpu().numpy()

    def kv_bytes(seqs):
        if quant is None:
            return acc.decode_kv_bytes(ctx[seqs], case.n_kv, case.head_dim, acc.ELEM_BYTES[dtype], window)
        return acc.quant_decode_kv_bytes(ctx[seqs], case.n_kv, case.head_dim)

    def run(seqs, threads=0):
        sel = np.asarray([[b, h] for b in seqs for h in range(case.n_q)], np.int32)
        t0 = time.perf_counter()
        oracle.decode(q, kp, vp, dtype, bt, ctx, case.scale, sel=sel, window=window, alibi=alibi,
                      n_threads=threads, **kw)
        return time.perf_counter() - t0

    t1 = run([0])
    n = int(min(case.batch, max(1, math.ceil(target_s / max(t1, 1e-6)))))
    seqs = list(range(n))
    t_all = run(seqs)
    reps = max(1, int(target_s / max(t_all, 1e-6))) if n == case.batch else 1
    dt = t_all + sum(run(seqs) for _ in range(reps - 1))
    kv = reps * kv_bytes(seqs)
    # One thread: whole sequences, about a quarter of the budget.
    t1s = run([0], threads=1)
    n1 = int(min(case.batch, max(1, (target_s / 4) // max(t1s, 1e-6))))
    seqs1 = list(range(n1))
    dt1 = t1s if n1 == 1 else run(seqs1, threads=1)
    kv1 = kv_bytes(seqs1)
    what = f"{dtype} codes" if quant is not None else dtype
    return _cpu_record(
        kv / dt / 1e9, "GB/s",
        f"fp64 oracle decode over a {what} cache of {n} of {case.batch} sequences (all {case.n_q} query "
        f"heads), {reps} pass(es), {kv} KV bytes in {dt:.2f} s",
        kv1 / dt1 / 1e9, f"{n1} sequence(s), {kv1} KV bytes in {dt1:.2f} s")


def cpu_baseline_prefill(case, target_s: float, alibi=None):
    """Time the CPU oracle on random causal prefill rows, scaled to TFLOP/s, on all host
    threads and on one."""
    import numpy as np

    import oracle

    q, k, v = _stored(case.q), _stored(case.k), _stored(case.v)
    rng = np.random.default_rng(0)

    def run(n, threads=0):
        rows = np.stack([rng.integers(0, case.batch, n), rng.integers(0, case.n_q, n),
                         rng.integers(0, case.seq_len, n)], axis=1).astype(np.int32)
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, case.dtype, True, case.scale, sel=rows, alibi=alibi, n_threads=threads)
        dt = time.perf_counter() - t0
        flops = float(4 * case.head_dim * (rows[:, 2].astype(np.int64) + 1).sum())
        return dt, flops

    dt, _ = run(64)
    n = int(max(64, min(1 << 16, 64 * target_s / max(dt, 1e-6))))
    dt, flops = run(n)
    dt1, _ = run(16, threads=1)
    n1 = int(max(16, min(1 << 14, 16 * (target_s / 4) / max(dt1, 1e-6))))
    dt1, flops1 = run(n1, threads=1)
    return _cpu_record(flops / dt / 1e12, "TFLOP/s",
                       f"fp64 oracle causal prefill of {n} random (b, h, i) rows ({flops:.3e} FLOP) in {dt:.2f} s",
                       flops1 / dt1 / 1e12, f"{n1} random rows ({flops1:.3e} FLOP) in {dt1:.2f} s", digits=9)


def cpu_baseline_chunk(c, target_s: float, unit: str):
    """Time the CPU oracle's chunked-prefill definition (each query row at its position over
    the paged cache, the chunk appended), on all host threads and on one. "TFLOP/s": random
    (b, i, h) rows, counting 4 d FLOP per key a row attends to. "GB/s": whole sequences (all
    rows and heads), counting each sequence's K/V bytes once, as the GPU rate does."""
    import numpy as np

    import oracle
    from paged_gqa_attention_attn_amd import accounting as acc

    kp, vp = _stored(c.k_pool).copy(), _stored(c.v_pool).copy()
    oracle.kv_append(_stored(c.chunk_k), _stored(c.chunk_v), c.chunk_slots.cpu().numpy(), kp, vp)
    q, bt, ctx = _stored(c.q), c.block_table.cpu().numpy(), c.context_lens.cpu().numpy()
    rng = np.random.default_rng(0)

    def run(n, threads=0):
        if unit == "TFLOP/s":
            sel = np.stack([rng.integers(0, c.batch, n), rng.integers(0, c.chunk_len, n),
                            rng.integers(0, c.n_q, n)], axis=1).astype(np.int32)
            keys = (ctx[sel[:, 0]].astype(np.int64) - c.chunk_len + sel[:, 1] + 1).clip(min=0)
            work = float(4 * c.head_dim * keys.sum())
        else:
            n = min(n, c.batch)
            sel = np.asarray([[b, i, h] for b in range(n) for i in range(c.chunk_len) for h in range(c.n_q)],
                             np.int32)
            work = float(acc.decode_kv_bytes(ctx[:n], c.n_kv, c.head_dim, acc.ELEM_BYTES[c.dtype]))
        t0 = time.perf_counter()
        oracle.chunked_prefill(q, kp, vp, c.dtype, bt, ctx, c.scale, sel=sel, n_threads=threads)
        return time.perf_counter() - t0, work, n

    per = 1e12 if unit == "TFLOP/s" else 1e9
    n0 = 32 if unit == "TFLOP/s" else 1
    dt, _, _ = run(n0)
    dt, work, n = run(int(max(n0, min(1 << 16, n0 * target_s / max(dt, 1e-6)))))
    dt1, _, _ = run(max(1, n0 // 4), threads=1)
    dt1, work1, n1 = run(int(max(1, min(1 << 14, max(1, n0 // 4) * (target_s / 4) / max(dt1, 1e-6)))), threads=1)
    what = "random (b, i, h) rows" if unit == "TFLOP/s" else f"sequences of {c.batch} (all rows and heads)"
    kind = "FLOP" if unit == "TFLOP/s" else "KV bytes"
    return _cpu_record(work / dt / per, unit,
                       f"fp64 oracle, chunk rows over the paged prefix: {n} {what} ({work:.3e} {kind}) in {dt:.2f} s",
                       work1 / dt1 / per, f"{n1} {what} ({work1:.3e} {kind}) in {dt1:.2f} s", digits=9)


def bench_decode(args, cfg: int):
    import torch

    import paged_gqa_attention_attn_amd as pa
    from paged_gqa_attention_attn_amd import accounting as acc
    from paged_gqa_attention_attn_amd import workloads as wl

    if cfg == 8:
        win = wl.WINDOW_TOKENS
        sets = [wl.make_window_decode_case(device="cuda", seed=wl.WINDOW_CASE_SEED + 1000 * i)
                for i in range(args.sets)]
    else:
        win = 0
        seed0 = wl.CONFIG_SEEDS[cfg]
        sets = [wl.make_config(cfg, device="cuda", seed=seed0 + 1000 * i) for i in range(args.sets)]
    c0 = sets[0]
    if args.partition_tokens:
        pa.set_decode_partition_tokens(args.partition_tokens)
    elem = acc.ELEM_BYTES[c0.dtype]
    out = torch.empty((c0.batch, c0.n_q, c0.head_dim), dtype=torch.float32, device="cuda")
    ws_bytes = max(pa.decode_workspace_bytes(s.batch, s.n_q, s.max_blocks_per_seq, s.k_pool)
                   for s in sets)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    slopes = wl.geometric_alibi_slopes(c0.n_q, "cuda") if args.alibi else None

    def step(i):
        s = sets[i % len(sets)]
        if args.unfused:
            pa.kv_append(s.new_k, s.new_v, s.slot_mapping, s.k_pool, s.v_pool)
        decode(s)

    def decode(s):
        if args.unfused:
            pa.paged_attn_decode(s.q, s.k_pool, s.v_pool, s.block_table, s.context_lens, s.scale,
                                 out=out, workspace=ws, window=win, alibi_slopes=slopes)
        else:
            pa.paged_attn_decode_append(s.q, s.new_k, s.new_v, s.slot_mapping, s.k_pool, s.v_pool,
                                        s.block_table, s.context_lens, s.scale, out=out,
                                        workspace=ws, window=win, alibi_slopes=slopes)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps

    # The decode launches alone, back to back, between two events on the launch
    # stream: elapsed / steps is the average duration of one decode launch.
    stream = torch.cuda.current_stream()
    dec_ms = time_launches(lambda i: decode(sets[i % len(sets)]), args.steps)

    # Per-launch spread: an event pair around each decode launch (each pair adds
    # its own overhead, so these sit above the back-to-back average).
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        decode(sets[i % len(sets)])
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    pct = {f"p{q}": round(per[min(len(per) - 1, int(q / 100 * len(per)))], 2) for q in (10, 50, 90)}

    kv = sum(acc.decode_kv_bytes(s.context_lens.cpu().tolist(), s.n_kv, s.head_dim, elem, win)
             for s in sets) / len(sets)
    io = acc.decode_io_bytes(c0.batch, c0.n_q, c0.head_dim, elem, 4, c0.max_blocks_per_seq)
    achieved = (kv + io) / (dec_ms * 1e-3) / 1e9
    rec = {
        "metric": "paged GQA decode attention: KV GB/s (% HBM peak) and µs/step at 1 GPU",
        "value": round(kv / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100 * kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c0.dtype,
        "data": "synthetic",
        "config": {
            "workload": c0.name, "batch": c0.batch, "n_q": c0.n_q, "n_kv": c0.n_kv,
            "head_dim": c0.head_dim, "block_size": c0.block_size,
            "context_lens": "2048 each" if cfg == 2 else
            ("32768 each" if cfg == 4 else ("U[128,8192], 16 sharers of a 1024-token prefix"
                                            if cfg == 3 else
                                            ("16384 each" if cfg == 8 else "{7, 33}"))),
            "window": win, "alibi": "geometric slopes" if args.alibi else None,
            "kv_bytes_per_step": int(kv), "input_sets_rotated": len(sets),
            "step": ("kv_append of one new token per sequence, then paged decode (two launches)"
                     if args.unfused else
                     "one launch: append of one new token per sequence + paged decode"),
        },
        "roofline": {
            "kernel": "decode partition kernel (decode_mfma_kernel for bf16/f16 groups of 4, 8 "
                      "or 16 heads, else decode_partition_kernel; with the fused append unless "
                      "--unfused), plus the log-sum-exp reduce kernel when a context is split",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode", args.workload),
            "algorithmic_bytes_per_launch": int(kv + io), "avg_launch_us": round(dec_ms * 1e3, 2),
            "launch_us_event_pairs": pct,
            "device_copy_gbs": device_copy_gbs(),
            "source_hash": source_hash("decode"),
        },
    }
    if cfg == 3:
        uniq = sum(acc.decode_unique_kv_bytes(s.context_lens.cpu().tolist(), s.n_kv, s.head_dim,
                                              elem, s.shared_prefix_blocks * 16, len(s.sharers))
                   for s in sets) / len(sets)
        rec["unique_kv_gbs"] = round(uniq / (ms * 1e-3) / 1e9, 2)
    flops = acc.decode_flops(c0.context_lens.cpu().tolist(), c0.n_q, c0.head_dim, win)
    rec["tflops"] = round(flops / (dec_ms * 1e-3) / 1e12, 3)
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_decode(c0, args.cpu_seconds, win,
                                                  slopes.cpu().numpy() if args.alibi else None)
    return rec


def bench_prefill(args):
    import torch

    import paged_gqa_attention_attn_amd as pa
    from paged_gqa_attention_attn_amd import accounting as acc
    from paged_gqa_attention_attn_amd import workloads as wl

    n_sets = max(1, min(args.sets, 2))
    sets = [wl.make_config(5, device="cuda", seed=wl.CONFIG_SEEDS[5] + 1000 * i)
            for i in range(n_sets)]
    c0 = sets[0]
    out = torch.empty_like(c0.q, dtype=torch.float32)
    dout = torch.empty((c0.batch, c0.n_q, c0.head_dim), dtype=torch.float32, device="cuda")
    ws_bytes = pa.decode_workspace_bytes(c0.batch, c0.n_q, c0.block_table.shape[1], c0.k_pool)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    kf = [s.k.reshape(-1, s.n_kv, s.head_dim) for s in sets]
    vf = [s.v.reshape(-1, s.n_kv, s.head_dim) for s in sets]
    pws_bytes = pa.prefill_workspace_bytes(c0.q.dtype, c0.batch, c0.seq_len, c0.n_kv, c0.head_dim)
    pws = torch.empty(max(pws_bytes, 16), dtype=torch.uint8, device="cuda")

    slopes = wl.geometric_alibi_slopes(c0.n_q, "cuda") if args.alibi else None

    def prefill(s):
        pa.paged_attn_prefill(s.q, s.k, s.v, True, s.scale, out=out, workspace=pws,
                              alibi_slopes=slopes)

    def step(i):
        s = sets[i % n_sets]
        prefill(s)
        pa.kv_append(kf[i % n_sets], vf[i % n_sets], s.prompt_slots, s.k_pool, s.v_pool)
        pa.kv_append(s.new_k, s.new_v, s.new_slots, s.k_pool, s.v_pool)
        pa.paged_attn_decode(s.q_new, s.k_pool, s.v_pool, s.block_table, s.context_lens, s.scale,
                             out=dout, workspace=ws, alibi_slopes=slopes)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # The prefill launches alone, back to back, between two events on the launch stream.
    pre_ms = time_launches(lambda i: prefill(sets[i % n_sets]), args.steps)
    flops = acc.prefill_flops_causal(c0.batch, c0.seq_len, c0.n_q, c0.head_dim)
    achieved = flops / (pre_ms * 1e-3) / 1e12
    rec = {
        "metric": "causal prefill attention TFLOP/s (+ cache write and first decode step) at 1 GPU",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c0.dtype, "data": "synthetic",
        "config": {
            "workload": c0.name, "batch": c0.batch, "seq_len": c0.seq_len, "n_q": c0.n_q,
            "n_kv": c0.n_kv, "head_dim": c0.head_dim, "causal": True,
            "alibi": "geometric slopes" if args.alibi else None,
            "causal_flops": flops,
            "full_square_flops": acc.prefill_flops_full_square(c0.batch, c0.seq_len, c0.n_q,
                                                              c0.head_dim),
            "step": "causal prefill + kv_append of the prompt + kv_append of one token + "
                    "decode at context 4097",
        },
        "roofline": {
            "kernel": "paged_attn_prefill", "bound": "mfma", "achieved": round(achieved, 2),
            # one call = the f16 staging of V (bf16 only) + the prefill kernel
            "launches_per_call": 2 if pws_bytes else 1,
            "pv_product": "f16 on an exact f16 copy of V, P in 11 bits" if pws_bytes
                          else "input dtype (bf16: P in hi + lo parts)",
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("prefill", args.workload),
            "algorithmic_flops_per_launch": flops, "avg_launch_us": round(pre_ms * 1e3, 2),
            "source_hash": source_hash("prefill"),
        },
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_prefill(c0, args.cpu_seconds,
                                                   slopes.cpu().numpy() if args.alibi else None)
    return rec


def device_copy_gbs(n_bytes: int = 256 * 2**20, reps: int = 20) -> float:
    """Read + write GB/s of a plain device copy of n_bytes, for context beside the roofline."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return round(2 * n_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)


def bench_chunked_prefill(args):
    """A 1024-token prompt chunk of each of 2 sequences over a 3072-token paged prefix
    (LLaMA-3-8B attention shape): kv_append of the chunk, then chunked prefill."""
    import torch

    import paged_gqa_attention_attn_amd as pa
    from paged_gqa_attention_attn_amd import accounting as acc
    from paged_gqa_attention_attn_amd import workloads as wl

    B, C, P = 2, 1024, 3072
    n_sets = max(1, min(args.sets, 2))
    sets = [wl.make_chunk_case(batch=B, chunk_len=C, prefix_lens=[P] * B, n_q=32, n_kv=8,
                               head_dim=128, dtype="bf16", seed=1006 + 1000 * i, device="cuda",
                               name="chunked_prefill_b2_prefix3072_chunk1024")
            for i in range(n_sets)]
    c0 = sets[0]
    out = torch.empty_like(c0.q, dtype=torch.float32)

    def prefill(s):
        pa.paged_attn_chunked_prefill(s.q, s.k_pool, s.v_pool, s.block_table, s.context_lens,
                                      s.scale, out=out)

    def step(i):
        s = sets[i % n_sets]
        pa.kv_append(s.chunk_k, s.chunk_v, s.chunk_slots, s.k_pool, s.v_pool)
        prefill(s)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pre_ms = time_launches(lambda i: prefill(sets[i % n_sets]), args.steps)
    flops = acc.chunked_prefill_flops(c0.context_lens.cpu().tolist(), C, c0.n_q, c0.head_dim)
    achieved = flops / (pre_ms * 1e-3) / 1e12
    rec = {
        "metric": "chunked prefill attention over a paged prefix, TFLOP/s (+ the chunk's cache write) at 1 GPU",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c0.dtype, "data": "synthetic",
        "config": {"workload": c0.name, "batch": B, "chunk_len": C, "prefix_len": P, "n_q": c0.n_q,
                   "n_kv": c0.n_kv, "head_dim": c0.head_dim, "flops": flops,
                   "step": "kv_append of the 2x1024 chunk tokens + chunked prefill"},
        "roofline": {"kernel": "chunked_prefill call: f16 copy of the V blocks read (bf16 caches) + "
                               "prefill kernel with paged keys", "bound": "mfma",
                     "launches_per_call": 2 if c0.dtype == "bf16" else 1,
                     "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill", args.workload),
                     "algorithmic_flops_per_launch": flops, "avg_launch_us": round(pre_ms * 1e3, 2),
                     "source_hash": source_hash("prefill")},
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_chunk(c0, args.cpu_seconds, "TFLOP/s")
    return rec


def bench_decode_multi(args):
    """Speculative verification on the 8B decode shape: 4 new tokens per sequence (B=32,
    n_q=32, n_kv=8, d=128, contexts of 2048 including them): kv_append of the 128 new
    tokens, then one multi-row decode launch."""
    import torch

    import paged_gqa_attention_attn_amd as pa
    from paged_gqa_attention_attn_amd import accounting as acc
    from paged_gqa_attention_attn_amd import workloads as wl

    B, R, ctx = 32, 4, 2048
    sets = [wl.make_chunk_case(batch=B, chunk_len=R, prefix_lens=[ctx - R] * B, n_q=32, n_kv=8,
                               head_dim=128, dtype="bf16", seed=1007 + 1000 * i, device="cuda",
                               name="llama3_8b_decode_b32_ctx2048_4_rows")
            for i in range(args.sets)]
    c0 = sets[0]
    out = torch.empty_like(c0.q, dtype=torch.float32)

    def decode(s):
        pa.paged_attn_decode_multi(s.q, s.k_pool, s.v_pool, s.block_table, s.context_lens, s.scale,
                                   out=out)

    def step(i):
        s = sets[i % len(sets)]
        pa.kv_append(s.chunk_k, s.chunk_v, s.chunk_slots, s.k_pool, s.v_pool)
        decode(s)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dec_ms = time_launches(lambda i: decode(sets[i % len(sets)]), args.steps)
    kv = acc.decode_kv_bytes([ctx] * B, c0.n_kv, c0.head_dim, 2)
    io = acc.decode_io_bytes(B * R, c0.n_q, c0.head_dim, 2, 4, c0.max_blocks_per_seq)
    achieved = (kv + io) / (dec_ms * 1e-3) / 1e9
    rec = {
        "metric": "multi-row paged decode (4 new tokens per sequence): KV GB/s (% HBM peak) at 1 GPU",
        "value": round(kv / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100 * kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c0.dtype, "data": "synthetic",
        "config": {"workload": c0.name, "batch": B, "q_rows": R, "n_q": c0.n_q, "n_kv": c0.n_kv,
                   "head_dim": c0.head_dim, "context_lens": "2048 each (including the 4 new tokens)",
                   "kv_bytes_per_step": int(kv),
                   "step": "kv_append of 4 new tokens per sequence + one multi-row decode launch"},
        "roofline": {"kernel": "multi-row decode kernel (matrix cores)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_multi", args.workload),
                     "algorithmic_bytes_per_launch": int(kv + io), "avg_launch_us": round(dec_ms * 1e3, 2),
                     "source_hash": source_hash("decode_multi")},
        "tflops": round(4 * R * c0.n_q * c0.head_dim * ctx * B / (dec_ms * 1e-3) / 1e12, 3),
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_chunk(c0, args.cpu_seconds, "GB/s")
    return rec


def bench_decode_quant(args, fmt: str):
    """The 8B decode shape (B=32, n_q=32, n_kv=8, d=128, contexts 2048) over a one-byte
    cache: kv_append_quant of the 32 new tokens, then decode_quant."""
    import torch

    import paged_gqa_attention_attn_amd as pa
    from paged_gqa_attention_attn_amd import accounting as acc
    from paged_gqa_attention_attn_amd import workloads as wl

    B, ctx = 32, 2048
    name = f"llama3_8b_decode_b32_ctx2048_{fmt}_cache"
    sets = [wl.make_quant_decode_case(fmt=fmt, batch=B, n_q=32, n_kv=8, head_dim=128,
                                      context_lens=[ctx] * B, seed=1009 + 1000 * i, device="cuda",
                                      name=name) for i in range(args.sets)]
    c0 = sets[0]
    out = torch.empty((B, c0.n_q, c0.head_dim), dtype=torch.float32, device="cuda")
    ws_bytes = pa.quant_decode_workspace_bytes(B, c0.n_q, c0.max_blocks_per_seq, c0.k_pool, fmt)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def decode(s):
        # the attention launch of a step: the fused append + decode, or decode alone
        if args.unfused:
            pa.paged_attn_decode_quant(s.q, s.k_pool, s.v_pool, s.k_scale, s.v_scale, fmt, s.block_table,
                                       s.context_lens, s.scale, out=out, workspace=ws)
        else:
            pa.paged_attn_decode_quant_append(s.q, s.new_k, s.new_v, s.slot_mapping, s.k_pool, s.v_pool,
                                              s.k_scale, s.v_scale, fmt, s.block_table, s.context_lens,
                                              s.scale, out=out, workspace=ws)

    def step(i):
        s = sets[i % len(sets)]
        if args.unfused:
            pa.kv_append_quant(s.new_k, s.new_v, s.slot_mapping, s.k_pool, s.v_pool, s.k_scale,
                               s.v_scale, fmt)
        decode(s)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dec_ms = time_launches(lambda i: decode(sets[i % len(sets)]), args.steps)
    kv = acc.quant_decode_kv_bytes([ctx] * B, c0.n_kv, c0.head_dim)
    io = acc.decode_io_bytes(B, c0.n_q, c0.head_dim, 2, 4, c0.max_blocks_per_seq)
    achieved = (kv + io) / (dec_ms * 1e-3) / 1e9
    rec = {
        "metric": f"paged GQA decode over an {fmt.upper()} KV cache: KV GB/s (% HBM peak) and "
                  "µs/step at 1 GPU",
        "value": round(kv / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100 * kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{fmt} cache, bf16 q, fp32 accumulate", "data": "synthetic",
        "config": {"workload": name, "batch": B, "n_q": c0.n_q, "n_kv": c0.n_kv,
                   "head_dim": c0.head_dim, "block_size": 16, "context_lens": "2048 each",
                   "kv_bytes_per_step": int(kv), "input_sets_rotated": len(sets),
                   "step": ("kv_append_quant of one new token per sequence, then decode_quant "
                            "(two launches)") if args.unfused else
                           "one decode_quant_append launch: the new token's quantising append fused "
                           "into decode"},
        "roofline": {"kernel": "decode_quant_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_quant", args.workload),
                     "algorithmic_bytes_per_launch": int(kv + io), "avg_launch_us": round(dec_ms * 1e3, 2),
                     "source_hash": source_hash("decode_quant")},
        "tflops": round(acc.decode_flops([ctx] * B, c0.n_q, c0.head_dim) / (dec_ms * 1e-3) / 1e12, 3),
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline_decode(
            c0, args.cpu_seconds,
            quant=(c0.fmt, c0.q_dtype, c0.k_scale.cpu().numpy(), c0.v_scale.cpu().numpy()))
    return rec


def bench_copy(args):
    """A plain device copy of a known size: the reference that scales the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 64 * 2**20                      # 64 Mi fp32 = 256 MiB each way
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    return {"metric": "plain device copy (counter calibration)", "value": round(2 * 4 * n / ms / 1e6, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "copy_256MiB", "bytes_read_per_launch": 4 * n,
                       "bytes_written_per_launch": 4 * n}}


# Workloads measured beside the default one (same steps and warm-up), each reported as a
# compact sub-record of the default line: the 70B-shaped long-context decode, the
# variable-length batch, the causal prefill + cache write + decode, and the 8B decode on
# the VALU decode kernel (the design without matrix cores in decode).
SUB_RECORDS = [("decode_70b_longctx", 4, None), ("decode_varlen", 3, None),
               ("prefill_then_decode", 5, None), ("decode_8b_valu_kernel", 2, {"decode_matrix_cores": 0})]


def compact(rec: dict) -> dict:
    """The measured figures of a full bench record."""
    out = {k: rec[k] for k in ("metric", "value", "unit", "us_per_step", "pct_hbm_peak", "tflops", "dtype")
           if k in rec}
    out["workload"] = rec["config"]["workload"]
    r = rec["roofline"]
    out["roofline"] = {k: r[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "avg_launch_us")}
    if "cpu_baseline" in rec:
        out["cpu_baseline"] = rec["cpu_baseline"]
    return out


def sub_records(args) -> dict:
    import paged_gqa_attention_attn_amd as pa
    sub = argparse.Namespace(**vars(args))
    sub.cpu_seconds = args.sub_cpu_seconds
    recs = {}
    for name, cfg, options in SUB_RECORDS:
        sub.workload = name   # names the counter summary of this workload (none for the VALU kernel)
        saved = {k: pa.set_option(k, v) for k, v in (options or {}).items()}
        try:
            rec = bench_prefill(sub) if cfg == 5 else bench_decode(sub, cfg)
        finally:
            for k, v in saved.items():
                pa.set_option(k, v)
        c = compact(rec)
        if options:
            c["options"] = options
        recs[name] = c
        # The buffers of a finished sub-record stay in torch's cache for the next one to
        # reuse. When they were handed back to the driver (torch.cuda.empty_cache()), a
        # decode timed within the next second ran 5% slower (variable-length decode:
        # 195 us right after, 184-186 us after a pause of a second or more).
    return recs


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this library has no "
              "multi-GPU path. Decode would shard by sequence or by KV head with no exchange "
              "inside attention, or by context range with one log-sum-exp merge of the partials.",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    cfg = WORKLOADS[args.workload]
    if cfg == 0:
        rec = bench_copy(args)
    else:
        rec = (bench_prefill(args) if cfg == 5 else bench_chunked_prefill(args) if cfg == 6
               else bench_decode_multi(args) if cfg == 7
               else bench_decode_quant(args, "fp8") if cfg == 9
               else bench_decode_quant(args, "int8") if cfg == 10 else bench_decode(args, cfg))
    if args.workload == "decode_8b" and not args.no_sub_records and not args.unfused and not args.alibi:
        rec["sub_records"] = sub_records(args)
    rec["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
