#!/usr/bin/env python3
"""Benchmark of one GQA decode step on one MI355X.

A step is the whole hot path over one batch: KV producer (norm, RoPE,
append), split-K decode partials, log-sum-exp combine, all through the C ABI
on the current stream.  Inputs are seeded synthetic caches already resident
in HBM when the timed region starts.

Prints ONE JSON line:
  value          KV GB/s of the whole step (algorithmic visible-KV bytes / step time)
  roofline       the dominant kernel (decode partials): algorithmic bytes per launch
                 / its mean launch time, timed with HIP events on the launch stream,
                 against the 8 TB/s HBM peak; traffic from rocprofv3 counters when
                 they were taken on the current kernel source, else null
  cpu_baseline   the CPU oracle (scalar double precision) on a bounded sample of
                 the same workload, on this host's cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s & % of HBM peak; seq-steps/s at B=32, ctx 8K, d128"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "gqa_decode_attention_kv_amd", "csrc")
# The partial kernel's template and the contiguous-cache instantiation.
KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("decode_partial_kernel.h", "decode_partial.hip",
                                               "launch.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


PREFILL_SRCS = [os.path.join(CSRC, f) for f in ("prefill_kernel.h", "prefill_attn.hip", "prefill_args.h")]


def prefill_source_hash() -> str:
    h = hashlib.sha256()
    for path in PREFILL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, source_hash=None):
    """HBM bytes per partial-kernel launch from the committed counter runs, if
    they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload)
    want = source_hash if source_hash is not None else kernel_source_hash()
    if not rec or rec.get("kernel_source_sha256_16") != want:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inputs, min_seconds: float = 10.0, max_rounds: int = 8) -> dict:
    """Time the oracle (produce + single-pass attention of every head) on whole
    sequences of the workload, one thread per sequence group, until at least
    min_seconds of wall time (or max_rounds sequences groups) have run."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    w = inputs.workload
    o = oracle.load()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    norm = None
    if w.qk_norm.enabled:
        norm = dict(enabled=True, eps=w.qk_norm.eps, offset=w.qk_norm.offset, w_q=inputs.w_q,
                    w_k=inputs.w_k)
    ck, cv = inputs.cache_k, inputs.cache_v
    vs, ks = inputs.v_scale, inputs.k_scale
    t0 = time.perf_counter()
    q = o.kv_produce(rope=w.rope.as_dict(), norm=norm, q_in=inputs.q_in, k_in=inputs.k_in,
                     v_in=inputs.v_in, positions=inputs.positions, k_dtype=w.k_dtype,
                     v_dtype=w.v_dtype, cache_k=ck, cache_v=cv, v_scale=vs, k_scale=ks)
    t_produce = time.perf_counter() - t0
    seqs_done, kv_bytes, elapsed = 0, 0, t_produce
    order = list(range(w.batch))
    per_round = min(w.batch, threads)
    rounds = 0
    while rounds < max_rounds and (elapsed < min_seconds or rounds == 0):
        seqs = [order[(rounds * per_round + i) % w.batch] for i in range(per_round)]

        def one(b):
            pairs = [(b, h) for h in range(w.n_heads)]
            o.decode(q=q, cache_k=ck, cache_v=cv, v_scale=vs, k_scale=ks, k_dtype=w.k_dtype,
                     v_dtype=w.v_dtype, seq_lens=inputs.seq_lens, window=w.window,
                     softcap=w.softcap, pairs=pairs, sinks=inputs.sinks)

        t0 = time.perf_counter()
        with ThreadPoolExecutor(per_round) as ex:
            list(ex.map(one, seqs))
        elapsed += time.perf_counter() - t0
        for b in seqs:
            lo, hi = w.visible(int(inputs.seq_lens[b]))
            kv_bytes += (hi - lo) * w.n_kv_heads * w.kv_row_bytes()
        seqs_done += len(seqs)
        rounds += 1
    gbs = kv_bytes / elapsed / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": per_round, "kind": "oracle",
            "sample": (f"{seqs_done} sequence-steps of {w.name} (produce for all {w.batch} sequences, "
                       f"then single-pass double-precision attention of all {w.n_heads} heads of "
                       f"each sampled sequence), {elapsed:.1f} s wall on {per_round} threads"),
            "seq_steps_per_s": round(seqs_done / elapsed, 3)}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_cpu_baseline(inputs, q, min_seconds: float = 10.0) -> dict:
    """Time the oracle's chunk attention on a bounded sample of (sequence,
    token, head) queries of the workload, on this host's cores."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    w = inputs.workload
    o = oracle.load()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    rng = np.random.default_rng(5)
    T, lens = w.chunk, inputs.seq_lens
    flops, elapsed, n = 0, 0.0, 0
    while elapsed < min_seconds and n < 64 * threads:
        tr = [(int(rng.integers(w.batch)), int(rng.integers(T)), int(rng.integers(w.n_heads)))
              for _ in range(threads)]

        def one(x):
            o.prefill(q=q, cache_k=inputs.cache_k, cache_v=inputs.cache_v, v_scale=inputs.v_scale,
                      k_scale=inputs.k_scale, k_dtype=w.k_dtype, v_dtype=w.v_dtype, seq_lens=lens,
                      window=w.window, softcap=w.softcap, sinks=inputs.sinks, triples=[x])

        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, tr))
        elapsed += time.perf_counter() - t0
        for b, t, _ in tr:
            p = int(lens[b]) - T + t
            lo = max(0, p + 1 - w.window) if w.window > 0 else 0
            flops += 4 * w.head_dim * (p + 1 - lo)
        n += len(tr)
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{n} (sequence, token, head) queries of {w.name}, each its double-precision "
                       f"attention over its causal prefix, {elapsed:.1f} s wall on {threads} threads")}


def prefill_main(args) -> int:
    """One JSON line for a chunk (prefill) workload: the chunk producer plus
    the chunk's causal attention per step; roofline of the attention kernel
    against the bf16 matrix-core peak."""
    import numpy as np
    import torch

    from gqa_decode_attention_kv_amd import workloads as W
    from gqa_decode_attention_kv_amd.step import DevicePrefill

    name = args.prefill
    w = W.PREFILL[name]
    inputs = W.make_prefill_inputs(w)
    paged = W.make_paged(inputs, args.paged) if args.paged else None
    st = DevicePrefill(inputs, paged=paged)
    flops = W.prefill_flops(w, inputs.seq_lens)
    t_w, n_w = time.perf_counter(), 0
    while n_w < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        st.step()
        n_w += 1
        if n_w % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    K = args.steps
    EVERY = 5
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range((K + EVERY - 1) // EVERY)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        st.produce()
        if i % EVERY == 0:
            ev[i // EVERY][0].record()
            st.attn()
            ev[i // EVERY][1].record()
        else:
            st.attn()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / K
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    assert torch.isfinite(st.out).all().item(), "non-finite output"
    tflops_step = flops / (ms_step * 1e-3) / 1e12
    tflops_attn = flops / (attn_ms * 1e-3) / 1e12
    tokens = w.batch * w.chunk
    result = {
        "metric": "prefill chunk attention TFLOP/s (algorithmic) and tokens/s",
        "value": round(tflops_step, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": n_w, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "batch": w.batch, "chunk": w.chunk,
                   "ctx": int(inputs.seq_lens.max()), "n_heads": w.n_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "kv_cache": {(1, 1): "bf16/bf16", (1, 2): "bf16/int8(vq8)",
                                (2, 2): "q8"}[(w.k_dtype, w.v_dtype)],
                   "window": w.window, "softcap": w.softcap,
                   "layout": f"paged(block_size={args.paged})" if args.paged else "contiguous",
                   "parallelism": "single-gpu"},
        "tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "flops_per_step": flops,
        "attn_ms": round(attn_ms, 5),
        "roofline": {"kernel": "prefill_attn_kernel", "bound": "mfma",
                     "achieved": round(tflops_attn, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops_attn / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if args.paged else measured_traffic(name, prefill_source_hash()),
                     "algorithmic_flops_per_launch": flops,
                     "kernel_source_sha256_16": prefill_source_hash(),
                     "note": "the kernel issues twice the algorithmic matrix flops (q and the "
                             "softmax weights enter as a bf16 high part and remainder)"},
    }
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.load()
        ck, cv = inputs.cache_k.copy(), inputs.cache_v.copy()
        vs = inputs.v_scale.copy() if inputs.v_scale is not None else None
        ks = inputs.k_scale.copy() if inputs.k_scale is not None else None
        norm = None
        if w.qk_norm.enabled:
            norm = dict(enabled=True, eps=w.qk_norm.eps, offset=w.qk_norm.offset,
                        w_q=inputs.w_q, w_k=inputs.w_k)
        q = o.kv_produce_chunk(rope=w.rope.as_dict(), norm=norm, q_in=inputs.q_in,
                               k_in=inputs.k_in, v_in=inputs.v_in, start_positions=inputs.start,
                               k_dtype=w.k_dtype, v_dtype=w.v_dtype, cache_k=ck, cache_v=cv,
                               v_scale=vs, k_scale=ks)
        inputs.cache_k, inputs.cache_v, inputs.v_scale, inputs.k_scale = ck, cv, vs, ks
        result["cpu_baseline"] = prefill_cpu_baseline(inputs, q)
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="keep warming up until this much wall time has passed (clocks settle)")
    ap.add_argument("--workload", default=None, help="workload name (default: the B=32 ctx-8K one)")
    ap.add_argument("--split-size", type=int, default=None)
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK_SIZE",
                    help="use the paged cache layout with this block size (0: contiguous)")
    ap.add_argument("--fused", action="store_true",
                    help="run the step as one launch (uaii_decode_step) instead of three calls")
    ap.add_argument("--prefill", default=None, metavar="WORKLOAD",
                    help="time a chunk (prefill) workload instead of the decode step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this decode path runs on one GPU "
              "(the kernel on one GPU's share); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from gqa_decode_attention_kv_amd import workloads as W
    from gqa_decode_attention_kv_amd.step import DeviceStep

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_probe:
        # A plain 1 GiB device copy: the counters' reading of it calibrates
        # FETCH_SIZE and WRITE_SIZE against known bytes.
        n = 1 << 28  # 1 GiB of f32
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"bench: copy probe moved {n * 4} bytes each way", file=sys.stderr, flush=True)
        del src, dst
    if args.prefill:
        return prefill_main(args)
    name = args.workload or W.HEADLINE
    w = W.WORKLOADS[name]
    t_gen = time.perf_counter()
    inputs = W.make_inputs(w)
    t_gen = time.perf_counter() - t_gen
    print(f"bench: {name} inputs generated in {t_gen:.1f} s", file=sys.stderr, flush=True)
    paged = W.make_paged(inputs, args.paged) if args.paged else None
    st = DeviceStep(inputs, split_size=args.split_size, paged=paged)
    kv_bytes = w.kv_bytes()

    # Warm-up: at least --warmup steps and --min-warmup-s seconds.  The first
    # tens of milliseconds of GPU work in a process can run several times
    # slower than steady state; they are kept out of the timed region.
    t_w = time.perf_counter()
    n_w = 0
    one_step = st.fused_step if args.fused else st.step
    while n_w < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        one_step()
        n_w += 1
        if n_w % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    K = args.steps
    # The partial kernel is bracketed by an event pair on every EVERY-th step
    # (an event pair costs a few microseconds of GPU time; sampling keeps the
    # whole-step time honest while still timing the kernel live).
    EVERY = 10
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range((K + EVERY - 1) // EVERY)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        if args.fused:
            # The single launch is the whole step and its dominant kernel.
            if i % EVERY == 0:
                ev[i // EVERY][0].record()
                st.fused_step()
                ev[i // EVERY][1].record()
            else:
                st.fused_step()
            continue
        st.produce()
        if i % EVERY == 0:
            ev[i // EVERY][0].record()
            st.attn()
            ev[i // EVERY][1].record()
        else:
            st.attn()
        st.combine()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / K
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_mean = float(np.mean(attn_ms))
    assert torch.isfinite(st.out).all().item(), "non-finite output"

    step_gbs = kv_bytes / (ms_step * 1e-3) / 1e9
    attn_gbs = kv_bytes / (attn_mean * 1e-3) / 1e9
    traffic = measured_traffic(name) if not (args.paged or args.fused) else None
    result = {
        "metric": METRIC,
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": n_w,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "batch": w.batch, "ctx": int(inputs.seq_lens.max()),
                   "n_heads": w.n_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "kv_cache": ("q8" if w.k_dtype == 2 else
                                {0: "f32", 1: "bf16"}[w.k_dtype] + "/" +
                                {0: "f32", 1: "bf16", 2: "int8(vq8)"}[w.v_dtype]),
                   "split_size": st.split_size, "window": w.window, "softcap": w.softcap,
                   "rope_scaling": {0: "plain", 1: "llama3", 2: "linear", 3: "yarn"}[w.rope.scaling],
                   "attention_sink": w.sink,
                   "layout": f"paged(block_size={args.paged})" if args.paged else "contiguous",
                   "launches_per_step": 1 if args.fused else 3,
                   "parallelism": "single-gpu"},
        "pct_hbm_peak": round(100.0 * step_gbs / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(w.batch / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "attn_partial_ms": round(attn_mean, 5),
        "wall_s_timed": round(wall, 3),
        "roofline": {
            "kernel": ("decode_partial_kernel (single-launch step)" if args.fused
                       else "decode_partial_kernel"),
            "bound": "hbm",
            "achieved": round(attn_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "kernel_source_sha256_16": kernel_source_hash(),
        },
    }
    if not args.no_cpu_baseline:
        del st
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
