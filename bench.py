#!/usr/bin/env python3
"""Benchmark of one GQA decode step on one MI355X.

A step is the whole hot path over one batch: KV producer (norm, RoPE,
append), split-K decode partials, log-sum-exp combine, all through the C ABI
on the current stream.  Inputs are seeded synthetic caches already resident
in HBM when the timed region starts.

Prints ONE JSON line:
  value          KV GB/s of the whole step (algorithmic visible-KV bytes / step time)
  roofline       the dominant kernel (decode partials): algorithmic bytes per launch
                 / its mean launch time (50 or more launches back to back under
                 one HIP event pair on the launch stream, right behind the timed
                 steps), against the 8 TB/s HBM peak; traffic from rocprofv3
                 counters when they were taken on the current kernel source,
                 else null
  hbm_stream_probe  a plain streaming read of 1 GiB run before the warm-up: the
                 read rate this part sustains in practice
                 (--stream-probe alone; --gather-probe BYTES reads the same
                 bytes in scattered pieces, a paged cache's pattern, or with
                 --gather-order kv the contiguous cache's K and V in turn)
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


def host_cpu() -> dict:
    """Host core counts and CPU model: every core the host has, the cores this
    process may run on (its affinity mask), and the thread budget used here,
    which is that mask capped at 16 (the host-core share of one GPU's job)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"host_cores": os.cpu_count() or affinity, "affinity_cores": affinity,
            "threads": max(1, min(16, affinity)), "cpu_model": model}


def _oracle_decode_rate(o, q, inputs, threads: int, min_seconds: float, max_seqs: int) -> dict:
    """Single-pass oracle attention of all heads of whole sequences, `threads`
    sequences at a time, until min_seconds of wall time or max_seqs sequences."""
    from concurrent.futures import ThreadPoolExecutor

    w = inputs.workload
    ck, cv = inputs.cache_k, inputs.cache_v
    vs, ks = inputs.v_scale, inputs.k_scale

    def one(b):
        pairs = [(b, h) for h in range(w.n_heads)]
        o.decode(q=q, cache_k=ck, cache_v=cv, v_scale=vs, k_scale=ks, k_dtype=w.k_dtype,
                 v_dtype=w.v_dtype, seq_lens=inputs.seq_lens, window=w.window,
                 softcap=w.softcap, pairs=pairs, sinks=inputs.sinks)

    seqs_done, kv_bytes, elapsed, rounds = 0, 0, 0.0, 0
    with ThreadPoolExecutor(threads) as ex:
        while seqs_done < max_seqs and (elapsed < min_seconds or rounds == 0):
            seqs = [(seqs_done + i) % w.batch for i in range(threads)]
            t0 = time.perf_counter()
            list(ex.map(one, seqs))
            elapsed += time.perf_counter() - t0
            for b in seqs:
                lo, hi = w.visible(int(inputs.seq_lens[b]))
                kv_bytes += (hi - lo) * w.n_kv_heads * w.kv_row_bytes()
            seqs_done += len(seqs)
            rounds += 1
    return {"value": round(kv_bytes / elapsed / 1e9, 4), "unit": "GB/s", "threads": threads,
            "seq_steps_per_s": round(seqs_done / elapsed, 3), "sequences": seqs_done,
            "seconds": round(elapsed, 2)}


def cpu_baseline(inputs, min_seconds: float = 8.0) -> dict:
    """Time the oracle as it stands (scalar double precision, no tuning) on a
    bounded sample of the workload: the producer for every sequence, then the
    single-pass attention of every head of whole sequences, once on one
    thread and once on all the threads this job may use."""
    import oracle

    w = inputs.workload
    o = oracle.load()
    cpu = host_cpu()
    norm = None
    if w.qk_norm.enabled:
        norm = dict(enabled=True, eps=w.qk_norm.eps, offset=w.qk_norm.offset, w_q=inputs.w_q,
                    w_k=inputs.w_k)
    t0 = time.perf_counter()
    q = o.kv_produce(rope=w.rope.as_dict(), norm=norm, q_in=inputs.q_in, k_in=inputs.k_in,
                     v_in=inputs.v_in, positions=inputs.positions, k_dtype=w.k_dtype,
                     v_dtype=w.v_dtype, cache_k=inputs.cache_k, cache_v=inputs.cache_v,
                     v_scale=inputs.v_scale, k_scale=inputs.k_scale)
    t_produce = time.perf_counter() - t0
    one = _oracle_decode_rate(o, q, inputs, 1, min_seconds / 2, max_seqs=w.batch)
    allc = _oracle_decode_rate(o, q, inputs, cpu["threads"], min_seconds, max_seqs=8 * w.batch)
    return {"value": allc["value"], "unit": "GB/s", "cores": cpu["threads"], "kind": "oracle",
            "sample": (f"{w.name}: the producer for all {w.batch} sequences ({t_produce:.2f} s, "
                       f"one thread), then double-precision single-pass attention of all "
                       f"{w.n_heads} heads of whole sequences: {allc['sequences']} sequence-steps "
                       f"in {allc['seconds']} s on {allc['threads']} threads (the job's core "
                       f"share), {one['sequences']} in {one['seconds']} s on 1 thread"),
            "seq_steps_per_s": allc["seq_steps_per_s"],
            "threads_1": one, "threads_all": allc,
            "host_cores": cpu["host_cores"], "affinity_cores": cpu["affinity_cores"],
            "cpu_model": cpu["cpu_model"]}


PROBE_LIBRARY = os.path.join(ROOT, "gqa_decode_attention_kv_amd", "libuaii_probe.so")


GATHER_ORDERS = {
    "random": "seeded random permutation",
    "sequential": "sequential",
    "kv": "the two halves in turn, one piece each",
}


def gather_order(n_pieces: int, per: int, order_kind: str):
    """The piece indices of gather_probe, a permutation of range(n_pieces)
    read per pieces at a time by each work-group (int64 CPU tensor)."""
    import torch

    if order_kind == "random":
        gen = torch.Generator().manual_seed(20240611)
        order = torch.randperm(n_pieces, generator=gen)
    elif order_kind == "sequential":
        order = torch.arange(n_pieces)
    elif order_kind == "kv":
        if per % 2 or n_pieces % per:
            raise ValueError("the kv order needs an even number of pieces per group dividing the buffer")
        halfper = per // 2
        base = torch.arange(n_pieces // per)[:, None] * halfper + torch.arange(halfper)[None, :]
        order = torch.stack([base, base + n_pieces // 2], dim=-1).reshape(-1)
    else:
        raise ValueError(f"unknown gather order {order_kind!r} (one of {sorted(GATHER_ORDERS)})")
    assert order.numel() == n_pieces and int(order.min()) >= 0 and int(order.max()) < n_pieces
    return order


def gather_probe(piece_bytes: int, order_kind: str = "random", nbytes: int = 1 << 30,
                 per_group: int = 2 << 20, min_seconds: float = 0.3) -> dict:
    """The read ceiling of a decode kernel's access pattern: nbytes of device
    memory read as pieces of piece_bytes, per_group bytes of pieces per
    work-group of four waves, 16-byte non-temporal loads; timed like
    stream_probe.  order_kind "random" takes the pieces in a seeded random
    order (a paged cache: one piece is one cache block of one kv head, e.g.
    4096 = 16 rows of d128 bf16); "kv" gives each work-group consecutive
    pieces of both halves of the buffer in turn (the contiguous cache's K
    and V arrays read chunk by chunk, e.g. 131072 = 512 rows of d128 bf16);
    "sequential" reads every group's range in order (the control: it should
    match stream_probe)."""
    import ctypes as C

    import torch

    if not os.path.exists(PROBE_LIBRARY):
        raise RuntimeError(f"{PROBE_LIBRARY} is missing; run __graft_entry__.build()")
    lib = C.CDLL(PROBE_LIBRARY)
    lib.uaii_probe_gather_read.restype = C.c_int
    lib.uaii_probe_gather_read.argtypes = [C.c_void_p, C.c_size_t, C.c_size_t, C.c_void_p, C.c_int,
                                           C.c_int, C.c_void_p, C.c_void_p]
    n_pieces = nbytes // piece_bytes
    per = max(1, per_group // piece_bytes)
    order = gather_order(n_pieces, per, order_kind)
    order = order.to(torch.int32).to("cuda")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(-(-n_pieces // per), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.uaii_probe_gather_read(src.data_ptr(), n_pieces, piece_bytes, order.data_ptr(), n_pieces, per,
                                        sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"uaii_probe_gather_read failed ({rc})")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(20):
            launch()
        n_settle += 20
        torch.cuda.synchronize()
    reps = 100
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        launch()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    gbs = n_pieces * piece_bytes / (us * 1e-6) / 1e9
    del src, sink, order
    torch.cuda.empty_cache()
    return {"kernel": "gather_read_kernel", "bytes": n_pieces * piece_bytes, "piece_bytes": piece_bytes,
            "pieces_per_group": per, "order": GATHER_ORDERS[order_kind],
            "us_per_launch": round(us, 2), "achieved": round(gbs, 1), "unit": "GB/s",
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "launches": n_settle + reps}


def stream_probe(nbytes: int = 1 << 30, per_group: int = 2 << 20, min_seconds: float = 0.3) -> dict:
    """The practical HBM read ceiling: a plain streaming read of nbytes of
    device memory (16-byte non-temporal loads, one sequential stream per
    work-group of four waves, per_group bytes each), launched back to back
    for at least min_seconds; the rate comes from one event pair around the
    last launches.  Running it first also brings the clocks to steady state
    before the decode step is warmed up."""
    import ctypes as C

    import torch

    if not os.path.exists(PROBE_LIBRARY):
        raise RuntimeError(f"{PROBE_LIBRARY} is missing; run __graft_entry__.build()")
    lib = C.CDLL(PROBE_LIBRARY)
    lib.uaii_probe_stream_read.restype = C.c_int
    lib.uaii_probe_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_size_t, C.c_void_p,
                                           C.c_void_p]
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    groups = -(-nbytes // per_group)
    sink = torch.zeros(groups, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.uaii_probe_stream_read(src.data_ptr(), nbytes, per_group, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"uaii_probe_stream_read failed ({rc})")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(20):
            launch()
        n_settle += 20
        torch.cuda.synchronize()
    reps = 100
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        launch()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    gbs = nbytes / (us * 1e-6) / 1e9
    del src, sink
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel", "bytes": nbytes, "bytes_per_group": per_group, "groups": groups,
            "us_per_launch": round(us, 2), "achieved": round(gbs, 1), "unit": "GB/s",
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "launches": n_settle + reps}


def settle_kernel(launch, seconds: float, kernel: str) -> dict:
    """Launch a kernel back to back, untimed, for `seconds` of wall time."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            launch(n)
            n += 1
        torch.cuda.synchronize()
    return {"kernel": kernel, "launches": n, "seconds": round(time.perf_counter() - t0, 3)}


MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3


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
    against the matrix-core peak of its operand type (bf16, or f32 for f32
    caches)."""
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
    probe = None if args.no_stream_probe else stream_probe()
    settle = settle_kernel(lambda i: st.attn(), args.settle_s, "prefill_attn_kernel")
    n_w = args.warmup
    for i in range(n_w):
        st.step()
    torch.cuda.synchronize()
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        st.step()
    stop.record()
    # The attention kernel alone: max(50, K) launches back to back under one
    # event pair, queued right behind the timed steps.
    n_loop = max(50, K)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n_loop):
        st.attn()
    b.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / K
    attn_ms = a.elapsed_time(b) / n_loop
    assert torch.isfinite(st.out).all().item(), "non-finite output"
    tflops_step = flops / (ms_step * 1e-3) / 1e12
    tflops_attn = flops / (attn_ms * 1e-3) / 1e12
    tokens = w.batch * w.chunk
    f32_cache = (w.k_dtype, w.v_dtype) == (0, 0)
    peak = MFMA_F32_PEAK_TFLOPS if f32_cache else MFMA_BF16_PEAK_TFLOPS
    result = {
        "metric": "prefill chunk attention TFLOP/s (algorithmic) and tokens/s",
        "value": round(tflops_step, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": n_w, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if f32_cache else "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch": w.batch, "chunk": w.chunk,
                   "ctx": int(inputs.seq_lens.max()), "n_heads": w.n_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "kv_cache": {(1, 1): "bf16/bf16", (1, 2): "bf16/int8(vq8)",
                                (2, 2): "q8", (0, 0): "f32/f32"}[(w.k_dtype, w.v_dtype)],
                   "window": w.window, "softcap": w.softcap,
                   "layout": f"paged(block_size={args.paged})" if args.paged else "contiguous",
                   "parallelism": "single-gpu"},
        "tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "flops_per_step": flops,
        "attn_ms": round(attn_ms, 5),
        "attn_launches_timed": n_loop,
        "settle": settle,
        "hbm_stream_probe": probe,
        "roofline": {"kernel": "prefill_attn_kernel", "bound": "mfma",
                     "achieved": round(tflops_attn, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops_attn / peak, 4),
                     "traffic": None if args.paged else measured_traffic(name, prefill_source_hash()),
                     "algorithmic_flops_per_launch": flops,
                     "kernel_source_sha256_16": prefill_source_hash(),
                     "note": "f32 caches: f32 matrix products, the algorithmic flops" if f32_cache else
                             "the kernel issues twice the algorithmic matrix flops (q and the "
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
    ap.add_argument("--copies", type=int, default=0,
                    help="rotate among this many copies of the device buffers (0: one copy "
                         "from 1 GiB of visible KV up, else enough to pass 2 GiB, at most 8)")
    ap.add_argument("--settle-s", type=float, default=0.2,
                    help="run the dominant kernel alone, untimed, for this long before the "
                         "warm-up steps (its first launches in a process are slow)")
    ap.add_argument("--no-stream-probe", action="store_true",
                    help="skip the streaming-read probe that runs before the warm-up")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only run the streaming-read probe (1 GiB) and print its JSON line")
    ap.add_argument("--stream-mib", type=int, default=1024, metavar="M",
                    help="with --stream-probe: read M MiB instead of 1 GiB (512 work-groups unless "
                         "--stream-groups is given)")
    ap.add_argument("--stream-groups", type=int, default=0, metavar="G",
                    help="with --stream-probe: split the read into G equal work-group streams "
                         "(default 512, 2 MiB each for 1 GiB); G not a multiple of the 256 CUs "
                         "leaves some CUs more streams than others")
    ap.add_argument("--gather-probe", type=int, default=0, metavar="PIECE_BYTES",
                    help="only run the scattered-piece read probe (1 GiB in pieces of PIECE_BYTES, "
                         "a paged cache's pattern) and print its JSON line")
    ap.add_argument("--gather-order", default="random", choices=sorted(GATHER_ORDERS),
                    help="order of the pieces of --gather-probe: random (a paged cache), kv (the "
                         "contiguous cache's K and V chunks in turn) or sequential (the control)")
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
    if args.gather_probe:
        probe = gather_probe(args.gather_probe, args.gather_order)
        wl = f"gather-read-1GiB-{args.gather_probe}B-pieces"
        if args.gather_order != "random":
            wl += f"-{args.gather_order}"
        print(json.dumps({"metric": "read of device memory in scattered pieces, GB/s",
                          "value": probe["achieved"], "unit": "GB/s", "n_gpus": 1,
                          "higher_is_better": True, "data": "synthetic",
                          "config": {"workload": wl},
                          "probe": probe}), flush=True)
        return 0
    if args.stream_probe:
        if args.stream_mib < 1 or args.stream_mib > (64 << 10):
            print("bench.py: --stream-mib must be in 1..65536", file=sys.stderr)
            return 2
        nbytes = args.stream_mib << 20
        wl = "stream-read-1GiB" if args.stream_mib == 1024 else f"stream-read-{args.stream_mib}MiB"
        groups = args.stream_groups or 512
        if groups < 1 or groups > (1 << 20):
            print("bench.py: --stream-groups must be in 1..1048576", file=sys.stderr)
            return 2
        per = -(-nbytes // groups)  # bytes per work-group, rounded up
        per = -(-per // 16) * 16     # to whole 16-byte loads
        probe = stream_probe(nbytes=nbytes, per_group=per)
        if args.stream_groups:
            wl += f"-{-(-nbytes // per)}-groups"
        print(json.dumps({"metric": "plain streaming read of device memory, GB/s",
                          "value": probe["achieved"], "unit": "GB/s", "n_gpus": 1,
                          "higher_is_better": True, "data": "synthetic",
                          "config": {"workload": wl}, "probe": probe}), flush=True)
        return 0
    if args.prefill:
        return prefill_main(args)
    name = args.workload or W.HEADLINE
    w = W.WORKLOADS[name]
    t_gen = time.perf_counter()
    inputs = W.make_inputs(w)
    t_gen = time.perf_counter() - t_gen
    print(f"bench: {name} inputs generated in {t_gen:.1f} s", file=sys.stderr, flush=True)
    paged = W.make_paged(inputs, args.paged) if args.paged else None
    kv_bytes = w.kv_bytes()
    # Workloads whose visible bytes are under 1 GiB rotate among R copies of
    # their device buffers (same contents, other addresses), so that the
    # copies together exceed the last-level cache and every step streams
    # from HBM.
    R = args.copies if args.copies > 0 else (1 if kv_bytes >= (1 << 30) else
                                             min(8, -(-(2 << 30) // kv_bytes)))
    steps = [DeviceStep(inputs, split_size=args.split_size, paged=paged) for _ in range(R)]
    st = steps[0]

    # The practical read ceiling first.
    probe = None if args.no_stream_probe else stream_probe()
    # Then the dominant kernel alone, back to back and untimed, for
    # --settle-s seconds: on this part the first hundred or so launches after
    # the GPU has been idle (at process start, or after a tenth of a second
    # of host work) run up to 20% slower while the clocks come back up (the
    # partial kernel at B=32 ctx 8K: about 180 us falling to 155 us over
    # about 15 ms), so without this the --warmup steps alone would not reach
    # the steady state being measured.
    settle = settle_kernel(lambda i: (steps[i % R].fused_step() if args.fused else steps[i % R].attn()),
                           args.settle_s, "decode_step (one launch)" if args.fused
                           else "decode_partial_kernel")

    n_w = args.warmup
    for i in range(n_w):
        steps[i % R].fused_step() if args.fused else steps[i % R].step()
    torch.cuda.synchronize()

    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        if args.fused:
            steps[i % R].fused_step()
        else:
            steps[i % R].step()
    stop.record()

    # The dominant kernel alone (the partials; with --fused the single
    # launch): max(50, K) launches back to back under one event pair on the
    # step's stream, queued right behind the timed steps.  Nothing waits in
    # between: after even a short idle spell (a tenth of a second of host
    # work) this part runs the next hundred or so partial launches up to 20%
    # slower while its clocks come back up.
    n_loop = max(50, K)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n_loop):
        steps[i % R].fused_step() if args.fused else steps[i % R].attn()
    b.record()
    stop.synchronize()
    wall = time.perf_counter() - t0
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / K
    attn_mean = a.elapsed_time(b) / n_loop
    for st in steps:
        assert torch.isfinite(st.out).all().item(), "non-finite output"
    consistent = bool(args.fused or attn_mean <= ms_step)
    if not consistent:
        print(f"bench: partial kernel {attn_mean:.5f} ms per launch exceeds the whole step "
              f"({ms_step:.5f} ms)", file=sys.stderr, flush=True)

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
        "attn_launches_timed": n_loop,
        "attn_partial_le_step": consistent,
        "settle": settle,
        "cache_copies": R,
        "wall_s_timed": round(wall, 3),
        "hbm_stream_probe": probe,
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
        del st, steps
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
