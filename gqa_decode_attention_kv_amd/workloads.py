"""Seeded synthetic workloads for the GQA decode step.

This module only draws random inputs and describes shapes; it holds none of
the step's arithmetic (no norm, rotation, rounding to a cache format chosen
by the method, quantiser or softmax).  The GPU path and the CPU oracle both
consume what it returns, as data.

Recipe (every draw is ``numpy.random.default_rng([seed, stream, ...])``,
standard normal float32 unless stated):
  * lengths: fixed, or uniform integers in [lo, hi] (stream 0);
  * q_in [B][H][d], k_in and v_in [B][Hkv][d]: streams 1, 2, 3;
  * QK-norm weights w_q, w_k [d]: stream 4, as mean + std * N(0, 1);
  * cached keys and values: one block per (b, kv head), streams 5 (K) and
    6 (V), filling only the visible cached rows [lo_b, L_b - 1).  bf16
    entries keep the top 16 bits of the float32 draw (a random bf16 number);
    f32 entries are the draw itself.  int8 rows are drawn directly as codes
    (rounded N(0,1) * 127 / 2.8, clipped to +-127) with an f32 scale near
    2.8 / 127: values from stream 7, q8 keys from stream 9;
  * attention sinks (one logit per query head): 2 + 3 * N(0, 1), stream 10;
  * every other cache row (before the window, the new token's slot and
    beyond) holds a NaN poison (int8 codes 0 with a NaN scale), so a kernel
    that reads outside the visible range cannot pass a test.

Blocks are filled from a thread pool; each block has its own seed, so the
result does not depend on the number of threads.

Paged caches (``make_paged``) hold the same logical rows: logical block j of
sequence b is copied to physical block table[b][j] of a pool
[num_blocks][Hkv][block_size][d], where the table is a seeded random
permutation of the pool (stream 8) and a few blocks stay unused.  Every pool
row that no logical row maps to is NaN-poisoned, like the invisible rows.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

F32, BF16, I8 = 0, 1, 2
NEOX, INTERLEAVED = 0, 1
PLAIN, LLAMA3, LINEAR, YARN = 0, 1, 2, 3

BF16_NAN = np.uint16(0x7FC0)
STORAGE = {F32: np.float32, BF16: np.uint16, I8: np.int8}
ELEM_BYTES = {F32: 4, BF16: 2, I8: 1}


@dataclass(frozen=True)
class Rope:
    pairing: int = NEOX
    scaling: int = PLAIN
    theta: float = 10000.0
    factor: float = 1.0
    low: float = 1.0
    high: float = 4.0
    orig: int = 8192
    truncate: bool = True      # YaRN: round the blend edges to whole pair indices
    attn_factor: float = 0.0   # YaRN: 0 = 1 + 0.1 ln(factor)

    def as_dict(self) -> dict:
        return dict(pairing=self.pairing, scaling=self.scaling, theta=self.theta,
                    factor=self.factor, low=self.low, high=self.high, orig=self.orig,
                    truncate=self.truncate, attn_factor=self.attn_factor)


@dataclass(frozen=True)
class QKNorm:
    enabled: bool = False
    eps: float = 1e-6
    offset: int = 0
    w_mean: float = 1.0
    w_std: float = 0.1


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    lens: tuple            # ("fixed", L) or ("uniform", lo, hi): keys incl. the new one
    capacity: int
    k_dtype: int = BF16
    v_dtype: int = BF16
    rope: Rope = field(default_factory=Rope)
    qk_norm: QKNorm = field(default_factory=QKNorm)
    window: int = 0
    softcap: float = 0.0
    split_size: int = 512
    seed: tuple = (0,)
    sink: bool = False         # a per-head attention sink in the combine
    chunk: int = 0             # prefill: new tokens per sequence (0: a decode step)

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    def seq_lens(self) -> np.ndarray:
        if self.lens[0] == "fixed":
            return np.full(self.batch, self.lens[1], dtype=np.int32)
        _, lo, hi = self.lens
        rng = np.random.default_rng([*self.seed, 0])
        return rng.integers(lo, hi, endpoint=True, size=self.batch).astype(np.int32)

    def visible(self, L: int) -> tuple[int, int]:
        """[lo, L): keys attended by a sequence of L keys (window counts the new key)."""
        lo = L - self.window if (self.window > 0 and L > self.window) else 0
        return lo, L

    def max_splits(self) -> int:
        return int(-(-int(self.seq_lens().max()) // self.split_size))

    def kv_row_bytes(self) -> int:
        """Algorithmic bytes per visible (token, kv head): K row + V row (+ int8 scales)."""
        d = self.head_dim
        b = d * ELEM_BYTES[self.k_dtype] + d * ELEM_BYTES[self.v_dtype]
        return b + (4 if self.v_dtype == I8 else 0) + (4 if self.k_dtype == I8 else 0)

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode step reads (visible rows only)."""
        rows = sum(hi - lo for lo, hi in (self.visible(int(L)) for L in self.seq_lens()))
        return rows * self.n_kv_heads * self.kv_row_bytes()


# The workloads of the decode step.  Names give the model shape they follow.
# Split sizes: 2 splits for the tiny step and 512 for the Llama-3.2-1B shape, as
# those workloads are defined; elsewhere the size is a tuned launch parameter
# (measured best on MI355X; the sizes are reported with every result).
WORKLOADS = {
    # 128 cached tokens plus the new one at position 128; two splits of 65 keys.
    "tiny": Workload("tiny", 1, 4, 2, 64, ("fixed", 129), 129, F32, F32,
                     Rope(NEOX, PLAIN, 10000.0), split_size=65, seed=(1,)),
    "llama3.2-1b": Workload("llama3.2-1b", 1, 32, 8, 64, ("fixed", 4096), 4096, BF16, BF16,
                            Rope(INTERLEAVED, LLAMA3, 500000.0, 32.0, 1.0, 4.0, 8192),
                            split_size=512, seed=(2,)),
    "llama3.1-8b-ragged": Workload("llama3.1-8b-ragged", 32, 32, 8, 128, ("uniform", 512, 8192),
                                   8192, BF16, BF16,
                                   Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0, 8192),
                                   split_size=512, seed=(3,)),
    "qwen3-vq8": Workload("qwen3-vq8", 16, 32, 8, 128, ("fixed", 16384), 16384, BF16, I8,
                          Rope(NEOX, PLAIN, 1000000.0),
                          QKNorm(True, 1e-6, 0, 1.0, 0.1), split_size=4096, seed=(4,)),
    "gemma2-local": Workload("gemma2-local", 8, 16, 8, 256, ("fixed", 32768), 32768, BF16, BF16,
                             Rope(NEOX, PLAIN, 10000.0), QKNorm(True, 1e-6, 1, 0.0, 0.1),
                             window=4096, softcap=50.0, split_size=512, seed=(5, 0)),
    "gemma2-global": Workload("gemma2-global", 8, 16, 8, 256, ("fixed", 32768), 32768, BF16, BF16,
                              Rope(NEOX, PLAIN, 1000000.0), QKNorm(True, 1e-6, 1, 0.0, 0.1),
                              window=0, softcap=50.0, split_size=4096, seed=(5, 1)),
    # The same Gemma-2 pair read the other way: the "RMSNorm gain (1 + w)" of
    # the configuration taken as the layer's input norm, off this path, so no
    # QK-norm (same seeds, so the draws are those of the pair above).
    "gemma2-local-noqknorm": Workload("gemma2-local-noqknorm", 8, 16, 8, 256, ("fixed", 32768), 32768,
                                      BF16, BF16, Rope(NEOX, PLAIN, 10000.0), window=4096,
                                      softcap=50.0, split_size=512, seed=(5, 0)),
    "gemma2-global-noqknorm": Workload("gemma2-global-noqknorm", 8, 16, 8, 256, ("fixed", 32768),
                                       32768, BF16, BF16, Rope(NEOX, PLAIN, 1000000.0), window=0,
                                       softcap=50.0, split_size=4096, seed=(5, 1)),
    # The measured workload: B=32 sequences of 8192 keys, 32/8 heads, d=128, bf16 KV.
    # Split size 4096 (tuned): 2 splits per sequence, 512 work items, each taken
    # by one cooperative work-group of four waves (two work-groups per CU).
    "llama3.1-8b-b32-ctx8k": Workload("llama3.1-8b-b32-ctx8k", 32, 32, 8, 128, ("fixed", 8192),
                                      8192, BF16, BF16,
                                      Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0, 8192),
                                      split_size=4096, seed=(6,)),
    # The headline shape with the q8 cache (int8 keys and values, one f32
    # scale each per token per kv head).
    "llama3.1-8b-q8": Workload("llama3.1-8b-q8", 32, 32, 8, 128, ("fixed", 8192), 8192, I8, I8,
                               Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0, 8192),
                               split_size=1024, seed=(7,)),
    # Llama-3.1-70B attention: 64/8 heads of 128 (groups of eight query heads),
    # the headline's batch, context and rotary scaling, over the bf16, q8 and
    # vq8 caches.
    "llama3.1-70b-b32-ctx8k": Workload("llama3.1-70b-b32-ctx8k", 32, 64, 8, 128, ("fixed", 8192), 8192,
                                       BF16, BF16, Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0, 8192),
                                       split_size=4096, seed=(10,)),
    "llama3.1-70b-q8": Workload("llama3.1-70b-q8", 32, 64, 8, 128, ("fixed", 8192), 8192, I8, I8,
                                Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0, 8192),
                                split_size=1024, seed=(11,)),
    "llama3.1-70b-vq8": Workload("llama3.1-70b-vq8", 32, 64, 8, 128, ("fixed", 8192), 8192, BF16, I8,
                                 Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0, 8192),
                                 split_size=4096, seed=(12,)),
    # gpt-oss-20b attention: 64/8 heads of 64, YaRN (theta 150000, factor 32,
    # beta 1..32 over 4096, edges not rounded), a per-head sink, and the exact
    # f32 cache (its sampler moves too far under vq8); full-attention layers
    # and 128-key sliding-window layers alternate.
    "gpt-oss-20b-full": Workload("gpt-oss-20b-full", 32, 64, 8, 64, ("fixed", 8192), 8192, F32, F32,
                                 Rope(NEOX, YARN, 150000.0, 32.0, 1.0, 32.0, 4096, False),
                                 split_size=1024, seed=(8, 0), sink=True),
    "gpt-oss-20b-sliding": Workload("gpt-oss-20b-sliding", 32, 64, 8, 64, ("fixed", 8192), 8192,
                                    F32, F32,
                                    Rope(NEOX, YARN, 150000.0, 32.0, 1.0, 32.0, 4096, False),
                                    window=128, split_size=64, seed=(8, 1), sink=True),
    # Gemma-3-27B attention: 32/16 heads of 128, QK-norm with gain (1 + w),
    # global layers with theta 1e6 and linear scaling 8, local layers with
    # theta 1e4 and a 1024-key window.
    "gemma3-27b-global": Workload("gemma3-27b-global", 8, 32, 16, 128, ("fixed", 32768), 32768,
                                  BF16, BF16, Rope(NEOX, LINEAR, 1000000.0, 8.0),
                                  QKNorm(True, 1e-6, 1, 0.0, 0.1), split_size=8192, seed=(9, 0)),
    "gemma3-27b-local": Workload("gemma3-27b-local", 8, 32, 16, 128, ("fixed", 32768), 32768,
                                 BF16, BF16, Rope(NEOX, PLAIN, 10000.0),
                                 QKNorm(True, 1e-6, 1, 0.0, 0.1), window=1024, split_size=256,
                                 seed=(9, 1)),
}

HEADLINE = "llama3.1-8b-b32-ctx8k"

# Prefill (chunk) workloads: `chunk` new tokens per sequence, `lens` keys in
# total (the chunk included), so lens - chunk tokens are already cached.
# Prompt lengths 160, 256 and 550 are the throughput battery's canonical
# prefill shapes on the Algenta page, with the Qwen3-1.7B (grouped-FA d128,
# QK-norm) and Llama-3.2-1B (d64) shapes it names; the others are a batched
# Llama-3.1-8B prompt, a chunk appended to an 8K context, and a Gemma-2
# local layer (window and softcap, d256).
PREFILL = {
    "prefill-qwen3-1.7b-p550": Workload("prefill-qwen3-1.7b-p550", 1, 16, 8, 128, ("fixed", 550), 550,
                                        BF16, BF16, Rope(NEOX, PLAIN, 1000000.0),
                                        QKNorm(True, 1e-6, 0, 1.0, 0.1), seed=(20,), chunk=550),
    "prefill-llama3.2-1b-p256": Workload("prefill-llama3.2-1b-p256", 1, 32, 8, 64, ("fixed", 256), 256,
                                         BF16, BF16,
                                         Rope(INTERLEAVED, LLAMA3, 500000.0, 32.0, 1.0, 4.0, 8192),
                                         seed=(21,), chunk=256),
    "prefill-llama3.1-8b-b8-p2048": Workload("prefill-llama3.1-8b-b8-p2048", 8, 32, 8, 128,
                                             ("fixed", 2048), 2048, BF16, BF16,
                                             Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0, 8192),
                                             seed=(22,), chunk=2048),
    "prefill-llama3.1-8b-b4-c512-ctx8k": Workload("prefill-llama3.1-8b-b4-c512-ctx8k", 4, 32, 8, 128,
                                                  ("fixed", 8192), 8192, BF16, BF16,
                                                  Rope(INTERLEAVED, LLAMA3, 500000.0, 8.0, 1.0, 4.0,
                                                       8192), seed=(23,), chunk=512),
    # The Qwen3 shape's vq8 cache (bf16 keys, int8 values with an f32 scale
    # per token): a 512-token chunk appended to 15872 cached tokens.
    "prefill-qwen3-vq8-b4-c512-ctx16k": Workload("prefill-qwen3-vq8-b4-c512-ctx16k", 4, 32, 8, 128,
                                                 ("fixed", 16384), 16384, BF16, I8,
                                                 Rope(NEOX, PLAIN, 1000000.0),
                                                 QKNorm(True, 1e-6, 0, 1.0, 0.1), seed=(25,), chunk=512),
    "prefill-gemma2-local-b2-c1024": Workload("prefill-gemma2-local-b2-c1024", 2, 16, 8, 256,
                                              ("fixed", 8192), 8192, BF16, BF16,
                                              Rope(NEOX, PLAIN, 10000.0), QKNorm(True, 1e-6, 1, 0.0, 0.1),
                                              window=4096, softcap=50.0, seed=(24,), chunk=1024),
    # The gpt-oss-20b shape over its exact f32 cache (YaRN, a sink per head):
    # a 512-token chunk appended to 3584 cached tokens, full-attention layer.
    "prefill-gpt-oss-20b-f32-b2-c512-ctx4k": Workload("prefill-gpt-oss-20b-f32-b2-c512-ctx4k", 2, 64, 8, 64,
                                                      ("fixed", 4096), 4096, F32, F32,
                                                      Rope(NEOX, YARN, 150000.0, 32.0, 1.0, 32.0, 4096,
                                                           False),
                                                      sink=True, seed=(26,), chunk=512),
}

PREFILL_HEADLINE = "prefill-llama3.1-8b-b8-p2048"


def shrink(w: Workload, **kw) -> Workload:
    """A copy of w with some fields replaced (for small test variants)."""
    return replace(w, **kw)


@dataclass
class Inputs:
    workload: Workload
    seq_lens: np.ndarray      # [B] int32, keys incl. the new one
    positions: np.ndarray     # [B] int32, slot of the new token = L_b - 1
    q_in: np.ndarray          # [B][H][d] f32
    k_in: np.ndarray          # [B][Hkv][d] f32
    v_in: np.ndarray          # [B][Hkv][d] f32
    w_q: np.ndarray | None    # [d] f32
    w_k: np.ndarray | None
    cache_k: np.ndarray       # [B][Hkv][cap][d] f32 or uint16 (bf16 bits)
    cache_v: np.ndarray       # [B][Hkv][cap][d] f32, uint16 or int8
    v_scale: np.ndarray | None  # [B][Hkv][cap] f32 (int8 values only)
    k_scale: np.ndarray | None = None  # [B][Hkv][cap] f32 (int8 keys only)
    sinks: np.ndarray | None = None    # [H] f32 attention-sink logits


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    np.random.default_rng(seed).standard_normal(dtype=np.float32, out=out)
    return out


def _fill_caches(w: Workload, lens: np.ndarray, first_new: np.ndarray):
    """Caches [B][Hkv][cap][d] whose rows [lo_b, first_new[b]) hold seeded
    values (lo_b: the window start of the token at first_new[b]) and every
    other row the poison; returns (cache_k, cache_v, v_scale, k_scale)."""
    B, Hkv, d, cap = w.batch, w.n_kv_heads, w.head_dim, w.capacity
    s = tuple(w.seed)
    cache_k = np.empty((B, Hkv, cap, d), dtype=STORAGE[w.k_dtype])
    cache_v = np.empty((B, Hkv, cap, d), dtype=STORAGE[w.v_dtype])
    v_scale = np.empty((B, Hkv, cap), dtype=np.float32) if w.v_dtype == I8 else None
    k_scale = np.empty((B, Hkv, cap), dtype=np.float32) if w.k_dtype == I8 else None

    def fill(bu):
        b, u = bu
        first = int(first_new[b])
        lo, _ = w.visible(first + 1)
        n = max(0, first - lo)            # cached visible rows: [lo, first)
        for arr, dt in ((cache_k, w.k_dtype), (cache_v, w.v_dtype)):
            slab = arr[b, u]
            if dt == F32:
                slab[:lo] = np.nan
                slab[lo + n:] = np.nan
            elif dt == BF16:
                slab[:lo] = BF16_NAN
                slab[lo + n:] = BF16_NAN
            else:
                slab[:lo] = 0
                slab[lo + n:] = 0
        def int8_rows(stream, codes, scale):
            rng = np.random.default_rng([*s, stream, b, u])
            z = rng.standard_normal((n, d), dtype=np.float32)
            codes[b, u, lo:lo + n] = np.clip(np.rint(z * (127.0 / 2.8)), -127, 127)
            scale[b, u, lo:lo + n] = (2.8 / 127.0) * (
                1.0 + 0.05 * rng.standard_normal(n, dtype=np.float32))

        if n > 0:
            if w.k_dtype == I8:
                int8_rows(9, cache_k, k_scale)
            else:
                zk = _normal([*s, 5, b, u], (n, d))
                if w.k_dtype == F32:
                    cache_k[b, u, lo:lo + n] = zk
                else:
                    cache_k[b, u, lo:lo + n] = zk.view(np.uint16)[:, 1::2]
            if w.v_dtype == I8:
                int8_rows(7, cache_v, v_scale)
            else:
                zv = _normal([*s, 6, b, u], (n, d))
                if w.v_dtype == F32:
                    cache_v[b, u, lo:lo + n] = zv
                else:
                    cache_v[b, u, lo:lo + n] = zv.view(np.uint16)[:, 1::2]
        for sc in (v_scale, k_scale):
            if sc is not None:
                sc[b, u, :lo] = np.nan
                sc[b, u, lo + n:] = np.nan

    jobs = [(b, u) for b in range(B) for u in range(Hkv)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, jobs))
    return cache_k, cache_v, v_scale, k_scale


def make_inputs(w: Workload, seq_lens=None) -> Inputs:
    B, H, Hkv, d, cap = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.capacity
    lens = w.seq_lens() if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    if lens.shape != (B,) or lens.min() < 1 or lens.max() > cap:
        raise ValueError(f"{w.name}: seq_lens must be [{B}] within [1, {cap}]")
    s = tuple(w.seed)
    q_in = _normal([*s, 1], (B, H, d))
    k_in = _normal([*s, 2], (B, Hkv, d))
    v_in = _normal([*s, 3], (B, Hkv, d))
    w_q = w_k = None
    if w.qk_norm.enabled:
        z = _normal([*s, 4], (2, d))
        w_q = (w.qk_norm.w_mean + w.qk_norm.w_std * z[0]).astype(np.float32)
        w_k = (w.qk_norm.w_mean + w.qk_norm.w_std * z[1]).astype(np.float32)

    sinks = (2.0 + 3.0 * _normal([*s, 10], (H,))).astype(np.float32) if w.sink else None
    cache_k, cache_v, v_scale, k_scale = _fill_caches(w, lens, (lens - 1).astype(np.int64))
    return Inputs(w, lens, (lens - 1).astype(np.int32), q_in, k_in, v_in, w_q, w_k,
                  cache_k, cache_v, v_scale, k_scale, sinks)


@dataclass
class PrefillInputs:
    workload: Workload
    seq_lens: np.ndarray      # [B] int32, keys incl. the chunk
    start: np.ndarray         # [B] int32, position of the chunk's first token = L_b - T
    q_in: np.ndarray          # [B][T][H][d] f32
    k_in: np.ndarray          # [B][T][Hkv][d] f32
    v_in: np.ndarray          # [B][T][Hkv][d] f32
    w_q: np.ndarray | None
    w_k: np.ndarray | None
    cache_k: np.ndarray       # [B][Hkv][cap][d]
    cache_v: np.ndarray
    v_scale: np.ndarray | None
    k_scale: np.ndarray | None = None
    sinks: np.ndarray | None = None


def make_prefill_inputs(w: Workload, seq_lens=None) -> PrefillInputs:
    """Inputs of one chunk step: T = w.chunk new tokens per sequence (streams
    1-3 drawn as [B][T][...]), cached rows [lo, L - T) seeded as for a decode
    step (lo: the window start of the chunk's first token), the chunk's slots
    and every other row poisoned."""
    B, H, Hkv, d, cap, T = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.capacity, w.chunk
    if T < 1:
        raise ValueError(f"{w.name}: not a prefill workload (chunk={T})")
    lens = w.seq_lens() if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    if lens.shape != (B,) or lens.min() < T or lens.max() > cap:
        raise ValueError(f"{w.name}: seq_lens must be [{B}] within [{T}, {cap}]")
    s = tuple(w.seed)
    q_in = _normal([*s, 1], (B, T, H, d))
    k_in = _normal([*s, 2], (B, T, Hkv, d))
    v_in = _normal([*s, 3], (B, T, Hkv, d))
    w_q = w_k = None
    if w.qk_norm.enabled:
        z = _normal([*s, 4], (2, d))
        w_q = (w.qk_norm.w_mean + w.qk_norm.w_std * z[0]).astype(np.float32)
        w_k = (w.qk_norm.w_mean + w.qk_norm.w_std * z[1]).astype(np.float32)
    sinks = (2.0 + 3.0 * _normal([*s, 10], (H,))).astype(np.float32) if w.sink else None
    start = (lens - T).astype(np.int32)
    cache_k, cache_v, v_scale, k_scale = _fill_caches(w, lens, start.astype(np.int64))
    return PrefillInputs(w, lens, start, q_in, k_in, v_in, w_q, w_k, cache_k, cache_v, v_scale,
                         k_scale, sinks)


def prefill_flops(w: Workload, seq_lens=None) -> int:
    """Algorithmic flops of a chunk's attention: 4 d per (query head, visible
    key) for the score and the weighted sum."""
    lens = w.seq_lens() if seq_lens is None else np.asarray(seq_lens)
    T, total = w.chunk, 0
    for L in lens:
        p = np.arange(int(L) - T, int(L), dtype=np.int64)   # positions of the chunk
        lo = np.maximum(0, p + 1 - w.window) if w.window > 0 else np.zeros_like(p)
        total += int(np.sum(p + 1 - lo))
    return 4 * w.head_dim * w.n_heads * total


@dataclass
class PagedInputs:
    block_size: int
    max_blocks: int
    num_blocks: int
    block_table: np.ndarray     # [B][max_blocks] int32
    pool_k: np.ndarray          # [num_blocks][Hkv][block_size][d]
    pool_v: np.ndarray
    pool_scale: np.ndarray | None  # [num_blocks][Hkv][block_size] (int8 values)
    pool_k_scale: np.ndarray | None = None  # same, int8 keys

    @property
    def capacity(self) -> int:
        return self.max_blocks * self.block_size


def _poison_like(dtype) -> object:
    return {np.dtype(np.float32): np.float32(np.nan), np.dtype(np.uint16): BF16_NAN,
            np.dtype(np.int8): np.int8(0)}[np.dtype(dtype)]


def make_paged(inputs, block_size: int, spare_blocks: int = 3) -> PagedInputs:
    """Scatter the contiguous caches of ``inputs`` into block pools."""
    w = inputs.workload
    B, Hkv, d, cap = w.batch, w.n_kv_heads, w.head_dim, w.capacity
    bs = int(block_size)
    mb = -(-cap // bs)
    nblk = B * mb + spare_blocks
    rng = np.random.default_rng([*w.seed, 8])
    table = rng.permutation(nblk)[: B * mb].astype(np.int32).reshape(B, mb)

    def scatter(cache, trailing):
        # cache [B][Hkv][cap]+trailing -> pool [nblk][Hkv][bs]+trailing
        pad = mb * bs - cap
        if pad:
            fill = np.full((B, Hkv, pad) + trailing, _poison_like(cache.dtype), dtype=cache.dtype)
            cache = np.concatenate([cache, fill], axis=2)
        blocks = cache.reshape((B, Hkv, mb, bs) + trailing)
        blocks = np.moveaxis(blocks, 2, 1).reshape((B * mb, Hkv, bs) + trailing)
        pool = np.full((nblk, Hkv, bs) + trailing, _poison_like(cache.dtype), dtype=cache.dtype)
        pool[table.reshape(-1)] = blocks
        return pool

    pk = scatter(inputs.cache_k, (d,))
    pv = scatter(inputs.cache_v, (d,))
    ps = scatter(inputs.v_scale, ()) if inputs.v_scale is not None else None
    pks = scatter(inputs.k_scale, ()) if inputs.k_scale is not None else None
    return PagedInputs(bs, mb, nblk, table, pk, pv, ps, pks)
