"""GPU parity of the chunk (prefill) path against the CPU oracle, through the
C ABI: uaii_kv_produce_chunk writes the chunk's T tokens, uaii_prefill_attn
computes their causal attention on the matrix cores.

* Small cases compare every output element, every produced cache row (and
  that no other row changed) and the rotated queries; they cover head dims
  64/128/256, GQA ratios 1-8, empty and non-empty caches, ragged batches,
  windows (1, inside the chunk, wider than the context), softcap, sinks,
  one-token chunks, several key tiles, the paged layout, and both kernel
  shapes (16 and 32 query rows per wave), over bf16, vq8, q8 and f32
  caches.
* The prefill workloads run at full size with sampled (sequence, token,
  head) outputs and every produced row.
* The chunk's attention agrees with the decode path run token by token.
Tolerances on the output are the decode path's: 1e-5 absolute for f32 K/V,
2e-3 for bf16 K/V (f32 accumulation), 1e-2 of the output's max-abs for int8
values (vq8, q8); produced int8 codes and scales are bit-exact.
"""
import numpy as np
import pytest

import oracle
import parity as P
from gqa_decode_attention_kv_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_decode_attention_kv_amd import binding
    binding.load()


def case(name, d, G, Hkv, T, lens, window=0, softcap=0.0, rope=None, norm=None, sink=False,
         seed=0, bs=None, kv=(W.BF16, W.BF16)):
    lens = tuple(int(x) for x in lens)
    qn = W.QKNorm(False) if norm is None else W.QKNorm(True, 1e-6, norm, 1.0 - norm, 0.1)
    w = W.Workload(name, len(lens), Hkv * G, Hkv, d, ("fixed", lens[0]), max(lens) + 3, kv[0],
                   kv[1], rope or W.Rope(W.NEOX, W.PLAIN, 1e4), qn, window, softcap, 512,
                   (4000 + seed,), sink, T)
    return w, np.array(lens, np.int32), bs


VQ8, Q8, F32 = (W.BF16, W.I8), (W.I8, W.I8), (W.F32, W.F32)


LLAMA3 = W.Rope(W.INTERLEAVED, W.LLAMA3, 5e5, 8.0)

SMALL = [
    case("d128-g4-empty-cache", 128, 4, 2, 100, [100, 100], seed=1),
    case("d128-g2-chunk-after-cache", 128, 2, 2, 70, [300, 71], rope=LLAMA3, seed=2),
    case("d64-g8-one-kv-head", 64, 8, 1, 33, [97], seed=3),
    case("d256-g2-window-softcap-norm", 256, 2, 2, 90, [250, 90], window=50, softcap=50.0, norm=1,
         seed=4),
    case("d128-g1-window1", 128, 1, 3, 20, [40], window=1, seed=5),
    case("d64-g4-sink", 64, 4, 2, 65, [130, 200], sink=True, seed=6),
    case("d128-g4-one-token", 128, 4, 2, 1, [500, 3], seed=7),
    case("d128-g8-several-tiles", 128, 8, 1, 257, [1000], norm=0, seed=8),
    case("d64-g1-window-wider", 64, 1, 4, 40, [70, 45], window=5000, seed=9),
    case("d128-g4-window-in-chunk", 128, 4, 2, 150, [400, 160], window=37, softcap=20.0, seed=10),
    case("d256-g8-sink-window", 256, 8, 1, 24, [64], window=30, sink=True, seed=11),
    case("d128-g4-b32-ragged", 128, 4, 2, 16,
         np.random.default_rng(12).integers(16, 201, 32), rope=LLAMA3, seed=12),
    case("d128-g4-paged-bs16", 128, 4, 2, 100, [333, 120], window=200, seed=13, bs=16),
    case("d64-g2-paged-bs64-sink", 64, 2, 2, 50, [50, 260], sink=True, seed=14, bs=64),
    # Grids of at least 512 work-groups run with 32 rows per wave: ragged
    # row tails, windows, sinks, softcap and paging on that path too.
    case("d128-g4-b32-two-blocks-ragged", 128, 4, 8, 72,
         np.random.default_rng(15).integers(72, 301, 32), window=100, sink=True, seed=15),
    case("d64-g8-b32-two-blocks-paged", 64, 8, 8, 40,
         np.random.default_rng(16).integers(40, 201, 32), softcap=30.0, seed=16, bs=16),
    # int8 caches: vq8 (bf16 keys, int8 values) and q8 (both int8), each
    # with one f32 scale per token per kv head
    case("vq8-d128-g4-chunk-norm", 128, 4, 2, 90, [300, 95], norm=0, seed=17, kv=VQ8),
    case("vq8-d64-g2-window-sink", 64, 2, 2, 60, [200, 61], window=50, sink=True, seed=18, kv=VQ8),
    case("vq8-d256-g2-softcap", 256, 2, 2, 40, [120], softcap=50.0, seed=19, kv=VQ8),
    case("q8-d128-g4-chunk", 128, 4, 2, 70, [260, 80], rope=LLAMA3, seed=20, kv=Q8),
    case("q8-d64-g8-window-paged", 64, 8, 1, 50, [180, 51], window=40, seed=21, kv=Q8, bs=32),
    case("q8-d256-g1-softcap", 256, 1, 2, 30, [90], softcap=20.0, seed=22, kv=Q8),
    case("vq8-d128-g4-b32-two-blocks", 128, 4, 8, 72,
         np.random.default_rng(23).integers(72, 241, 32), seed=23, kv=VQ8),
    # Two query blocks per wave stage 64 key rows per barrier and compute
    # them as two halves: int8 keys (each half's key scales) and a paged
    # int8-value cache on that path.
    case("q8-d128-g4-b32-two-blocks", 128, 4, 8, 72,
         np.random.default_rng(24).integers(72, 301, 32), window=150, seed=24, kv=Q8),
    case("vq8-d128-g2-b32-two-blocks-paged", 128, 2, 8, 140,
         np.random.default_rng(25).integers(140, 331, 32), sink=True, seed=25, kv=VQ8, bs=32),
    # f32 caches (f32 matrix products), head dims 64 and 128: the gpt-oss
    # shape (d64, G 8, sinks, a window), several tiles, paging, softcap, a
    # ragged batch on the two-blocks path.
    case("f32-d64-g8-sink-window", 64, 8, 1, 96, [300, 97], window=128, sink=True, seed=26, kv=F32),
    case("f32-d128-g4-several-tiles", 128, 4, 2, 130, [700, 131], rope=LLAMA3, seed=27, kv=F32),
    case("f32-d64-g2-paged-softcap", 64, 2, 2, 50, [250, 60], softcap=30.0, seed=28, kv=F32, bs=16),
    case("f32-d128-g1-window-in-chunk", 128, 1, 3, 70, [200], window=33, norm=1, seed=29, kv=F32),
    case("f32-d64-g8-b32-two-blocks", 64, 8, 8, 40,
         np.random.default_rng(30).integers(40, 201, 32), sink=True, seed=30, kv=F32),
]


def run_gpu(inputs, paged=None):
    from gqa_decode_attention_kv_amd.step import DevicePrefill
    st = DevicePrefill(inputs, paged=paged)
    st.out.fill_(float("nan"))
    st.step()
    torch.cuda.synchronize()
    return st


def oracle_side(inputs, copy_cache=True):
    o = oracle.load()
    w = inputs.workload
    ck = inputs.cache_k.copy() if copy_cache else inputs.cache_k
    cv = inputs.cache_v.copy() if copy_cache else inputs.cache_v
    vs, ks = inputs.v_scale, inputs.k_scale
    vs = (vs.copy() if copy_cache else vs) if vs is not None else None
    ks = (ks.copy() if copy_cache else ks) if ks is not None else None
    norm = None
    if w.qk_norm.enabled:
        norm = dict(enabled=True, eps=w.qk_norm.eps, offset=w.qk_norm.offset, w_q=inputs.w_q,
                    w_k=inputs.w_k)
    q = o.kv_produce_chunk(rope=w.rope.as_dict(), norm=norm, q_in=inputs.q_in, k_in=inputs.k_in,
                           v_in=inputs.v_in, start_positions=inputs.start, k_dtype=w.k_dtype,
                           v_dtype=w.v_dtype, cache_k=ck, cache_v=cv, v_scale=vs, k_scale=ks)
    return o, q, ck, cv, vs, ks


def chunk_rows(st, cache):
    """[B][Hkv][T](...) view of the chunk's slots (contiguous or through the table)."""
    w = st.w
    out = []
    for b in range(w.batch):
        pos = st.start[b] + np.arange(st.T)
        if st.paged:
            bs = st.paged.block_size
            blk = st.paged.block_table[b, pos // bs]
            out.append(np.stack([cache[blk, u, pos % bs] for u in range(w.n_kv_heads)]))
        else:
            out.append(cache[b][:, pos])
    return np.stack(out)


def host(t, dtype):
    return t.cpu().numpy().view(dtype)


def check_rows(st, ref_q, ck, cv, vs, ks):
    """The chunk's produced rows and rotated queries against the oracle's:
    V (codes and scales) bit-exact, K within 1 bf16 ulp (q8: codes within 1,
    scales within 1 ulp), q' within 1e-6 relative."""
    w = st.w
    rows = lambda a: np.stack([a[b][:, st.start[b] + np.arange(st.T)] for b in range(w.batch)])
    gpu = dict(k=chunk_rows(st, host(st.cache_k, W.STORAGE[w.k_dtype])),
               v=chunk_rows(st, host(st.cache_v, W.STORAGE[w.v_dtype])),
               scale=chunk_rows(st, host(st.v_scale, np.float32)) if st.v_scale is not None else None,
               k_scale=chunk_rows(st, host(st.k_scale, np.float32)) if st.k_scale is not None else None)
    ref = dict(k=rows(ck), v=rows(cv), scale=rows(vs) if vs is not None else None,
               k_scale=rows(ks) if ks is not None else None)
    P.check_slot(w, gpu, ref, st.q_out.cpu().numpy(), ref_q)


def run_small(w, lens, bs, prep=None):
    """One small chunk step on the GPU against the oracle: produced rows and
    queries, untouched rows elsewhere, and every output.  prep, if given,
    rewrites the seeded inputs first."""
    P.say(f"prefill case {w.name}: B={w.batch} H={w.n_heads}/{w.n_kv_heads} d={w.head_dim} "
          f"T={w.chunk} lens={lens.tolist()[:8]} W={w.window} cap={w.softcap} sink={w.sink} "
          f"paged={bs}")
    inputs = W.make_prefill_inputs(w, seq_lens=lens)
    if prep is not None:
        prep(inputs)
    paged = W.make_paged(inputs, bs) if bs else None
    if paged:
        before = [paged.pool_k, paged.pool_v, paged.pool_scale, paged.pool_k_scale]
    else:
        before = [inputs.cache_k, inputs.cache_v, inputs.v_scale, inputs.k_scale]
    before = [x.copy() if x is not None else None for x in before]
    st = run_gpu(inputs, paged)
    o, q, ck, cv, vs, ks = oracle_side(inputs)
    check_rows(st, q, ck, cv, vs, ks)
    # nothing but the chunk's slots changed
    for dev, old in zip((st.cache_k, st.cache_v, st.v_scale, st.k_scale), before):
        if dev is None:
            continue
        g = host(dev, old.dtype)
        mask = np.ones(g.shape[:3], bool)
        for b in range(w.batch):
            pos = st.start[b] + np.arange(st.T)
            if paged:
                blk = paged.block_table[b, pos // paged.block_size]
                mask[blk, :, pos % paged.block_size] = False
            else:
                mask[b, :, pos] = False
        assert np.array_equal(g[mask].view(np.uint8), old[mask].view(np.uint8)), \
            "cache rows outside the chunk changed"
    want = o.prefill(q=q, cache_k=ck, cache_v=cv, v_scale=vs, k_scale=ks, k_dtype=w.k_dtype,
                     v_dtype=w.v_dtype, seq_lens=lens, window=w.window, softcap=w.softcap,
                     sinks=inputs.sinks)
    out = st.out.cpu().numpy()
    tol, cls = P.out_tolerance(w, want)
    err = float(np.max(np.abs(out - want)))
    P.say(f"  max abs err {err:.3g} (tol {tol:.3g}, {cls})")
    assert np.all(np.isfinite(out)) and err <= tol, err


@pytest.mark.parametrize("spec", SMALL, ids=[c[0].name for c in SMALL])
def test_prefill_small(spec):
    run_small(*spec)


def scale_cached_keys(factor):
    """prep: multiply each cached bf16 key row [lo, L - T) by factor(j, n)
    (j = 0 .. n - 1 from the oldest row), re-stored by truncation like the
    generator's rows."""
    def prep(inputs):
        w = inputs.workload
        assert w.k_dtype == W.BF16
        for b in range(w.batch):
            first = int(inputs.start[b])
            lo, _ = w.visible(first + 1)
            n = first - lo
            if n <= 0:
                continue
            rows = inputs.cache_k[b, :, lo:first]
            f = (rows.astype(np.uint32) << 16).view(np.float32)
            f = f * factor(np.arange(n, dtype=np.float32), n)[None, :, None]
            inputs.cache_k[b, :, lo:first] = (f.view(np.uint32) >> 16).astype(np.uint16)
    return prep


def spike(j, n):
    out = np.ones(n, np.float32)
    out[n // 2] = 25.0
    return out


# Scores whose running max keeps growing (keys scaled up along the cache:
# about 11 log2 units more per 32-key tile), falling, or jumping once: the
# chunk kernel's softmax reference then moves mid-sequence, and the
# accumulator and sums are rescaled, on many tiles rather than only the
# first.
MOVING = [
    (case("ramp-up-d128-g4", 128, 4, 2, 64, [700, 400], seed=31), lambda j, n: 1.0 + 0.1 * j),
    (case("ramp-up-d128-g4-b32-two-blocks", 128, 4, 8, 72,
          np.random.default_rng(32).integers(300, 601, 32), seed=32), lambda j, n: 1.0 + 0.1 * j),
    (case("ramp-down-d64-g8", 64, 8, 1, 40, [500], seed=33), lambda j, n: 1.0 + 0.1 * (n - 1 - j)),
    (case("spike-d128-g2-window-sink", 128, 2, 2, 50, [400, 300], window=200, sink=True, seed=34),
     spike),
    (case("ramp-up-vq8-d128-g4-softcap", 128, 4, 2, 48, [600], softcap=50.0, seed=35, kv=VQ8),
     lambda j, n: 1.0 + 0.1 * j),
]


@pytest.mark.parametrize("spec", MOVING, ids=[c[0][0].name for c in MOVING])
def test_prefill_moving_reference(spec):
    (w, lens, bs), factor = spec
    run_small(w, lens, bs, prep=scale_cached_keys(factor))


@pytest.mark.parametrize("name", list(W.PREFILL))
def test_prefill_full_size(name):
    w = W.PREFILL[name]
    P.say(f"prefill full-size {name}: B={w.batch} H={w.n_heads}/{w.n_kv_heads} d={w.head_dim} "
          f"T={w.chunk} L={w.lens} W={w.window} cap={w.softcap}")
    inputs = W.make_prefill_inputs(w)
    st = run_gpu(inputs)
    o, q, ck, cv, vs, ks = oracle_side(inputs, copy_cache=False)
    check_rows(st, q, ck, cv, vs, ks)
    rng = np.random.default_rng(7)
    T = w.chunk
    tr = [(b, t, int(rng.integers(w.n_heads))) for b in range(w.batch) for t in (0, T - 1)]
    tr += [(int(rng.integers(w.batch)), int(rng.integers(T)), int(rng.integers(w.n_heads)))
           for _ in range(48)]
    want = o.prefill(q=q, cache_k=ck, cache_v=cv, v_scale=vs, k_scale=ks, k_dtype=w.k_dtype,
                     v_dtype=w.v_dtype, seq_lens=inputs.seq_lens, window=w.window,
                     softcap=w.softcap, sinks=inputs.sinks, triples=tr)
    out = st.out.cpu().numpy()
    got = np.stack([out[b, t, h] for b, t, h in tr])
    tol, cls = P.out_tolerance(w, want)
    err = float(np.max(np.abs(got - want)))
    P.say(f"  sampled {len(tr)} outputs: max abs err {err:.3g} (tol {tol:.3g}, {cls})")
    assert np.all(np.isfinite(out)) and err <= tol, err


def test_prefill_matches_decode_token_by_token():
    """Each chunk query's output equals the decode path's (partials and
    combine, f32 vector arithmetic) for the same query at the same length."""
    from gqa_decode_attention_kv_amd import binding as B
    w, lens, _ = SMALL[1]
    inputs = W.make_prefill_inputs(w, seq_lens=lens)
    st = run_gpu(inputs)
    T, S = st.T, 64
    max_splits = int(-(-int(lens.max()) // S))
    part_o = torch.empty((w.batch, w.n_heads, max_splits, w.head_dim), device="cuda")
    part_lse = torch.empty((w.batch, w.n_heads, max_splits), device="cuda")
    out = torch.empty((w.batch, w.n_heads, w.head_dim), device="cuda")
    worst = 0.0
    for t in range(T):
        q = st.q_out[:, t].contiguous()
        Lt = (lens - T + t + 1).astype(np.int32)
        B.decode_attn(st.shape, st.cache, q.data_ptr(), Lt, st.scale, w.window, w.softcap, S,
                      max_splits, part_o.data_ptr(), part_lse.data_ptr(), st.stream())
        B.decode_combine(st.shape, Lt, w.window, S, max_splits, part_o.data_ptr(),
                         part_lse.data_ptr(), out.data_ptr(), st.stream())
        torch.cuda.synchronize()
        worst = max(worst, float((out - st.out[:, t]).abs().max()))
    P.say(f"  prefill vs decode, {T} tokens: max abs difference {worst:.3g}")
    assert worst <= 2e-4, worst


def test_prefill_refusals_write_nothing():
    """A cache pair the chunk kernel does not take (bf16 keys with f32
    values) and a length shorter than the chunk are refused before any
    launch; nothing is written."""
    from gqa_decode_attention_kv_amd import binding as B
    w, lens, _ = SMALL[0]
    inputs = W.make_prefill_inputs(w, seq_lens=lens)
    st = run_gpu(inputs)
    before = st.out.clone()
    mixed = B.KVCache(B.BF16, B.F32, st.cache.capacity, st.cache.k, st.cache.v, None, None, 0,
                      0, 0, None)
    with pytest.raises(B.UaiiError, match="prefill over k_dtype=1, v_dtype=0"):
        B.prefill_attn(st.shape, mixed, st.q_out.data_ptr(), st.seq_lens, st.T, st.scale, 0,
                       0.0, None, st.out.data_ptr(), st.stream())
    with pytest.raises(B.UaiiError, match="seq_lens"):
        B.prefill_attn(st.shape, st.cache, st.q_out.data_ptr(), st.seq_lens - st.T, st.T, st.scale,
                       0, 0.0, None, st.out.data_ptr(), st.stream())
    torch.cuda.synchronize()
    assert torch.equal(before, st.out)


def scale_key_scales(factor):
    """prep for int8 keys (q8): multiply the per-token key scale of cached
    row lo + j by factor(j, n)."""
    def prep(inputs):
        w = inputs.workload
        assert w.k_dtype == W.I8
        for b in range(w.batch):
            first = int(inputs.start[b])
            lo, _ = w.visible(first + 1)
            n = first - lo
            if n > 0:
                inputs.k_scale[b, :, lo:first] *= factor(np.arange(n, dtype=np.float32), n)[None, :]
    return prep


def then(*preps):
    def prep(inputs):
        for p in preps:
            p(inputs)
    return prep


def huge_values(where, size=3e5):
    """prep: cached bf16 value rows lo + j for j in where(n) multiplied by
    `size` (beyond f16's range: the values must go through the product as
    stored)."""
    def prep(inputs):
        w = inputs.workload
        assert w.v_dtype == W.BF16
        for b in range(w.batch):
            first = int(inputs.start[b])
            lo, _ = w.visible(first + 1)
            n = first - lo
            if n <= 0:
                continue
            rows = lo + np.asarray(where(n), dtype=np.int64)
            f = (inputs.cache_v[b][:, rows].astype(np.uint32) << 16).view(np.float32) * np.float32(size)
            inputs.cache_v[b][:, rows] = (f.view(np.uint32) >> 16).astype(np.uint16)
    return prep


# Scores far beyond the moving-reference cases: keys scaled up along the
# cache so that the largest scores reach 430 to 670 log2 units (one lone
# spike key at 1070).  q enters the score product as a bf16 pair (about
# 2^-17 of q left out), an error in the score that grows with the score:
# about 1e-3 in the output near 600 log2 units (415 in natural units), and
# the 2e-3 bound is reached near 700 in a batch of 32 ragged items.  These
# cases hold the path to the bound up to that limit.
LARGE = [
    (case("scores-500-d128-g4", 128, 4, 2, 64, [700, 400], seed=41),
     scale_cached_keys(lambda j, n: 1.0 + 150.0 * j / n)),
    (case("scores-500-d64-g8-two-blocks", 64, 8, 8, 40,
          np.random.default_rng(42).integers(300, 601, 32), seed=42),
     scale_cached_keys(lambda j, n: 1.0 + 100.0 * j / n)),
    (case("scores-500-d256-g2-sink-window", 256, 2, 2, 50, [600, 300], window=400, sink=True,
          seed=43), scale_cached_keys(lambda j, n: 1.0 + 120.0 * j / n)),
    (case("scores-500-vq8-d128-g4", 128, 4, 2, 48, [640], seed=44, kv=VQ8),
     scale_cached_keys(lambda j, n: 1.0 + 150.0 * j / n)),
    (case("scores-500-q8-d128-g4", 128, 4, 2, 48, [640, 200], seed=45, kv=Q8),
     scale_key_scales(lambda j, n: 1.0 + 150.0 * j / n)),
    (case("scores-500-spike-paged", 128, 4, 2, 64, [500, 300], seed=46, bs=16),
     scale_cached_keys(lambda j, n: np.where(j == n // 3, 400.0, 1.0).astype(np.float32))),
    # Values beyond f16's range in low-weight rows (the first cached rows,
    # under ramped keys): they must neither overflow nor leak into the
    # output.
    (case("huge-values-low-weight-d128", 128, 4, 2, 64, [700, 400], seed=47),
     then(scale_cached_keys(lambda j, n: 1.0 + 20.0 * j / n),
          huge_values(lambda n: np.arange(0, min(n, 40), 3)))),
    (case("huge-values-low-weight-d64-two-blocks", 64, 4, 8, 72,
          np.random.default_rng(48).integers(300, 501, 32), seed=48),
     then(scale_cached_keys(lambda j, n: 1.0 + 20.0 * j / n),
          huge_values(lambda n: [0, 5, 33]))),
]


@pytest.mark.parametrize("spec", LARGE, ids=[c[0][0].name for c in LARGE])
def test_prefill_large_scores(spec):
    (w, lens, bs), prep = spec
    run_small(w, lens, bs, prep=prep)


def test_prefill_huge_values_with_weight():
    """Values of 1e5 and more in the rows that dominate the softmax: the
    output is of their size, and is checked relative to the largest visible
    value (f32 accumulation of bf16-split weights)."""
    w, lens, bs = case("huge-values-dominant", 128, 4, 2, 64, [600, 300], seed=49)
    prep = then(scale_cached_keys(lambda j, n: 1.0 + 3.0 * j / n),
                huge_values(lambda n: np.arange(n - 48, n)))
    inputs = W.make_prefill_inputs(w, seq_lens=lens)
    prep(inputs)
    st = run_gpu(inputs)
    o, q, ck, cv, vs, ks = oracle_side(inputs)
    want = o.prefill(q=q, cache_k=ck, cache_v=cv, v_scale=vs, k_scale=ks, k_dtype=w.k_dtype,
                     v_dtype=w.v_dtype, seq_lens=lens, window=w.window, softcap=w.softcap,
                     sinks=inputs.sinks)
    out = st.out.cpu().numpy()
    vmax = float(np.max(np.abs((cv.astype(np.uint32) << 16).view(np.float32)[np.isfinite(
        (cv.astype(np.uint32) << 16).view(np.float32))])))
    err = float(np.max(np.abs(out - want)))
    P.say(f"  max |out| {np.max(np.abs(want)):.3g}, max |v| {vmax:.3g}, max abs err {err:.3g} "
          f"({err / vmax:.3g} of max |v|)")
    assert vmax > 65520.0 and np.max(np.abs(want)) > 1e4
    assert np.all(np.isfinite(out)) and err <= 1e-5 * vmax, err
