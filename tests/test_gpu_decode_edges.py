"""GPU parity of the decode path on inputs with large score gaps, against the
CPU oracle, through the C ABI.

The seeded caches hold N(0,1) keys, so their scores sit within a few units
of each other.  Here the cached keys are edited before either side sees
them so that the softmax reference must move a long way:

* ramp up: key rows scaled by 1 + c*j/n along the cache, so the running max
  keeps growing from chunk to chunk, wave to wave and split to split, and
  every earlier state is rescaled by a tiny factor;
* ramp down: the reverse, so the first rows dominate and every later weight
  underflows;
* dominant key: one cached row per (sequence, kv head) set to a large
  multiple of the direction of its group's rotated queries, so that row
  outweighs all others by far (its output tends to that row's value);
* dominant new row (the single-launch step): the new token's key points
  along its group's queries, so the row the step merges after its last
  chunk dominates.

Score gaps reach well over 100 log2 units (each case states and checks its
own).  They run through every path of the partial kernel: one wave per work
item with more than one 512-row chunk per wave, cooperative interleaved
work-groups with more than one chunk per wave, paged caches (quarters and
lone waves), and the single-launch step; the combine sees up to 8 splits.
Softcap ("Universal AI Inference - Hugging Face decoder completeness", P1.4)
and the attention sink ("llamay - Models and formats", Architectures:
gpt-oss) are exercised on the same inputs.  Every output element, every
produced cache row and the split partials are compared at the class
tolerance (bf16 2e-3 absolute; int8 caches 1e-2 of the output's max-abs).

The last test writes quantiser near-tie vectors through the producer and
checks the int8 value codes and scales bit for bit against the stored
expected values (tests/golden/vq8_near_ties.json).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import parity as P
from gqa_decode_attention_kv_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)
COOP_BELOW = 2048   # the partial kernel runs items cooperatively below this count


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_decode_attention_kv_amd import binding
    binding.load()


def case(name, d, G, Hkv, kdt, vdt, lens, S, window=0, softcap=0.0, norm=None, sink=False,
         seed=0):
    lens = tuple(int(x) for x in lens)
    cap = max(lens) + 3
    qn = W.QKNorm(False) if norm is None else W.QKNorm(True, 1e-6, norm, 1.0 - norm, 0.1)
    w = W.Workload(name, len(lens), Hkv * G, Hkv, d, ("fixed", lens[0]), cap, kdt, vdt,
                   W.Rope(W.NEOX, W.PLAIN, 1e4), qn, window, softcap, S, (3000 + seed,), sink)
    return w, np.array(lens, np.int32)


def n_items(w, lens):
    """(split, kv head) work items the partial kernel launches."""
    n = 0
    for L in lens:
        lo, hi = w.visible(int(L))
        n += (hi - 1) // w.split_size - lo // w.split_size + 1
    return n * w.n_kv_heads


# -- input edits -------------------------------------------------------------

def _key_rows_as_f32(inputs, b, lo, hi):
    """Cached key rows [lo, hi) of sequence b, all kv heads, as float32
    (bf16 rows widened, f32 rows as stored; q8 rows as code * scale)."""
    w = inputs.workload
    rows = inputs.cache_k[b, :, lo:hi]
    if w.k_dtype == W.BF16:
        return (rows.astype(np.uint32) << 16).view(np.float32)
    if w.k_dtype == W.F32:
        return rows.copy()
    return rows.astype(np.float32) * inputs.k_scale[b, :, lo:hi, None]


def _store_key_rows(inputs, b, lo, hi, f):
    """Store float32 key rows back in the cache format (bf16 by keeping the
    top 16 bits, as the generator does)."""
    w = inputs.workload
    if w.k_dtype == W.BF16:
        inputs.cache_k[b, :, lo:hi] = (np.ascontiguousarray(f, np.float32).view(np.uint32)
                                       >> 16).astype(np.uint16)
    elif w.k_dtype == W.F32:
        inputs.cache_k[b, :, lo:hi] = f
    else:
        raise AssertionError("int8 keys are edited through their scales")


def scale_keys(factor):
    """prep: multiply cached key row lo + j (j = 0 .. n - 1) of every
    sequence by factor(j, n); int8 keys (q8) through their per-token scale."""
    def prep(inputs):
        w = inputs.workload
        for b in range(w.batch):
            L = int(inputs.seq_lens[b])
            lo, _ = w.visible(L)
            n = L - 1 - lo
            if n <= 0:
                continue
            fac = factor(np.arange(n, dtype=np.float32), n).astype(np.float32)
            if w.k_dtype == W.I8:
                inputs.k_scale[b, :, lo:L - 1] *= fac[None, :]
            else:
                f = _key_rows_as_f32(inputs, b, lo, L - 1) * fac[None, :, None]
                _store_key_rows(inputs, b, lo, L - 1, f)
    return prep


def ramp_up(c):
    return scale_keys(lambda j, n: 1.0 + c * j / max(1, n - 1))


def ramp_down(c):
    return scale_keys(lambda j, n: 1.0 + c * (n - 1 - j) / max(1, n - 1))


def rotated_queries(inputs):
    """q' [B][H][d] (double) from the oracle's norm and rotation pieces."""
    o = oracle.load()
    w = inputs.workload
    r = w.rope
    g = o.rope_freqs(w.head_dim, r.scaling, r.theta, r.factor, r.low, r.high, r.orig, r.truncate)
    q = np.zeros(inputs.q_in.shape, np.float64)
    for b in range(w.batch):
        for h in range(w.n_heads):
            x = inputs.q_in[b, h].astype(np.float64)
            if w.qk_norm.enabled:
                x = o.rms_norm(x, inputs.w_q, w.qk_norm.offset, w.qk_norm.eps)
            q[b, h] = o.rope_apply(x, r.pairing, g, int(inputs.positions[b]))
    return q


def dominant_key(strength, where=0.4, then=None):
    """prep: in every (sequence, kv head) the cached row at fraction `where`
    of the visible rows becomes strength * sqrt(d) * u, u the unit direction
    of the sum of the group's rotated queries, so its score is about
    strength * |q'| / sqrt(G) for each head of the group."""
    def prep(inputs):
        if then is not None:
            then(inputs)
        w = inputs.workload
        G, d = w.group, w.head_dim
        q = rotated_queries(inputs)
        for b in range(w.batch):
            L = int(inputs.seq_lens[b])
            lo, _ = w.visible(L)
            n = L - 1 - lo
            if n <= 0:
                continue
            j = lo + int(where * n)
            f = _key_rows_as_f32(inputs, b, j, j + 1)
            for u in range(w.n_kv_heads):
                s = q[b, u * G:(u + 1) * G].sum(axis=0)
                f[u, 0] = (strength * math.sqrt(d) * s / np.linalg.norm(s)).astype(np.float32)
            _store_key_rows(inputs, b, j, j + 1, f)
    return prep


def dominant_new_row(strength, then=None):
    """prep: the new token's key k_in points along the sum of its group's
    (unrotated, unnormed) queries.  The rotation at one position is the same
    orthogonal map for q and k, so the new row's score is about
    strength * |q| / sqrt(G) (requires QK-norm off)."""
    def prep(inputs):
        if then is not None:
            then(inputs)
        w = inputs.workload
        assert not w.qk_norm.enabled
        G, d = w.group, w.head_dim
        for b in range(w.batch):
            for u in range(w.n_kv_heads):
                s = inputs.q_in[b, u * G:(u + 1) * G].astype(np.float64).sum(axis=0)
                inputs.k_in[b, u] = (strength * math.sqrt(d) * s / np.linalg.norm(s)).astype(np.float32)
    return prep


def wild_value_scales(lo_exp, hi_exp, seed):
    """prep (int8 values): multiply the per-token value scale of every cached
    row by 10^u, u uniform in [lo_exp, hi_exp), so one chunk holds scales
    over several orders of magnitude (the matrix value pass writes each
    weight in digits of one scale per chunk)."""
    def prep(inputs):
        w = inputs.workload
        assert w.v_dtype == W.I8
        rng = np.random.default_rng(seed)
        for b in range(w.batch):
            L = int(inputs.seq_lens[b])
            lo, _ = w.visible(L)
            n = L - 1 - lo
            if n > 0:
                f = 10.0 ** rng.uniform(lo_exp, hi_exp, size=(w.n_kv_heads, n))
                inputs.v_scale[b, :, lo:L - 1] *= f.astype(np.float32)
    return prep


def spiky_queries(factor, comp=5):
    """prep: component `comp` of every query (before norm and rotation) is
    multiplied by `factor`, so the largest element of each rotated query is
    hundreds of times the others (the matrix key pass writes q in digits of
    one scale per head)."""
    def prep(inputs):
        inputs.q_in[:, :, comp] *= np.float32(factor)
    return prep


def chain(*preps):
    def prep(inputs):
        for p in preps:
            p(inputs)
    return prep


# -- score gap measurement --------------------------------------------------

def score_gap_log2(inputs, pairs):
    """Largest (max - min) visible score, in log2 units, over some
    (sequence, head) pairs, from the oracle's scores (softcap included)."""
    o = oracle.load()
    w = inputs.workload
    ref = P.OracleStep(inputs)
    gap = 0.0
    for b, h in pairs:
        L = int(inputs.seq_lens[b])
        s = o.scores(q=ref.q[b, h], cache_k=ref.ck, k_dtype=w.k_dtype, n_heads=w.n_heads, b=b,
                     h=h, L=L, window=w.window, softcap=w.softcap, k_scale=ref.ks)
        lo, _ = w.visible(L)
        s = s[lo:L]
        gap = max(gap, float(s.max() - s.min()) * LOG2E)
    return gap


def run_edge(w, lens, prep, mode, min_gap, block_size=None, fused=False, max_partials=None):
    items = n_items(w, lens)
    if mode == "lone":
        assert items >= COOP_BELOW, items
    elif mode == "coop":
        assert items < COOP_BELOW, items
    if fused and mode != "three":
        assert items <= 256, items  # one kernel
    inputs = W.make_inputs(w, seq_lens=lens)
    prep(inputs)
    pairs = [(b, h) for b in range(w.batch) for h in (0, w.n_heads - 1)]
    gap = score_gap_log2(inputs, pairs[:8])
    P.say(f"edge {w.name}: {items} work items ({mode}), score gap {gap:.1f} log2 units")
    assert gap >= min_gap, gap
    return P.run_and_compare(w, lens, max_partials_per_seq=max_partials, seed=7,
                             block_size=block_size, fused=fused, prep=prep)


# (workload, lens), prep, path, minimum score gap (log2 units), block size, partials per seq
EDGES = [
    # one wave per item (>= 2048 items), 600-row splits: two chunks per wave
    (case("lone-ramp-up-d64-g4", 64, 4, 32, W.BF16, W.BF16, [2400] * 16, 600, seed=1),
     ramp_up(30.0), "lone", 100.0, None, 3),
    # ragged lengths: items of unequal size, so the work-groups take the
    # serpentine placement (3.8 rounds of 256, the last one partial)
    (case("lone-ramp-down-d128-g4-ragged", 128, 4, 8, W.BF16, W.BF16,
          np.random.default_rng(2).integers(300, 901, 32), 40, seed=2),
     ramp_down(30.0), "lone", 100.0, None, 3),
    (case("paged-lone-ramp-down-d128-g4-ragged", 128, 4, 8, W.BF16, W.BF16,
          np.random.default_rng(2).integers(300, 901, 32), 40, seed=8),
     ramp_down(30.0), "lone", 100.0, 16, 3),
    # cooperative interleaved work-groups, 1024 rows (two chunks) per wave
    (case("coop-ramp-up-d128-g4", 128, 4, 2, W.BF16, W.BF16, [5000, 4500], 4096, seed=3),
     ramp_up(30.0), "coop", 100.0, None, None),
    # combine over 5 and 4 splits; the first split dominates
    (case("coop-ramp-down-d256-g2-5-splits", 256, 2, 2, W.BF16, W.BF16, [5000, 3100], 1024,
          seed=4), ramp_down(30.0), "coop", 100.0, None, None),
    # one dominant key inside the fourth of 8 splits
    (case("coop-dominant-key-d128-g4-8-splits", 128, 4, 2, W.BF16, W.BF16, [2000, 1500, 700],
          256, seed=5), dominant_key(20.0), "coop", 100.0, None, None),
    # softcap (scores pinned to +-50) with a sink and a window
    (case("coop-ramp-up-softcap-sink-window", 128, 4, 2, W.BF16, W.BF16, [3000, 1200], 512,
          window=2500, softcap=50.0, sink=True, seed=6),
     ramp_up(60.0), "coop", 100.0, None, None),
    (case("coop-dominant-key-softcap-d256", 256, 2, 2, W.BF16, W.BF16, [2600, 900], 512,
          softcap=50.0, seed=7), dominant_key(25.0, then=ramp_down(10.0)), "coop", 70.0, None,
     None),
    # int8 values: dominant key with a window and a sink
    (case("coop-dominant-key-vq8-window-sink", 128, 4, 2, W.BF16, W.I8, [3000, 800], 512,
          window=2000, sink=True, seed=8), dominant_key(20.0), "coop", 100.0, None, None),
    # int8 keys: ramp through the per-token key scales
    (case("coop-ramp-up-q8", 128, 4, 2, W.I8, W.I8, [4500, 2000], 1024, seed=9),
     ramp_up(30.0), "coop", 100.0, None, None),
    # QK-norm on (gain 1 + w): the dominant key follows the normed queries
    (case("coop-dominant-key-qknorm", 128, 4, 2, W.BF16, W.BF16, [1800, 1000], 256, norm=1,
          seed=10), dominant_key(20.0), "coop", 100.0, None, None),
    # paged caches: cooperative quarters (1024 rows a wave) and lone waves
    (case("paged-coop-ramp-up", 128, 4, 2, W.BF16, W.BF16, [5000, 2100], 4096, seed=11),
     ramp_up(30.0), "coop", 100.0, 16, None),
    (case("paged-lone-dominant-key-d64", 64, 4, 32, W.BF16, W.BF16, [2400] * 16, 600, seed=12),
     dominant_key(20.0), "lone", 100.0, 32, 3),
    (case("paged-coop-ramp-down-vq8-sink-window", 128, 4, 2, W.BF16, W.I8, [3000, 700], 512,
          window=2000, sink=True, seed=13), ramp_down(30.0), "coop", 100.0, 64, None),
    # int8 values on the matrix cores: value scales over six orders of
    # magnitude inside each chunk, on ramped keys (q8 G 4, vq8 G 2 d64 lone)
    (case("coop-ramp-up-wild-value-scales-q8", 128, 4, 2, W.I8, W.I8, [4500, 2000], 1024,
          seed=14), chain(ramp_up(30.0), wild_value_scales(-6.0, 0.0, 14)), "coop", 100.0, None,
     None),
    (case("lone-ramp-down-wild-value-scales-vq8-d64-g2", 64, 2, 32, W.BF16, W.I8, [2400] * 16,
          600, seed=15), chain(ramp_down(30.0), wild_value_scales(-6.0, 0.0, 15)), "lone", 100.0,
     None, 3),
    # queries with one element hundreds of times the others: q8 keys (q in
    # int8 digits), bf16 keys with G = 1 (key pass only on the matrix
    # cores), and a paged vq8 G = 2 d64 cache
    (case("coop-spiky-queries-q8", 128, 4, 2, W.I8, W.I8, [3000, 1500], 512, seed=16),
     spiky_queries(1000.0), "coop", 100.0, None, None),
    (case("coop-spiky-queries-vq8-g1", 128, 1, 4, W.BF16, W.I8, [3000, 1500], 512, seed=17),
     spiky_queries(1000.0), "coop", 100.0, None, None),
    (case("paged-coop-spiky-queries-vq8-g2-d64", 64, 2, 2, W.BF16, W.I8, [3000, 900], 1024,
          seed=18), spiky_queries(300.0), "coop", 100.0, 16, None),
    # groups of eight heads (the key pass, and for bf16 and int8 values the
    # value pass, on the matrix cores): bf16 cooperative and lone, f32 with
    # a sink, q8 with wild value scales, and a paged bf16 cache
    (case("coop-ramp-up-bf16-g8-d128", 128, 8, 1, W.BF16, W.BF16, [4500, 2000], 1024, seed=26),
     ramp_up(30.0), "coop", 100.0, None, None),
    (case("lone-dominant-key-bf16-g8-d64", 64, 8, 32, W.BF16, W.BF16, [2400] * 16, 600, seed=27),
     dominant_key(20.0), "lone", 100.0, None, 3),
    (case("coop-ramp-down-f32-g8-sink", 64, 8, 2, W.F32, W.F32, [3000, 1200], 512, sink=True,
          seed=28), ramp_down(30.0), "coop", 100.0, None, None),
    (case("coop-ramp-up-wild-value-scales-q8-g8", 128, 8, 1, W.I8, W.I8, [4500, 2000], 1024,
          seed=29), chain(ramp_up(30.0), wild_value_scales(-6.0, 0.0, 29)), "coop", 100.0, None,
     None),
    (case("paged-coop-ramp-up-bf16-g8", 128, 8, 2, W.BF16, W.BF16, [3000, 1500], 512, seed=30),
     ramp_up(30.0), "coop", 100.0, 16, None),
]


@pytest.mark.parametrize("spec", EDGES, ids=[e[0][0].name for e in EDGES])
def test_decode_large_score_gaps(spec):
    (w, lens), prep, mode, min_gap, bs, mp = spec
    run_edge(w, lens, prep, mode, min_gap, block_size=bs, max_partials=mp)


# The single-launch step (one kernel up to 256 work items): the split that
# holds the new token merges its row after its last chunk.
FUSED = [
    # the new row is negligible next to the ramped cache
    (case("fused-ramp-up", 128, 4, 2, W.BF16, W.BF16, [3000, 1700], 512, seed=21),
     ramp_up(30.0), 100.0, None),
    # the new row dominates a ramped-down cache
    (case("fused-new-row-dominant", 128, 4, 2, W.BF16, W.BF16, [3000, 900], 256, seed=22),
     dominant_new_row(20.0, then=ramp_down(10.0)), 60.0, None),
    (case("fused-new-row-dominant-softcap-sink-d256", 256, 2, 2, W.BF16, W.BF16, [2000, 600], 256,
          softcap=50.0, sink=True, seed=23), dominant_new_row(25.0), 60.0, None),
    (case("fused-dominant-key-vq8", 128, 4, 2, W.BF16, W.I8, [2500, 1300], 512, seed=24),
     dominant_key(20.0), 100.0, None),
    (case("fused-paged-ramp-down", 128, 4, 2, W.BF16, W.BF16, [3000, 1100], 1024, seed=25),
     ramp_down(30.0), 100.0, 16),
    # G = 8 over bf16 values: the new row's value merged into the matrix
    # pass's accumulator
    (case("fused-new-row-dominant-bf16-g8", 128, 8, 1, W.BF16, W.BF16, [2500, 900], 512, seed=31),
     dominant_new_row(20.0, then=ramp_down(10.0)), 60.0, None),
]


@pytest.mark.parametrize("spec", FUSED, ids=[e[0][0].name for e in FUSED])
def test_fused_large_score_gaps(spec):
    (w, lens), prep, min_gap, bs = spec
    run_edge(w, lens, prep, "coop", min_gap, block_size=bs, fused=True)


def test_vq8_producer_near_ties():
    """The producer's vq8 quantiser on values next to half-way points at
    non-power-of-two scales: codes and scales bit for bit equal to the
    stored expected values (exact rational arithmetic), and to the oracle."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "vq8_near_ties.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    d = 64
    w, lens = case("vq8-near-ties", d, 2, 1, W.BF16, W.I8, [5] * len(cases), 512, seed=30)

    def prep(inputs):
        inputs.v_in[:] = 0.0
        for b, c in enumerate(cases):
            inputs.v_in[b, 0, :len(c["v"])] = np.array(c["v"], np.float32)

    P.run_and_compare(w, lens, prep=prep)
    inputs = W.make_inputs(w, seq_lens=lens)
    prep(inputs)
    st = P.run_gpu(inputs)
    rows = st.cache_rows()
    for b, c in enumerate(cases):
        want = np.zeros(d, np.int8)
        want[:len(c["codes"])] = c["codes"]
        assert rows["v"][b, 0].tolist() == want.tolist(), b
        assert rows["scale"][b, 0] == np.float32(c["scale"]), b
