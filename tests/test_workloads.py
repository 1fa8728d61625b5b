"""Seeded input generation: deterministic, thread-count independent, poisoned
outside the visible rows."""
import numpy as np

from gqa_decode_attention_kv_amd import workloads as W


def test_deterministic_and_poisoned():
    w = W.shrink(W.WORKLOADS["gemma2-local"], batch=2, lens=("fixed", 40), capacity=48,
                 window=16)
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for name in ("q_in", "k_in", "v_in", "w_q", "w_k", "cache_k", "cache_v"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    lo, hi = w.visible(40)
    assert (lo, hi) == (24, 40)
    ck = a.cache_k
    assert np.all(ck[:, :, :lo] == W.BF16_NAN) and np.all(ck[:, :, hi - 1:] == W.BF16_NAN)
    assert not np.any(ck[:, :, lo:hi - 1] == W.BF16_NAN)
    assert np.array_equal(a.positions, a.seq_lens - 1)


def test_ragged_lengths_and_vq8():
    w = W.shrink(W.WORKLOADS["llama3.1-8b-ragged"], batch=5, capacity=8192)
    lens = w.seq_lens()
    assert lens.min() >= 512 and lens.max() <= 8192
    assert np.array_equal(lens, w.seq_lens())
    q = W.shrink(W.WORKLOADS["qwen3-vq8"], batch=2, lens=("fixed", 33), capacity=40)
    x = W.make_inputs(q)
    assert x.cache_v.dtype == np.int8 and np.all(np.abs(x.cache_v.astype(int)) <= 127)
    assert np.all(np.isnan(x.v_scale[:, :, 32:])) and np.all(x.v_scale[:, :, :32] > 0)


def test_kv_bytes():
    h = W.WORKLOADS[W.HEADLINE]
    assert h.kv_bytes() == 32 * 8 * 8192 * 128 * 4 == 1073741824
    assert W.WORKLOADS["qwen3-vq8"].kv_bytes() == 16 * 8 * 16384 * 388
    assert W.WORKLOADS["gemma2-local"].kv_bytes() == 8 * 8 * 4096 * 1024
    assert W.WORKLOADS["tiny"].kv_bytes() == 2 * 129 * 512


def test_gather_probe_orders():
    """The read probe's piece orders are permutations; the kv order gives
    each work-group consecutive pieces of the buffer's two halves in turn."""
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    n, per = 64, 8
    for kind in bench.GATHER_ORDERS:
        o = bench.gather_order(n, per, kind).tolist()
        assert sorted(o) == list(range(n)), kind
    assert bench.gather_order(n, per, "sequential").tolist() == list(range(n))
    kv = bench.gather_order(n, per, "kv").tolist()
    assert kv[:per] == [0, 32, 1, 33, 2, 34, 3, 35]
    assert kv[per:2 * per] == [4, 36, 5, 37, 6, 38, 7, 39]
    assert bench.gather_order(n, per, "random").tolist() == bench.gather_order(n, per, "random").tolist()
