"""The C-ABI library on the host: it loads, exports every function the header
declares, and refuses malformed or unsupported arguments before touching the
device, with a message that names the fact, its value and the supported
range.  These tests pass fake (never dereferenced) device addresses, so they
are skipped where a GPU is visible; the same refusals are exercised with real
buffers by the GPU tests."""
import math
import os
import re

import numpy as np
import pytest

from gqa_decode_attention_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uaii_decode.h")


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


host_only = pytest.mark.skipif(not _no_gpu(), reason="fake device addresses; host-only test")

FAKE = 0x7F0000000000  # 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uaii_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.load()
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert B.last_error() == ""


def test_struct_layouts_match_header():
    import ctypes as C
    assert C.sizeof(B.Shape) == 16
    assert C.sizeof(B.Rope) == 56 and B.Rope.theta.offset == 8
    assert B.Rope.truncate.offset == 44 and B.Rope.attention_factor.offset == 48
    assert C.sizeof(B.QKNorm) == 32 and B.QKNorm.q_weight.offset == 16
    assert C.sizeof(B.KVCache) == 72 and B.KVCache.k.offset == 16
    assert B.KVCache.block_table.offset == 40 and B.KVCache.num_blocks.offset == 56
    assert B.KVCache.k_scale.offset == 64


def shape(b=2, h=8, hkv=2, d=128):
    return B.Shape(b, h, hkv, d)


def cache(kd=B.BF16, vd=B.BF16, cap=64, k=FAKE, v=FAKE, s=None, ks=None):
    return B.KVCache(kd, vd, cap, k, v, s, None, 0, 0, 0, ks)


def attn(sh=None, ca=None, q=FAKE, lens=(10, 20), scale=None, window=0, softcap=0.0, split=16,
         max_splits=4, po=FAKE, pl=FAKE):
    sh = sh or shape()
    ca = ca or cache()
    scale = 1.0 / math.sqrt(sh.head_dim) if scale is None else scale
    B.decode_attn(sh, ca, q, lens, scale, window, softcap, split, max_splits, po, pl, 0)


def produce(sh=None, rope=None, norm=None, ca=None, pos=(3, 4), q_in=FAKE, q_out=FAKE):
    sh = sh or shape()
    rope = rope or B.Rope(B.ROPE_NEOX, B.ROPE_PLAIN, 1e4, 1.0, 1.0, 4.0, 8192)
    B.kv_produce(sh, rope, norm, q_in, FAKE, FAKE, pos, ca or cache(), q_out, 0)


def combine(sh=None, lens=(10, 20), window=0, split=16, max_splits=4, out=FAKE):
    B.decode_combine(sh or shape(), lens, window, split, max_splits, FAKE, FAKE, out, 0)


def combine_sink(sh=None, lens=(10, 20), window=0, split=16, max_splits=4, sinks=FAKE, out=FAKE):
    B.decode_combine_sink(sh or shape(), lens, window, split, max_splits, FAKE, FAKE, sinks, out, 0)


def step(sh=None, rope=None, norm=None, ca=None, lens=(10, 20), scale=None, window=0, softcap=0.0,
         split=16, max_splits=4, sinks=None, q_out=FAKE, counters=FAKE, out=FAKE):
    sh = sh or shape()
    rope = rope or B.Rope(B.ROPE_NEOX, B.ROPE_PLAIN, 1e4, 1.0, 1.0, 4.0, 8192)
    scale = 1.0 / math.sqrt(sh.head_dim) if scale is None else scale
    B.decode_step(sh, rope, norm, FAKE, FAKE, FAKE, lens, ca or cache(), scale, window, softcap,
                  split, max_splits, sinks, q_out, FAKE, FAKE, counters, out, 0)


def refused(fn, status, *needles):
    with pytest.raises(B.UaiiError) as ei:
        fn()
    assert ei.value.status == status, ei.value
    for n in needles:
        assert n in ei.value.message, (n, ei.value.message)
    return ei.value.message


INV, NI = B.ERR_INVALID_ARGUMENT, B.ERR_NOT_IMPLEMENTED


@host_only
@pytest.mark.parametrize("case", [
    ("head_dim 96", lambda: attn(sh=shape(d=96)), NI, ["head_dim=96 is not supported", "{64, 128, 256}"]),
    ("head_dim 32", lambda: attn(sh=shape(d=32)), NI, ["head_dim=32"]),
    ("batch 40", lambda: attn(sh=shape(b=40), lens=[1] * 40), NI, ["batch=40 is not supported", "1..32"]),
    ("batch 0", lambda: attn(sh=shape(b=0)), INV, ["batch=0"]),
    ("gqa not integral", lambda: attn(sh=shape(h=6, hkv=4)), INV, ["n_heads=6", "n_kv_heads=4"]),
    ("gqa 3", lambda: attn(sh=shape(h=6, hkv=2)), NI, ["n_heads/n_kv_heads=3", "{1, 2, 4, 8}"]),
    ("scale", lambda: attn(scale=0.1), NI, ["scale=0.1", "1/sqrt(head_dim)=0.0883883"]),
    ("scale nan", lambda: attn(scale=float("nan")), INV, ["scale="]),
    ("window", lambda: attn(window=-1), INV, ["window=-1"]),
    ("softcap neg", lambda: attn(softcap=-1.0), INV, ["softcap=-1"]),
    ("softcap inf", lambda: attn(softcap=float("inf")), INV, ["softcap=inf"]),
    ("split 0", lambda: attn(split=0), INV, ["split_size=0"]),
    ("max_splits", lambda: attn(lens=(10, 40), split=16, max_splits=2), INV,
     ["max_splits=2", "need 3"]),
    ("len 0", lambda: attn(lens=(0, 5)), INV, ["seq_lens[0]=0", "[1, 64]"]),
    ("len > cap", lambda: attn(lens=(65, 5)), INV, ["seq_lens[0]=65"]),
    ("int8 keys, bf16 values", lambda: attn(ca=cache(kd=B.I8, vd=B.BF16)), NI,
     ["k_dtype=int8 with v_dtype=1", "q8"]),
    ("q8 no key scale", lambda: attn(ca=cache(kd=B.I8, vd=B.I8, s=FAKE)), INV, ["k_scale is NULL"]),
    ("q8 key scale misaligned", lambda: attn(ca=cache(kd=B.I8, vd=B.I8, s=FAKE, ks=FAKE + 2)), INV,
     ["cache.k_scale", "4-byte aligned"]),
    ("bad k dtype", lambda: attn(ca=cache(kd=7)), INV, ["k_dtype=7"]),
    ("bad v dtype", lambda: attn(ca=cache(vd=5)), INV, ["v_dtype=5"]),
    ("vq8 no scale", lambda: attn(ca=cache(vd=B.I8)), INV, ["v_scale is NULL"]),
    ("cap 0", lambda: attn(ca=cache(cap=0)), INV, ["capacity=0"]),
    ("k null", lambda: attn(ca=cache(k=None)), INV, ["cache.k is NULL"]),
    ("k misaligned", lambda: attn(ca=cache(k=FAKE + 8)), INV, ["cache.k", "16-byte aligned"]),
    ("q null", lambda: attn(q=None), INV, ["q is NULL"]),
    ("part_o null", lambda: attn(po=None), INV, ["part_o is NULL"]),
    ("lens null", lambda: attn(lens=None), INV, ["seq_lens is NULL"]),
], ids=lambda c: c[0])
def test_decode_attn_refusals(case):
    _, fn, status, needles = case
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_decode_attn: ")


@host_only
@pytest.mark.parametrize("case", [
    ("rope null", lambda: B.load().uaii_kv_produce(None, None, None, FAKE, FAKE, FAKE, None, None,
                                                    FAKE, 0), None, []),
    ("theta 0", lambda: produce(rope=B.Rope(0, 0, 0.0, 1, 1, 4, 8192)), INV, ["rope.theta=0"]),
    ("pairing 2", lambda: produce(rope=B.Rope(2, 0, 1e4, 1, 1, 4, 8192)), INV, ["rope.pairing=2"]),
    ("scaling 4", lambda: produce(rope=B.Rope(0, 4, 1e4, 1, 1, 4, 8192)), NI,
     ["unsupported rope_scaling.type=4", "yarn=3"]),
    ("linear factor 0", lambda: produce(rope=B.Rope(0, 2, 1e4, 0.0, 1, 4, 8192)), INV,
     ["rope.factor=0 is invalid for linear"]),
    ("yarn factor", lambda: produce(rope=B.Rope(0, 3, 1.5e5, 0.5, 1, 32, 4096)), INV,
     ["rope.factor=0.5 is invalid for yarn"]),
    ("yarn betas", lambda: produce(rope=B.Rope(0, 3, 1.5e5, 32, 32, 32, 4096)), INV,
     ["beta_fast)=32 must be finite and > beta_slow=32"]),
    ("yarn beta_slow", lambda: produce(rope=B.Rope(0, 3, 1.5e5, 32, 0, 32, 4096)), INV,
     ["beta_slow)=0"]),
    ("yarn orig", lambda: produce(rope=B.Rope(0, 3, 1.5e5, 32, 1, 32, 0)), INV,
     ["original_max_position=0"]),
    ("yarn attention factor", lambda: produce(rope=B.Rope(0, 3, 1.5e5, 32, 1, 32, 4096, 0, -1.0)),
     INV, ["rope.attention_factor=-1"]),
    ("llama3 factor", lambda: produce(rope=B.Rope(1, 1, 5e5, 0.5, 1, 4, 8192)), INV, ["rope.factor=0.5"]),
    ("llama3 high<=low", lambda: produce(rope=B.Rope(1, 1, 5e5, 8, 4, 4, 8192)), INV,
     ["high_freq_factor=4"]),
    ("llama3 low", lambda: produce(rope=B.Rope(1, 1, 5e5, 8, 0, 4, 8192)), INV, ["low_freq_factor=0"]),
    ("llama3 orig", lambda: produce(rope=B.Rope(1, 1, 5e5, 8, 1, 4, 0)), INV,
     ["original_max_position=0"]),
    ("norm eps", lambda: produce(norm=B.QKNorm(1, 0.0, 0, FAKE, FAKE)), INV, ["qk_norm.eps=0"]),
    ("norm offset", lambda: produce(norm=B.QKNorm(1, 1e-6, 2, FAKE, FAKE)), INV, ["qk_norm.offset=2"]),
    ("norm weight", lambda: produce(norm=B.QKNorm(1, 1e-6, 1, None, FAKE)), INV,
     ["qk_norm.q_weight is NULL"]),
    ("position", lambda: produce(pos=(3, 64)), INV, ["positions[1]=64", "capacity=64"]),
    ("position neg", lambda: produce(pos=(-1, 0)), INV, ["positions[0]=-1"]),
    ("q_in misaligned", lambda: produce(q_in=FAKE + 4), INV, ["q_in", "16-byte aligned"]),
    ("q_out null", lambda: produce(q_out=None), INV, ["q_out is NULL"]),
    ("head_dim", lambda: produce(sh=shape(d=80)), NI, ["head_dim=80"]),
], ids=lambda c: c[0])
def test_kv_produce_refusals(case):
    name, fn, status, needles = case
    if status is None:
        assert fn() == INV
        assert "shape is NULL" in B.last_error()
        return
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_kv_produce: ")


@host_only
@pytest.mark.parametrize("case", [
    ("window", lambda: combine(window=-3), INV, ["window=-3"]),
    ("split", lambda: combine(split=0), INV, ["split_size=0"]),
    ("max_splits", lambda: combine(lens=(100, 1), max_splits=3), INV, ["max_splits=3"]),
    ("out null", lambda: combine(out=None), INV, ["out is NULL"]),
    ("batch", lambda: combine(sh=shape(b=33), lens=[1] * 33), NI, ["batch=33"]),
], ids=lambda c: c[0])
def test_decode_combine_refusals(case):
    _, fn, status, needles = case
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_decode_combine: ")


@host_only
@pytest.mark.parametrize("case", [
    ("sinks null", lambda: combine_sink(sinks=None), INV, ["sinks is NULL"]),
    ("sinks misaligned", lambda: combine_sink(sinks=FAKE + 2), INV, ["sinks", "4-byte aligned"]),
    ("window", lambda: combine_sink(window=-3), INV, ["window=-3"]),
    ("out null", lambda: combine_sink(out=None), INV, ["out is NULL"]),
    ("head_dim", lambda: combine_sink(sh=shape(d=48)), NI, ["head_dim=48"]),
], ids=lambda c: c[0])
def test_decode_combine_sink_refusals(case):
    _, fn, status, needles = case
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_decode_combine_sink: ")


@host_only
def test_valid_call_without_device_reports_device_error():
    """A fully valid call reaches the launch; with no GPU the HIP error is
    reported as UAII_ERR_DEVICE with HIP's own text."""
    with pytest.raises(B.UaiiError) as ei:
        combine()
    assert ei.value.status == B.ERR_DEVICE
    assert "HIP error" in ei.value.message


@host_only
def test_error_text_is_per_call():
    with pytest.raises(B.UaiiError):
        attn(sh=shape(d=96))
    assert "head_dim=96" in B.last_error()
    assert B.load().uaii_decode_attn(None, None, None, None, 0.0, 0, 0.0, 1, 1, None, None,
                                     None) == INV
    assert "shape is NULL" in B.last_error()


@host_only
@pytest.mark.parametrize("case", [
    ("block size 8", dict(block_size=8), NI, ["block_size=8 is not supported"]),
    ("block size 48", dict(block_size=48), NI, ["block_size=48"]),
    ("block size 2048", dict(block_size=2048), NI, ["block_size=2048"]),
    ("max_blocks 0", dict(max_blocks=0), INV, ["max_blocks=0"]),
    ("num_blocks 0", dict(num_blocks=0), INV, ["num_blocks=0"]),
    ("capacity mismatch", dict(capacity=100), INV, ["capacity=100 must equal max_blocks*block_size=64"]),
    ("table misaligned", dict(table=FAKE + 2), INV, ["cache.block_table", "4-byte aligned"]),
], ids=lambda c: c[0])
def test_paged_cache_refusals(case):
    _, kw, status, needles = case
    c = B.KVCache(B.BF16, B.BF16, kw.get("capacity", 64), FAKE, FAKE, None,
                  kw.get("table", FAKE), kw.get("block_size", 16), kw.get("max_blocks", 4),
                  kw.get("num_blocks", 10))
    refused(lambda: attn(ca=c), status, *needles)
    refused(lambda: produce(ca=c, pos=(3, 4)), status, *needles)


@host_only
@pytest.mark.parametrize("case", [
    ("head_dim 96", lambda: step(sh=shape(d=96)), NI, ["head_dim=96 is not supported"]),
    ("batch 40", lambda: step(sh=shape(b=40), lens=[1] * 40), NI, ["batch=40"]),
    ("theta 0", lambda: step(rope=B.Rope(0, 0, 0.0, 1, 1, 4, 8192)), INV, ["rope.theta=0"]),
    ("scaling 4", lambda: step(rope=B.Rope(0, 4, 1e4, 1, 1, 4, 8192)), NI,
     ["unsupported rope_scaling.type=4"]),
    ("norm eps", lambda: step(norm=B.QKNorm(1, 0.0, 0, FAKE, FAKE)), INV, ["qk_norm.eps=0"]),
    ("scale", lambda: step(scale=0.1), NI, ["scale=0.1"]),
    ("window", lambda: step(window=-1), INV, ["window=-1"]),
    ("softcap", lambda: step(softcap=-2.0), INV, ["softcap=-2"]),
    ("len > cap", lambda: step(lens=(65, 5)), INV, ["seq_lens[0]=65"]),
    ("len 0", lambda: step(lens=(0, 5)), INV, ["seq_lens[0]=0"]),
    ("max_splits", lambda: step(lens=(10, 40), split=16, max_splits=2), INV, ["max_splits=2"]),
    ("q_out null", lambda: step(q_out=None), INV, ["q_out is NULL"]),
    ("counters null", lambda: step(counters=None), INV, ["counters is NULL"]),
    ("counters misaligned", lambda: step(counters=FAKE + 2), INV, ["counters", "4-byte aligned"]),
    ("sinks misaligned", lambda: step(sinks=FAKE + 2), INV, ["sinks", "4-byte aligned"]),
    ("out null", lambda: step(out=None), INV, ["out is NULL"]),
    ("vq8 no scale", lambda: step(ca=cache(vd=B.I8)), INV, ["v_scale is NULL"]),
    ("paged block size", lambda: step(ca=B.KVCache(B.BF16, B.BF16, 64, FAKE, FAKE, None, FAKE, 8,
                                                   8, 10)), NI, ["block_size=8"]),
], ids=lambda c: c[0])
def test_decode_step_refusals(case):
    _, fn, status, needles = case
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_decode_step: ")


@host_only
def test_decode_step_valid_call_reaches_the_launch():
    """A valid single-launch step with and without sinks gets past
    validation; with no GPU the launch fails with HIP's own text."""
    for sinks in (None, FAKE):
        with pytest.raises(B.UaiiError) as ei:
            step(sinks=sinks)
        assert ei.value.status == B.ERR_DEVICE
        assert ei.value.message.startswith("uaii_decode_step: HIP error")


def produce_chunk(sh=None, ca=None, start=(0, 4), n=8, q_out=FAKE):
    sh = sh or shape()
    rope = B.Rope(B.ROPE_NEOX, B.ROPE_PLAIN, 1e4, 1.0, 1.0, 4.0, 8192)
    B.kv_produce_chunk(sh, rope, None, FAKE, FAKE, FAKE, start, n, ca or cache(), q_out, 0)


def prefill(sh=None, ca=None, lens=(10, 20), n=8, scale=None, window=0, softcap=0.0, sinks=None,
            q=FAKE, out=FAKE):
    sh = sh or shape()
    scale = 1.0 / math.sqrt(sh.head_dim) if scale is None else scale
    B.prefill_attn(sh, ca or cache(), q, lens, n, scale, window, softcap, sinks, out, 0)


@host_only
@pytest.mark.parametrize("case", [
    ("n_tokens 0", lambda: produce_chunk(n=0), INV, ["n_tokens=0"]),
    ("n_tokens too many", lambda: produce_chunk(n=70000), NI, ["n_tokens=70000", "1..65535"]),
    ("start + n > cap", lambda: produce_chunk(start=(0, 60)), INV,
     ["start_positions[1]=60 with n_tokens=8", "capacity=64"]),
    ("start negative", lambda: produce_chunk(start=(-1, 0)), INV, ["start_positions[0]=-1"]),
    ("start null", lambda: B.load().uaii_kv_produce_chunk(
        B.Shape(2, 8, 2, 128), B.Rope(0, 0, 1e4, 1, 1, 4, 8192), None, FAKE, FAKE, FAKE, None, 4,
        cache(), FAKE, None), None, []),
    ("q_out null", lambda: produce_chunk(q_out=None), INV, ["q_out is NULL"]),
    ("head_dim", lambda: produce_chunk(sh=shape(d=32)), NI, ["head_dim=32"]),
], ids=lambda c: c[0])
def test_kv_produce_chunk_refusals(case):
    name, fn, status, needles = case
    if status is None:
        assert fn() == INV
        assert "start_positions is NULL" in B.last_error()
        return
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_kv_produce_chunk: ")


@host_only
@pytest.mark.parametrize("case", [
    ("f32 cache at head_dim 256", lambda: prefill(sh=shape(d=256), ca=cache(kd=B.F32, vd=B.F32)), NI,
     ["f32 caches with head_dim=256 is not supported", "64 and 128"]),
    ("bf16 keys, f32 values", lambda: prefill(ca=cache(kd=B.BF16, vd=B.F32)), NI,
     ["prefill over k_dtype=1, v_dtype=0 is not supported", "(1,1), (1,2), (2,2), (0,0)"]),
    ("f32 keys, int8 values", lambda: prefill(ca=cache(kd=B.F32, vd=B.I8, s=FAKE)), NI,
     ["k_dtype=0, v_dtype=2"]),
    ("vq8 without scales", lambda: prefill(ca=cache(vd=B.I8)), INV, ["v_scale is NULL"]),
    ("len < n_tokens", lambda: prefill(lens=(5, 20)), INV, ["seq_lens[0]=5", "n_tokens=8"]),
    ("len > cap", lambda: prefill(lens=(65, 20)), INV, ["seq_lens[0]=65"]),
    ("n_tokens 0", lambda: prefill(n=0), INV, ["n_tokens=0"]),
    ("window", lambda: prefill(window=-2), INV, ["window=-2"]),
    ("softcap", lambda: prefill(softcap=float("nan")), INV, ["softcap=nan"]),
    ("scale", lambda: prefill(scale=0.2), NI, ["scale=0.2"]),
    ("q null", lambda: prefill(q=None), INV, ["q is NULL"]),
    ("out misaligned", lambda: prefill(out=FAKE + 4), INV, ["out", "16-byte aligned"]),
    ("sinks misaligned", lambda: prefill(sinks=FAKE + 1), INV, ["sinks", "4-byte aligned"]),
    ("gqa 3", lambda: prefill(sh=shape(h=6, hkv=2)), NI, ["n_heads/n_kv_heads=3"]),
], ids=lambda c: c[0])
def test_prefill_attn_refusals(case):
    _, fn, status, needles = case
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_prefill_attn: ")


@host_only
def test_prefill_valid_calls_reach_the_launch():
    for fn in (lambda: prefill(), lambda: prefill(sinks=FAKE, window=3, softcap=5.0),
               lambda: prefill(ca=cache(vd=B.I8, s=FAKE)),
               lambda: prefill(ca=cache(kd=B.I8, vd=B.I8, s=FAKE, ks=FAKE)),
               lambda: produce_chunk()):
        with pytest.raises(B.UaiiError) as ei:
            fn()
        assert ei.value.status == B.ERR_DEVICE


def step_noalloc(sh=None, ca=None, lens=(10, 20), split=16, window=0, q_out=FAKE, out=FAKE):
    sh = sh or shape()
    rope = B.Rope(B.ROPE_NEOX, B.ROPE_PLAIN, 1e4, 1.0, 1.0, 4.0, 8192)
    B.decode_step_noalloc(sh, rope, None, FAKE, FAKE, FAKE, lens, ca or cache(),
                          1.0 / math.sqrt(sh.head_dim), window, 0.0, split, None, q_out, out, 0)


@host_only
@pytest.mark.parametrize("case", [
    # 32 * 64 * 512 splits * 129 * 4 bytes > 16 MiB
    ("partials beyond the scratch", lambda: step_noalloc(sh=shape(b=32, h=64, hkv=8, d=128),
                                                         ca=cache(cap=8192), lens=[8192] * 32,
                                                         split=16),
     NI, ["static scratch holds", "split_size=16"]),
    ("counters beyond the scratch", lambda: step_noalloc(sh=shape(b=32, h=1024, hkv=1024, d=64),
                                                         lens=[1] * 32, split=64),
     NI, ["batch*n_kv_heads=32768"]),
    ("len 0", lambda: step_noalloc(lens=(0, 5)), INV, ["seq_lens[0]=0"]),
    ("len > cap", lambda: step_noalloc(lens=(65, 5)), INV, ["seq_lens[0]=65"]),
    ("split 0", lambda: step_noalloc(split=0), INV, ["split_size=0"]),
    ("window", lambda: step_noalloc(window=-1), INV, ["window=-1"]),
    ("out null", lambda: step_noalloc(out=None), INV, ["out is NULL"]),
    ("head_dim", lambda: step_noalloc(sh=shape(d=96)), NI, ["head_dim=96"]),
], ids=lambda c: c[0])
def test_decode_step_noalloc_refusals(case):
    _, fn, status, needles = case
    msg = refused(fn, status, *needles)
    assert msg.startswith("uaii_decode_step_noalloc: ")


@host_only
def test_decode_step_noalloc_valid_call_reaches_the_device():
    """A valid call gets past validation; with no GPU, taking the scratch
    address on the device fails with HIP's own text."""
    with pytest.raises(B.UaiiError) as ei:
        step_noalloc()
    assert ei.value.status == B.ERR_DEVICE
    assert ei.value.message.startswith("uaii_decode_step_noalloc: HIP error")
