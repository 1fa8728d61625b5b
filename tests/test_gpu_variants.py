"""GPU parity of the cache, rotary and softmax variants against the CPU
oracle, through the C ABI:

* q8 cache: int8 keys and values, each with an f32 scale per token per kv
  head ("llamay - Models and formats", The KV cache, in three precisions);
* attention sink: one logit per query head in the softmax denominator
  (same page, Architectures: gpt-oss), applied by uaii_decode_combine_sink;
* linear RoPE scaling ("Algenta - Model support matrix", Decoder families:
  gemma3) and YaRN ("Universal AI Inference - Hugging Face decoder
  completeness", P0.2; llamay Architectures: gpt-oss).

Small cases compare every output element, produced cache row and split
partial; the named workloads run at full size with sampled outputs and
partials.  Tolerances are those of the other parity tests (int8 caches:
1e-2 of the output's max-abs; f32 1e-5; bf16 2e-3).
"""
import numpy as np
import pytest

import parity as P
from gqa_decode_attention_kv_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gqa_decode_attention_kv_amd import binding
    binding.load()


GPT_OSS_YARN = W.Rope(W.NEOX, W.YARN, 150000.0, 32.0, 1.0, 32.0, 4096, False)


def case(name, d, G, Hkv, kdt, vdt, lens, S, window=0, softcap=0.0, rope=None, norm=None,
         sink=False, seed=0):
    lens = tuple(int(x) for x in lens)
    cap = max(lens) + 3
    qn = W.QKNorm(False) if norm is None else W.QKNorm(True, 1e-6, norm, 1.0 - norm, 0.1)
    w = W.Workload(name, len(lens), Hkv * G, Hkv, d, ("fixed", lens[0]), cap, kdt, vdt,
                   rope or W.Rope(W.NEOX, W.PLAIN, 1e4), qn, window, softcap, S, (2000 + seed,),
                   sink)
    return w, np.array(lens, np.int32)


SMALL = [
    # q8 over head dims, group sizes, windows, softcap and ragged lengths
    case("q8-d128-g4", 128, 4, 2, W.I8, W.I8, [700, 1025, 1], 512,
         rope=W.Rope(W.INTERLEAVED, W.LLAMA3, 5e5, 8.0), seed=1),
    case("q8-d64-g8-window", 64, 8, 2, W.I8, W.I8, [900, 40], 256, window=200, seed=2),
    case("q8-d256-g2-softcap", 256, 2, 2, W.I8, W.I8, [1300, 513], 512, softcap=50.0, norm=1,
         seed=3),
    case("q8-d128-g1-split1", 128, 1, 3, W.I8, W.I8, [33, 2], 1, seed=4),
    case("q8-d64-g2-multichunk", 64, 2, 1, W.I8, W.I8, [2100], 1100, norm=0, seed=5),
    # attention sink, alone and with window / softcap / int8 values
    case("sink-f32-d64-g8", 64, 8, 2, W.F32, W.F32, [1000, 129, 1], 256, rope=GPT_OSS_YARN,
         sink=True, seed=6),
    case("sink-f32-d64-g8-window128", 64, 8, 2, W.F32, W.F32, [1000, 100], 128, window=128,
         rope=GPT_OSS_YARN, sink=True, seed=7),
    case("sink-bf16-d128-softcap", 128, 4, 2, W.BF16, W.BF16, [600, 77], 256, softcap=30.0,
         sink=True, seed=8),
    case("sink-vq8-d128", 128, 2, 2, W.BF16, W.I8, [800], 512, sink=True, seed=9),
    # linear scaling and YaRN
    case("linear-bf16-d128-g2", 128, 2, 4, W.BF16, W.BF16, [2000, 5], 512,
         rope=W.Rope(W.NEOX, W.LINEAR, 1e6, 8.0), norm=1, seed=10),
    case("linear-f32-d256-interleaved", 256, 1, 2, W.F32, W.F32, [300], 128,
         rope=W.Rope(W.INTERLEAVED, W.LINEAR, 1e4, 0.5), seed=11),
    case("yarn-truncated-bf16-d128", 128, 4, 2, W.BF16, W.BF16, [3000, 17], 1024,
         rope=W.Rope(W.INTERLEAVED, W.YARN, 1e4, 16.0, 1.0, 32.0, 4096, True), seed=12),
    case("yarn-attn-factor-f32-d64", 64, 4, 2, W.F32, W.F32, [500], 128,
         rope=W.Rope(W.NEOX, W.YARN, 150000.0, 32.0, 1.0, 32.0, 4096, False, 1.7), norm=0,
         seed=13),
    case("yarn-q8-d128", 128, 4, 2, W.I8, W.I8, [1200], 512,
         rope=W.Rope(W.NEOX, W.YARN, 1e6, 4.0, 2.0, 64.0, 32768, True), seed=14),
    # int8 caches at G = 8 (the key pass on the matrix cores in two groups
    # of four heads, 256-row chunks): cooperative items, a window, softcap
    # with a sink, d64, and one wave per item
    case("vq8-d128-g8", 128, 8, 2, W.BF16, W.I8, [1500, 700, 3], 512, seed=15),
    case("q8-d128-g8-softcap-sink", 128, 8, 1, W.I8, W.I8, [2000, 65], 256, softcap=30.0,
         sink=True, seed=16),
    case("vq8-d64-g8-window", 64, 8, 2, W.BF16, W.I8, [1700, 90], 256, window=600, seed=17),
    case("q8-d128-g8-lone", 128, 8, 8, W.I8, W.I8, [2048] * 8, 64, seed=18),
    # f32 caches at G = 8 (the key pass on the f32 matrix cores): cooperative
    # items with softcap at d128, and one wave per item with the sink and
    # gpt-oss's YaRN at d64 and with a window at d128
    case("f32-d128-g8-softcap", 128, 8, 2, W.F32, W.F32, [1500, 700, 3], 512, softcap=30.0,
         seed=19),
    case("f32-d64-g8-lone-sink", 64, 8, 8, W.F32, W.F32, [2048] * 8, 64, rope=GPT_OSS_YARN,
         sink=True, seed=20),
    case("f32-d128-g8-lone-window", 128, 8, 8, W.F32, W.F32, [2048] * 8, 64, window=900,
         seed=21),
    # one wave per item over items of unequal size (ragged lengths, 40-key
    # splits, about 3900 items): the work-groups take the serpentine
    # placement, here through the int8 and f32 kernels
    case("q8-d128-g8-lone-ragged", 128, 8, 8, W.I8, W.I8,
         np.random.default_rng(22).integers(300, 901, 32), 40, seed=22),
    case("vq8-d128-g4-lone-ragged", 128, 4, 8, W.BF16, W.I8,
         np.random.default_rng(23).integers(300, 901, 32), 40, seed=23),
    case("f32-d64-g8-lone-ragged-sink", 64, 8, 8, W.F32, W.F32,
         np.random.default_rng(24).integers(300, 901, 32), 40, rope=GPT_OSS_YARN, sink=True,
         seed=24),
]


@pytest.mark.parametrize("spec", SMALL, ids=[c[0].name for c in SMALL])
def test_variant_small(spec):
    w, lens = spec
    P.run_and_compare(w, lens)


PAGED = [
    (SMALL[0], 16), (SMALL[1], 32), (SMALL[5], 16), (SMALL[11], 64), (SMALL[14], 16),
    (SMALL[15], 32), (SMALL[18], 16), (SMALL[19], 32), (SMALL[20], 16), (SMALL[21], 16),
]


@pytest.mark.parametrize("spec,bs", PAGED, ids=[f"{c[0].name}-bs{b}" for c, b in PAGED])
def test_variant_paged(spec, bs):
    w, lens = spec
    P.run_and_compare(w, lens, block_size=bs)


FULL = ["llama3.1-8b-q8", "gpt-oss-20b-full", "gpt-oss-20b-sliding", "gemma3-27b-global",
        "gemma3-27b-local", "llama3.1-70b-q8", "llama3.1-70b-vq8", "llama3.1-70b-b32-ctx8k"]


@pytest.mark.parametrize("name", FULL)
def test_variant_full_size(name):
    P.check_full_size(W.WORKLOADS[name])


def test_sink_far_below_is_the_plain_combine():
    """A sink of -1e30 contributes e^(sink - M) = 0: the sink combine then
    gives the plain combine's output bit for bit, and a sink far above every
    score drives the output to 0 (all mass on the sink)."""
    from gqa_decode_attention_kv_amd import binding as B
    w, lens = SMALL[5]
    inputs = W.make_inputs(w, seq_lens=lens)
    st = P.run_gpu(inputs)
    plain = torch.empty_like(st.out)
    B.decode_combine(st.shape, st.seq_lens, w.window, st.split_size, st.max_splits,
                     st.part_o.data_ptr(), st.part_lse.data_ptr(), plain.data_ptr(), st.stream())
    far = torch.full((w.n_heads,), -1e30, dtype=torch.float32, device=st.out.device)
    low = torch.empty_like(st.out)
    B.decode_combine_sink(st.shape, st.seq_lens, w.window, st.split_size, st.max_splits,
                          st.part_o.data_ptr(), st.part_lse.data_ptr(), far.data_ptr(),
                          low.data_ptr(), st.stream())
    high_sink = torch.full((w.n_heads,), 1e4, dtype=torch.float32, device=st.out.device)
    high = torch.empty_like(st.out)
    B.decode_combine_sink(st.shape, st.seq_lens, w.window, st.split_size, st.max_splits,
                          st.part_o.data_ptr(), st.part_lse.data_ptr(), high_sink.data_ptr(),
                          high.data_ptr(), st.stream())
    torch.cuda.synchronize()
    assert torch.equal(low, plain)
    assert float(high.abs().max()) == 0.0
    # and the workload's own sinks moved the output (the sink is not a no-op)
    assert not torch.equal(st.out, plain)
