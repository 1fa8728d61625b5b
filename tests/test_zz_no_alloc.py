"""uaii_decode_step_noalloc, the one-call decode step for callers that
cannot allocate: its partials and arrival counters live in the library's
static per-GPU scratch.  Through the C ABI it must give what
uaii_decode_step gives with caller-owned buffers (the same kernels, so the
same bits), and both must match the oracle at the class tolerance.  Calls
follow one another on the same scratch with shrinking inputs: a large step
(three kernels), a one-kernel step, a smaller one-kernel step with a sink,
and a paged one; a step too large for the scratch is refused before
anything is written."""
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


def case(name, d, G, Hkv, kdt, vdt, lens, S, window=0, softcap=0.0, norm=None, sink=False,
         seed=0, rope=None):
    lens = tuple(int(x) for x in lens)
    cap = max(lens) + 3
    qn = W.QKNorm(False) if norm is None else W.QKNorm(True, 1e-6, norm, 1.0 - norm, 0.1)
    w = W.Workload(name, len(lens), Hkv * G, Hkv, d, ("fixed", lens[0]), cap, kdt, vdt,
                   rope or W.Rope(W.NEOX, W.PLAIN, 1e4), qn, window, softcap, S, (4000 + seed,),
                   sink)
    return w, np.array(lens, np.int32)


def noalloc_step(st, split_size=None):
    from gqa_decode_attention_kv_amd import binding as B
    B.decode_step_noalloc(st.shape, st.rope, st.qk_norm, st.q_in.data_ptr(), st.k_in.data_ptr(),
                          st.v_in.data_ptr(), st.seq_lens, st.cache, st.scale, st.w.window,
                          st.w.softcap, split_size or st.split_size,
                          st.sinks.data_ptr() if st.sinks is not None else None,
                          st.q_out.data_ptr(), st.out.data_ptr(), st.stream())


def run_pair(w, lens, block_size=None):
    """The same step through uaii_decode_step (caller buffers) and through
    uaii_decode_step_noalloc; returns (out with buffers, out without)."""
    from gqa_decode_attention_kv_amd.step import DeviceStep
    P.say(f"case {w.name}: B={w.batch} H={w.n_heads}/{w.n_kv_heads} d={w.head_dim} "
          f"lens={lens.tolist()[:8]} S={w.split_size} paged={block_size}")
    inputs = W.make_inputs(w, seq_lens=lens)
    paged = W.make_paged(inputs, block_size) if block_size else None
    a = DeviceStep(inputs, paged=paged)
    b = DeviceStep(inputs, paged=paged)
    a.out.fill_(float("nan"))
    b.out.fill_(float("nan"))
    a.fused_step()
    noalloc_step(b)
    torch.cuda.synchronize()
    assert torch.equal(a.q_out, b.q_out)
    for k in ("k", "v"):
        assert np.array_equal(a.cache_rows()[k], b.cache_rows()[k])
    ref = P.OracleStep(inputs)
    want = ref.decode().reshape(a.out.shape)
    tol, cls = P.out_tolerance(w, want)
    got_a, got_b = a.out.cpu().numpy(), b.out.cpu().numpy()
    err = float(np.max(np.abs(got_b - want)))
    P.say(f"  no-alloc vs oracle {err:.3g} (tol {tol:.3g}, {cls}); "
          f"vs uaii_decode_step {float(np.max(np.abs(got_b - got_a))):.3g}")
    assert err <= tol, (err, tol)
    assert np.array_equal(got_a, got_b), "no-alloc step differs from uaii_decode_step"
    return b


STEPS = [
    # 32 x 8 kv heads x 4 splits = 1024 items: the three kernels back to back
    case("b32-d128-g4-three-kernels", 128, 4, 8, W.BF16, W.BF16,
         np.random.default_rng(1).integers(1500, 2049, 32), 512, seed=1,
         rope=W.Rope(W.INTERLEAVED, W.LLAMA3, 5e5, 8.0)),
    # one kernel (<= 256 items), then a smaller one
    case("b4-d128-g4-one-kernel", 128, 4, 2, W.BF16, W.BF16, [1, 17, 513, 1500], 512, seed=2),
    case("b2-d64-g8-sink-window", 64, 8, 2, W.F32, W.F32, [300, 64], 128, window=100, sink=True,
         seed=3),
    case("b1-vq8-qknorm", 128, 4, 1, W.BF16, W.I8, [700], 256, norm=0, seed=4),
]


def test_no_alloc_matches_decode_step_on_consecutive_calls():
    for w, lens in STEPS:
        run_pair(w, lens)


def test_no_alloc_paged_after_contiguous():
    w, lens = case("paged-b3-d256-g2-softcap", 256, 2, 2, W.BF16, W.BF16, [900, 40, 513], 256,
                   softcap=50.0, seed=5)
    run_pair(w, lens, block_size=16)
    w, lens = case("small-after-paged", 64, 2, 2, W.F32, W.F32, [129], 65, seed=6)
    run_pair(w, lens)


def test_no_alloc_refuses_steps_beyond_the_scratch():
    """Partials over 16 MiB are refused before any launch: q_out, out and the
    cache stay as they were, and a following valid call still works."""
    from gqa_decode_attention_kv_amd import binding as B
    from gqa_decode_attention_kv_amd.step import DeviceStep
    w, lens = STEPS[0]
    inputs = W.make_inputs(w, seq_lens=lens)
    st = DeviceStep(inputs)
    st.out.fill_(7.0)
    st.q_out.fill_(7.0)
    k0 = st.cache_k.clone()
    torch.cuda.synchronize()
    # split 16 at 2048 keys: 32 * 32 * 128 splits * 129 * 4 bytes = 67.6 MB
    with pytest.raises(B.UaiiError, match="static scratch holds"):
        noalloc_step(st, split_size=16)
    torch.cuda.synchronize()
    assert bool((st.out == 7.0).all()) and bool((st.q_out == 7.0).all())
    assert torch.equal(k0, st.cache_k)
    run_pair(*STEPS[1])
