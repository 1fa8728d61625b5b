"""GPU parity for the paged cache layout: the same logical cache scattered
into block pools through a random block table (the generator's paged
scatter), against the CPU oracle on the contiguous form.  Cases cover block
sizes 16..1024, windows that start inside a block, one-key sequences, vq8
scales, d64/d128/256, and the B=32 ctx-8K workload at full size."""
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


def case(name, d, G, Hkv, kdt, vdt, lens, S, bs, window=0, softcap=0.0, norm=None, seed=0,
         pairing=W.NEOX, scaling=W.PLAIN, theta=1e4):
    lens = tuple(int(x) for x in lens)
    qn = W.QKNorm(False) if norm is None else W.QKNorm(True, 1e-6, norm, 1.0 - norm, 0.1)
    w = W.Workload(name, len(lens), Hkv * G, Hkv, d, ("fixed", lens[0]), max(lens) + 5, kdt, vdt,
                   W.Rope(pairing, scaling, theta, 8.0, 1.0, 4.0, 8192), qn, window, softcap, S,
                   (2000 + seed,))
    return w, np.array(lens, np.int32), bs


PAGED = [
    case("bf16-d128-g4-bs16-ragged", 128, 4, 2, W.BF16, W.BF16, [1, 700, 1500], 512, 16, seed=1,
         pairing=W.INTERLEAVED, scaling=W.LLAMA3, theta=5e5),
    case("vq8-d128-g4-bs32-norm", 128, 4, 2, W.BF16, W.I8, [513, 1024], 256, 32, norm=0, seed=2),
    case("bf16-d256-g2-bs64-window-softcap", 256, 2, 2, W.BF16, W.BF16, [1000, 90], 128, 64,
         window=100, softcap=50.0, norm=1, seed=3),
    case("f32-d64-g2-bs16-tiny", 64, 2, 2, W.F32, W.F32, [129], 65, 16, seed=4),
    case("bf16-d64-g8-bs1024", 64, 8, 1, W.BF16, W.BF16, [2500, 17], 512, 1024, seed=5),
    case("bf16-d128-g1-bs16-window37", 128, 1, 4, W.BF16, W.BF16, [400, 36, 1000], 100, 16,
         window=37, seed=6),
    case("vq8-f32k-d64-g4-bs16-window", 64, 4, 2, W.F32, W.I8, [777, 300], 64, 16, window=333,
         seed=7),
    case("bf16-d128-g4-bs128-multichunk", 128, 4, 2, W.BF16, W.BF16, [2100, 1500], 1500, 128,
         seed=8),
    case("vq8-d256-g2-bs16-softcap-multichunk", 256, 2, 2, W.BF16, W.I8, [1600], 1100, 16,
         softcap=50.0, seed=9),
    case("bf16-d128-g8-bs16-softcap", 128, 8, 2, W.BF16, W.BF16, [1500, 300], 512, 16, softcap=30.0,
         seed=10),
]


@pytest.mark.parametrize("spec", PAGED, ids=[c[0].name for c in PAGED])
def test_paged_case(spec):
    w, lens, bs = spec
    P.run_and_compare(w, lens, max_partials_per_seq=8, seed=1, block_size=bs)


def test_paged_matches_contiguous():
    """The paged and contiguous layouts give the same outputs up to f32
    rounding (the tile grid and hence summation order can differ)."""
    w, lens, bs = PAGED[0]
    inputs = W.make_inputs(w, seq_lens=lens)
    a = P.run_gpu(inputs)
    b = P.run_gpu(inputs, paged=W.make_paged(inputs, bs))
    assert float((a.out - b.out).abs().max()) < 1e-6
    assert torch.equal(a.q_out, b.q_out)


def test_paged_full_size_b32_ctx8k():
    """B=32 sequences of 8192 keys, 32/8 heads, d128, bf16, block size 16,
    through a random block table; sampled outputs and partials."""
    w = W.WORKLOADS[W.HEADLINE]
    P.say(f"paged full-size {w.name}, block_size 16")
    inputs = W.make_inputs(w)
    paged = W.make_paged(inputs, 16)
    st = P.run_gpu(inputs, paged=paged)
    ref = P.OracleStep(inputs, copy_cache=False)
    rng = np.random.default_rng(5)
    pairs = [(b, int(h)) for b in range(w.batch) for h in rng.choice(w.n_heads, 3, replace=False)]
    out = st.out.cpu().numpy()
    want = ref.decode(pairs)
    got = np.stack([out[b, h] for b, h in pairs])
    err = float(np.max(np.abs(got - want)))
    P.check_slot(w, st.cache_rows(), ref.slot_rows(), st.q_out.cpu().numpy(), ref.q)
    sel = {b: [h for bb, h in pairs if bb == b][:1] for b in range(w.batch)}
    P.compare_partials(st, ref, w, inputs.seq_lens, pick=lambda b: sel[b])
    P.say(f"  sampled {len(pairs)} outputs: max abs err {err:.3g}")
    assert err <= P.TOL_BF16
