"""Randomised parity sweep over the fact space: batch, head_dim, GQA ratio,
cache dtypes, lengths (including one key), window edges, softcap, split size,
RoPE pairing and scaling, QK-norm.  Every cell compares all outputs, the
produced cache rows and the split partials (a sample when there are many)
with the CPU oracle.  Cells are drawn from a fixed seed."""
import numpy as np
import pytest

import parity as P
from gqa_decode_attention_kv_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CELLS = 28


def draw_cell(i):
    rng = np.random.default_rng([20260, i])
    d = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([1, 2, 3, 5, 32] if d < 256 else [1, 2, 3]))
    maxL = 2000 if B <= 5 else 300
    lens = rng.integers(1, maxL + 1, B)
    if i % 5 == 0:
        lens[0] = 1
    L0 = int(lens.max())
    W_choice = [0, 1, 7, max(1, L0 - 1), L0, L0 + 5]
    window = int(W_choice[i % len(W_choice)])
    softcap = float(rng.choice([0.0, 1.0, 50.0]))
    S = int(rng.choice([1, 16, 512, 4096])) if L0 <= 64 else int(rng.choice([16, 100, 512, 4096]))
    kv = [(W.F32, W.F32), (W.BF16, W.BF16), (W.BF16, W.I8), (W.F32, W.I8), (W.F32, W.BF16)][i % 5]
    pairing = int(rng.integers(0, 2))
    scaling = int(rng.integers(0, 2))
    theta = float(rng.choice([1e4, 5e5, 1e6]))
    norm = [None, 0, 1][i % 3]
    qn = W.QKNorm(False) if norm is None else W.QKNorm(True, 1e-6, norm, 1.0 - norm, 0.1)
    w = W.Workload(f"sweep{i}", B, Hkv * G, Hkv, d, ("fixed", L0), L0 + int(rng.integers(0, 9)),
                   kv[0], kv[1], W.Rope(pairing, scaling, theta, float(rng.choice([2.0, 8.0, 32.0])),
                                        1.0, 4.0, 8192), qn, window, softcap, S, (30000 + i,))
    return w, lens.astype(np.int32)


CELLS = [draw_cell(i) for i in range(N_CELLS)]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("cell", CELLS, ids=[c[0].name for c in CELLS])
def test_sweep_cell(cell):
    w, lens = cell
    P.run_and_compare(w, lens, max_partials_per_seq=6, seed=int(w.seed[0]))
