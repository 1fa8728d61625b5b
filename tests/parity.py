"""Helpers that run one decode step on the GPU and the same step in the CPU
oracle, and compare them.  Not a test module (no test_ prefix)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from gqa_decode_attention_kv_amd import workloads as W

# Tolerances on the final output (max abs error; vq8 relative to max |out|).
TOL_F32 = 1e-5
TOL_BF16 = 2e-3
TOL_VQ8_REL = 1e-2


def out_tolerance(w: W.Workload, ref: np.ndarray) -> tuple[float, str]:
    """Absolute tolerance for workload w (the int8 bound, vq8 and q8, is
    relative to the oracle output's max-abs)."""
    if w.v_dtype == W.I8:
        return TOL_VQ8_REL * float(np.max(np.abs(ref))), "int8 1e-2 x max|out|"
    if w.k_dtype == W.BF16 or w.v_dtype == W.BF16:
        return TOL_BF16, "bf16 2e-3"
    return TOL_F32, "f32 1e-5"


def say(msg: str):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def _workers():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


class OracleStep:
    """The oracle's version of the step on its own copy of the inputs."""

    def __init__(self, inputs: W.Inputs, copy_cache: bool = True):
        o = oracle.load()
        w = inputs.workload
        self.o, self.w, self.inputs = o, w, inputs
        self.ck = inputs.cache_k.copy() if copy_cache else inputs.cache_k
        self.cv = inputs.cache_v.copy() if copy_cache else inputs.cache_v
        vs, ks = inputs.v_scale, inputs.k_scale
        self.vs = (vs.copy() if copy_cache else vs) if vs is not None else None
        self.ks = (ks.copy() if copy_cache else ks) if ks is not None else None
        self.sinks = inputs.sinks
        norm = None
        if w.qk_norm.enabled:
            norm = dict(enabled=True, eps=w.qk_norm.eps, offset=w.qk_norm.offset,
                        w_q=inputs.w_q, w_k=inputs.w_k)
        self.q = o.kv_produce(rope=w.rope.as_dict(), norm=norm, q_in=inputs.q_in,
                              k_in=inputs.k_in, v_in=inputs.v_in, positions=inputs.positions,
                              k_dtype=w.k_dtype, v_dtype=w.v_dtype, cache_k=self.ck,
                              cache_v=self.cv, v_scale=self.vs, k_scale=self.ks)

    def slot_rows(self):
        b = np.arange(self.w.batch)
        p = self.inputs.positions
        k = self.ck[b, :, p]
        v = self.cv[b, :, p]
        s = self.vs[b, :, p] if self.vs is not None else None
        ks = self.ks[b, :, p] if self.ks is not None else None
        return dict(k=k, v=v, scale=s, k_scale=ks)

    def decode(self, pairs=None) -> np.ndarray:
        w = self.w
        kw = dict(q=self.q, cache_k=self.ck, cache_v=self.cv, v_scale=self.vs, k_scale=self.ks,
                  k_dtype=w.k_dtype, v_dtype=w.v_dtype, seq_lens=self.inputs.seq_lens,
                  window=w.window, softcap=w.softcap, sinks=self.sinks)
        if pairs is None:
            pairs = [(b, h) for b in range(w.batch) for h in range(w.n_heads)]
        pairs = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
        n = _workers()
        chunks = [c for c in np.array_split(pairs, n) if len(c)]
        with ThreadPoolExecutor(len(chunks)) as ex:
            parts = list(ex.map(lambda c: self.o.decode(pairs=c, **kw), chunks))
        return np.concatenate(parts, axis=0)

    def partial(self, b, h, sigma, split_size):
        w = self.w
        return self.o.split_partial(q_bh=self.q[b, h], cache_k=self.ck, cache_v=self.cv,
                                    v_scale=self.vs, k_scale=self.ks, k_dtype=w.k_dtype,
                                    v_dtype=w.v_dtype,
                                    n_heads=w.n_heads, b=b, h=h, L=int(self.inputs.seq_lens[b]),
                                    window=w.window, softcap=w.softcap, split_size=split_size,
                                    sigma=sigma)


def valid_splits(w: W.Workload, L: int, split_size: int):
    lo, hi = w.visible(L)
    return list(range(lo // split_size, (hi - 1) // split_size + 1))


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place (sign-magnitude ordering)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return np.abs(key(a) - key(b))


def check_slot(w: W.Workload, gpu: dict, ref: dict, q_gpu: np.ndarray, q_ref: np.ndarray) -> dict:
    """Produced rows: V bit-exact (f32 copy, bf16 RNE, int8 codes and scales),
    K within 1 bf16 ulp or 1e-6 relative (f32), q8 key codes within 1 and
    their scales within 1 f32 ulp, q' within 1e-6 relative."""
    res = {}
    qerr = np.max(np.abs(q_gpu.astype(np.float64) - q_ref)) / max(1e-30, np.max(np.abs(q_ref)))
    res["q_rel"] = float(qerr)
    assert qerr <= 1e-6, f"q_out relative error {qerr:.3g}"
    if w.k_dtype == W.BF16:
        u = bf16_ulps(gpu["k"], ref["k"])
        res["k_ulps"] = int(u.max())
        assert u.max() <= 1, f"K slot differs by {u.max()} bf16 ulps"
    elif w.k_dtype == W.I8:
        # The rotated key is rounded to f32 before quantising; a key whose
        # f32 rounding differs (a double-precision tie) could move a code by
        # one, so codes may differ by at most 1 and scales by 1 f32 ulp.
        dk = np.abs(gpu["k"].astype(np.int32) - ref["k"].astype(np.int32))
        du = np.abs(gpu["k_scale"].view(np.int32).astype(np.int64)
                    - ref["k_scale"].view(np.int32).astype(np.int64))
        res["k_code_diff"], res["k_scale_ulps"] = int(dk.max()), int(du.max())
        assert dk.max() <= 1 and du.max() <= 1, (dk.max(), du.max())
    else:
        kr = ref["k"].astype(np.float64)
        kerr = np.max(np.abs(gpu["k"].astype(np.float64) - kr)) / max(1e-30, np.max(np.abs(kr)))
        res["k_rel"] = float(kerr)
        assert kerr <= 1e-6, f"K slot relative error {kerr:.3g}"
    assert np.array_equal(gpu["v"], ref["v"]), "V slot differs (must be bit-exact)"
    if w.v_dtype == W.I8:
        assert np.array_equal(gpu["scale"].view(np.uint32), ref["scale"].view(np.uint32)), \
            "vq8 scales differ (must be bit-exact)"
    return res


def run_gpu(inputs, split_size=None, paged=None, fused=False):
    """One step on the GPU with NaN-filled partial buffers (so unwritten
    entries stay detectable): the three calls, or with fused=True the
    single-launch uaii_decode_step, run twice on the same inputs (the
    second run must reproduce the first bit for bit, which also shows that
    the arrival counters came back to zero)."""
    import torch
    from gqa_decode_attention_kv_amd.step import DeviceStep
    st = DeviceStep(inputs, split_size=split_size, paged=paged)
    st.part_o.fill_(float("nan"))
    st.part_lse.fill_(float("nan"))
    st.out.fill_(float("nan"))
    if not fused:
        st.step()
        torch.cuda.synchronize()
        return st
    st.fused_step()
    torch.cuda.synchronize()
    first = (st.out.clone(), st.q_out.clone())
    assert int(st.counters.abs().max()) == 0, "arrival counters not returned to zero"
    st.out.fill_(float("nan"))
    st.fused_step()
    torch.cuda.synchronize()
    assert torch.equal(st.out, first[0]), "second fused step differs from the first"
    assert torch.equal(st.q_out, first[1])
    assert int(st.counters.abs().max()) == 0, "arrival counters not returned to zero"
    return st


def compare_partials(st, ref, w, lens, pick=None, max_per_seq=None, rng=None):
    """Every valid split partial (or a sample) against the oracle's; splits
    outside the visible range must stay unwritten (NaN)."""
    po = st.part_o.cpu().numpy()
    pl = st.part_lse.cpu().numpy()
    worst = 0.0
    for b, L in enumerate(lens):
        valid = valid_splits(w, int(L), st.split_size)
        vset = set(valid)
        invalid = [sg for sg in range(st.max_splits) if sg not in vset]
        heads = range(w.n_heads) if pick is None else pick(b)
        for h in heads:
            if invalid:
                assert np.all(np.isnan(po[b, h, invalid])) and np.all(np.isnan(pl[b, h, invalid])), \
                    f"partial ({b},{h}) outside the visible range was written"
            chk = valid
            if pick is not None:
                chk = sorted({valid[0], valid[-1]})
            elif max_per_seq is not None and len(valid) > max_per_seq:
                chk = sorted({valid[0], valid[-1], *rng.choice(valid, max_per_seq - 2, replace=False).tolist()})
            for sg in chk:
                o, lse, n = ref.partial(b, h, sg, st.split_size)
                assert n > 0
                e_o = float(np.max(np.abs(po[b, h, sg] - o)))
                e_l = abs(float(pl[b, h, sg]) - lse)
                worst = max(worst, e_o)
                assert e_o <= out_tolerance(w, o)[0], (b, h, sg, e_o)
                assert e_l <= 1e-4 * max(1.0, abs(lse)), (b, h, sg, e_l, lse)
    return worst


def run_and_compare(w: W.Workload, lens, max_partials_per_seq=None, seed=0, block_size=None,
                    fused=False, prep=None):
    """Run one step on the GPU (three calls, or the single launch with
    fused=True) and in the oracle; compare every output element, the
    produced cache rows (and that nothing else in the caches changed) and
    the split partials.  ``prep(inputs)``, if given, edits the seeded inputs
    in place before either side sees them.  Returns (max abs error,
    tolerance, class)."""
    lens = np.asarray(lens, dtype=np.int32)
    say(f"case {w.name}{' fused' if fused else ''}: B={w.batch} H={w.n_heads}/{w.n_kv_heads} d={w.head_dim} "
        f"K/V={w.k_dtype}/{w.v_dtype} lens={lens.tolist()[:8]} S={w.split_size} W={w.window} "
        f"cap={w.softcap} rope={w.rope.pairing}/{w.rope.scaling} norm={w.qk_norm.enabled} "
        f"sink={w.sink}")
    inputs = W.make_inputs(w, seq_lens=lens)
    if prep is not None:
        prep(inputs)
    paged = W.make_paged(inputs, block_size) if block_size else None
    if paged:
        say(f"  paged: block_size={paged.block_size} max_blocks={paged.max_blocks} "
            f"num_blocks={paged.num_blocks}")
        ck0, cv0 = paged.pool_k.copy(), paged.pool_v.copy()
        vs0, ks0 = paged.pool_scale, paged.pool_k_scale
    else:
        ck0, cv0 = inputs.cache_k.copy(), inputs.cache_v.copy()
        vs0, ks0 = inputs.v_scale, inputs.k_scale
    vs0 = vs0.copy() if vs0 is not None else None
    ks0 = ks0.copy() if ks0 is not None else None
    st = run_gpu(inputs, paged=paged, fused=fused)
    ref = OracleStep(inputs)
    out = st.out.cpu().numpy()
    want = ref.decode().reshape(out.shape)
    tol, cls = out_tolerance(w, want)
    err = float(np.max(np.abs(out - want)))
    check_slot(w, st.cache_rows(), ref.slot_rows(), st.q_out.cpu().numpy(), ref.q)
    compare_partials(st, ref, w, lens, max_per_seq=max_partials_per_seq,
                     rng=np.random.default_rng(seed))
    mask = np.ones(ck0.shape[:3], bool)
    first, row = st.slot_index()
    mask[first, :, row] = False
    pairs = [(st.cache_k, ck0), (st.cache_v, cv0)]
    if st.v_scale is not None:
        pairs.append((st.v_scale, vs0))
    if st.k_scale is not None:
        pairs.append((st.k_scale, ks0))
    for dev, host in pairs:
        g = dev.cpu().numpy().view(host.dtype)
        assert np.array_equal(g[mask].view(np.uint8), host[mask].view(np.uint8)), \
            "cache rows other than the new token's slot changed"
    say(f"  max abs err {err:.3g} (tol {tol:.3g}, {cls})")
    assert err <= tol, (err, tol)
    return err, tol, cls


def check_full_size(w: W.Workload, block_size=None, fused=False):
    """A named workload at its full size, in the launch configuration the
    benchmark times: every produced cache row, and a sample of outputs
    (4 heads per sequence; every head for B = 1) and of split partials (the
    first and last valid split of 2 heads per sequence) against the oracle."""
    say(f"full-size {w.name}: B={w.batch} H={w.n_heads}/{w.n_kv_heads} d={w.head_dim} "
        f"cap={w.capacity} S={w.split_size} window={w.window} softcap={w.softcap} "
        f"K/V={w.k_dtype}/{w.v_dtype} rope={w.rope.scaling} sink={w.sink} paged={block_size} "
        f"fused={fused}")
    inputs = W.make_inputs(w)
    paged = W.make_paged(inputs, block_size) if block_size else None
    st = run_gpu(inputs, paged=paged, fused=fused)
    ref = OracleStep(inputs, copy_cache=False)  # inputs are on the device already
    rng = np.random.default_rng(99)
    H = w.n_heads
    pairs = []
    for b in range(w.batch):
        hs = rng.choice(H, size=min(H, 4 if w.batch > 1 else H), replace=False)
        pairs += [(b, int(h)) for h in hs]
    out = st.out.cpu().numpy()
    want = ref.decode(pairs)
    got = np.stack([out[b, h] for b, h in pairs])
    tol, cls = out_tolerance(w, want)
    err = float(np.max(np.abs(got - want)))
    check_slot(w, st.cache_rows(), ref.slot_rows(), st.q_out.cpu().numpy(), ref.q)
    sel = {b: [h for bb, h in pairs if bb == b][:2] for b in range(w.batch)}
    compare_partials(st, ref, w, inputs.seq_lens, pick=lambda b: sel[b])
    assert np.all(np.isfinite(out))
    say(f"  sampled {len(pairs)} outputs: max abs err {err:.3g} (tol {tol:.3g}, {cls})")
    assert err <= tol
    return err
