"""Pins of the CPU oracle: facts the oracle must reproduce that do not come
from the oracle itself -- closed forms, invariants, special cases that reduce
to a textbook result, values the pages state, and brute force on tiny inputs.

Every pin is a function ``pin_*(o)`` taking a loaded ``oracle.Oracle`` and
raising AssertionError on a mismatch.  ``test_oracle_pins.py`` runs them on
the oracle; ``test_oracle_teeth.py`` runs them on deliberately broken copies
of the oracle and requires each copy to fail at least one pin.

Page citations name the page title and section:
  UAII      "Universal AI Inference - Hugging Face decoder completeness"
  ALGENTA   "Algenta - Model support matrix"
  FREETOKEN "FreeToken PR #722 - serve Llama and Mistral llama-arch GGUF"
  LLAMAY    "llamay - Models and formats"
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(*seed):
    return np.random.default_rng(list(seed))


# ---------------------------------------------------------------------------
# RMSNorm  (UAII P1.1 Gemma RMSNorm (1+w); P1.2 Qwen3 QK-norm)
# ---------------------------------------------------------------------------

def pin_rms_norm_constant_vector(o):
    """x = c * 1 has mean square c^2, so y_i = c / sqrt(c^2 + eps) * (w_i + offset)."""
    d, eps = 64, 1e-6
    w = _rng(11).standard_normal(d).astype(np.float32)
    for c in (0.5, -3.0, 1e-3):
        for off in (0, 1):
            y = o.rms_norm(np.full(d, c), w, off, eps)
            want = c / math.sqrt(c * c + eps) * (w.astype(np.float64) + off)
            assert np.allclose(y, want, rtol=1e-14, atol=0), (c, off)


def pin_rms_norm_hand_row(o):
    """One hand-computed row per offset (UAII P1.1 asks for exactly this check):
    x = (3, 4): mean square 12.5; with eps = 0.5, r = 1/sqrt(13) exactly."""
    x = np.array([3.0, 4.0])
    w = np.array([1.0, 2.0], dtype=np.float32)
    r = 1.0 / math.sqrt(13.0)
    y0 = o.rms_norm(x, w, 0, 0.5)
    y1 = o.rms_norm(x, w, 1, 0.5)
    assert np.allclose(y0, [3 * r, 8 * r], rtol=1e-15, atol=0), y0
    assert np.allclose(y1, [6 * r, 12 * r], rtol=1e-15, atol=0), y1


def pin_rms_norm_offset_identity(o):
    """Gain (1 + w) with offset 1 equals gain w' = 1 + w with offset 0 (w on a
    1/256 grid, so 1 + w is exact in f32 and the two agree to rounding)."""
    d = 128
    x = _rng(12).standard_normal(d)
    w = (_rng(13).integers(-64, 64, d) / 256.0).astype(np.float32)
    a = o.rms_norm(x, w, 1, 1e-6)
    b = o.rms_norm(x, (1.0 + w).astype(np.float32), 0, 1e-6)
    assert np.allclose(a, b, rtol=1e-15, atol=0)
    c = o.rms_norm(x, w, 0, 1e-6)
    assert not np.allclose(a, c, rtol=1e-3)


def pin_rms_norm_unit_rms(o):
    """With w = 1, offset 0 and tiny eps the output has unit root-mean-square
    and is a positive multiple of x (scale invariance)."""
    d = 256
    x = 7.0 * _rng(14).standard_normal(d)
    y = o.rms_norm(x, np.ones(d, np.float32), 0, 1e-12)
    assert abs(math.sqrt(np.mean(y * y)) - 1.0) < 1e-12
    y2 = o.rms_norm(3.0 * x, np.ones(d, np.float32), 0, 1e-12)
    assert np.allclose(y, y2, rtol=1e-11, atol=0)


# ---------------------------------------------------------------------------
# RoPE frequencies  (UAII P0.2 RoPE scaling; FREETOKEN Changes and Results)
# ---------------------------------------------------------------------------

def pin_freqs_plain_geometric(o):
    """Plain frequencies theta^(-2i/d): g_0 = 1 and a constant ratio
    theta^(-2/d) between neighbours, i.e. g_i = exp(-2i ln(theta) / d)."""
    for d, theta in ((64, 1e4), (128, 5e5), (256, 1e6)):
        g = o.rope_freqs(d, O.PLAIN, theta)
        assert g[0] == 1.0
        i = np.arange(d // 2)
        assert np.allclose(g, np.exp(-2.0 * i * math.log(theta) / d), rtol=1e-13, atol=0)


def pin_freqs_llama31_first8(o):
    """'First 8 RoPE frequencies ... for Llama-3.1 8B config' (UAII P0.2 Tests):
    the eight highest frequencies lie in the unscaled band, so with llama3
    scaling (factor 8, low 1, high 4, original 8192) they equal the plain
    theta^(-i/64), theta = 5e5."""
    g = o.rope_freqs(128, O.LLAMA3, 5e5, 8.0, 1.0, 4.0, 8192)
    plain = np.exp(-np.arange(8) * math.log(5e5) / 64.0)
    assert np.allclose(g[:8], plain, rtol=1e-13, atol=0), g[:8]


def pin_freqs_llama3_recovered_factor(o):
    """FREETOKEN Changes/Results: the llama3 factor is the largest rope_freqs
    divisor f_i / g_i; it equals 32 for Llama-3.2-1B (d 64) and 8 for
    Llama-3.1-8B (d 128), both theta 5e5, low 1, high 4, original 8192.  The
    smallest divisor is 1 and the divisors never decrease with i."""
    for case in _golden("llama3_rope_factors.json")["cases"]:
        d, theta, factor = case["head_dim"], case["theta"], case["factor"]
        f = o.rope_freqs(d, O.PLAIN, theta)
        g = o.rope_freqs(d, O.LLAMA3, theta, factor, case["low"], case["high"], case["original"])
        div = f / g
        assert abs(div.max() - case["recovered_factor"]) < 1e-12, (case, div.max())
        assert abs(div.min() - 1.0) < 1e-15
        assert np.all(np.diff(div) >= -1e-12)


def pin_freqs_llama3_bands(o):
    """Band membership by wavelength lambda = 2 pi / f: below original/high the
    frequency is kept, above original/low it is divided by factor, between the
    two the divisor lies strictly inside (1, factor)."""
    for d, factor in ((64, 32.0), (128, 8.0), (256, 16.0)):
        f = o.rope_freqs(d, O.PLAIN, 5e5)
        g = o.rope_freqs(d, O.LLAMA3, 5e5, factor, 1.0, 4.0, 8192)
        lam = 2 * math.pi / f
        keep, scaled = lam < 8192 / 4.0, lam > 8192 / 1.0
        assert np.array_equal(g[keep], f[keep])
        assert np.allclose(g[scaled], f[scaled] / factor, rtol=1e-15, atol=0)
        mid = ~(keep | scaled)
        assert mid.any()
        assert np.all((f[mid] / g[mid] > 1.0) & (f[mid] / g[mid] < factor))


def pin_freqs_llama3_continuous(o):
    """The scaled frequency is continuous in the wavelength: on a dense grid of
    frequencies (huge head_dim, plain step r = theta^(2/d) - 1 ~ 4e-4)
    neighbouring divisors differ by O(r) (the smooth band's slope is bounded by
    a few r at factor 8), with no jump at either band edge."""
    d = 1 << 16
    f = o.rope_freqs(d, O.PLAIN, 5e5)
    g = o.rope_freqs(d, O.LLAMA3, 5e5, 8.0, 1.0, 4.0, 8192)
    div = f / g
    step = f[0] / f[1]
    assert np.all(div[1:] / div[:-1] <= 1.0 + 20.0 * (step - 1.0))
    assert np.all(div[1:] / div[:-1] >= 1.0 - 1e-12)


def pin_freqs_llama3_smooth_band_golden(o):
    """The divisors inside the smooth band for the two Llama shapes
    (tests/golden/llama3_smooth_band.json: FREETOKEN Changes/Results for the
    parameters, UAII P0.2 for Hugging Face's formulation), and which pair
    indices are kept, blended and divided."""
    for case in _golden("llama3_smooth_band.json")["cases"]:
        d, theta, factor = case["head_dim"], case["theta"], case["factor"]
        f = o.rope_freqs(d, O.PLAIN, theta)
        g = o.rope_freqs(d, O.LLAMA3, theta, factor, case["low"], case["high"], case["original"])
        div = f / g
        k0, k1 = case["kept"]
        s0, s1 = case["smooth"]
        c0, c1 = case["scaled"]
        assert np.all(div[k0:k1 + 1] == 1.0), case["model"]
        assert np.allclose(div[c0:c1 + 1], factor, rtol=1e-15, atol=0), case["model"]
        got = div[s0:s1 + 1]
        assert got.size == len(case["smooth_divisors"])
        for x, s in zip(got, case["smooth_divisors"]):
            decimals = len(s.split(".")[1])
            assert abs(x - float(s)) <= 0.5 * 10.0 ** -decimals * (1 + 1e-9), (case["model"], x, s)


def pin_freqs_llama3_blend_affine_in_frequency(o):
    """Inside the smooth band the frequency is a blend g = (1 - mu) f / factor
    + mu f.  Recovering mu = (g - f/factor) / (f - f/factor) on a dense grid of
    frequencies (huge head_dim), mu must be an affine function of f: it is a
    ramp in orig / wavelength = orig f / (2 pi), not in the wavelength and
    not a curve.  The line must reach 0 at the low-frequency edge (wavelength
    orig/low) and 1 at the high-frequency edge (wavelength orig/high), for
    several factors and band parameters."""
    for d, theta, factor, low, high, orig in ((1 << 16, 5e5, 8.0, 1.0, 4.0, 8192.0),
                                             (1 << 15, 5e5, 32.0, 1.0, 4.0, 8192.0),
                                             (1 << 15, 1e6, 4.0, 2.0, 8.0, 4096.0)):
        f = o.rope_freqs(d, O.PLAIN, theta)
        g = o.rope_freqs(d, O.LLAMA3, theta, factor, low, high, orig)
        lam = 2 * math.pi / f
        mid = (lam > orig / high) & (lam < orig / low)
        assert mid.sum() > 100
        fm = f[mid]
        mu = (g[mid] - fm / factor) / (fm - fm / factor)
        A = np.stack([fm, np.ones_like(fm)], axis=1)
        coef, *_ = np.linalg.lstsq(A, mu, rcond=None)
        assert np.max(np.abs(A @ coef - mu)) < 1e-9, (factor, np.max(np.abs(A @ coef - mu)))
        f_low_edge = 2 * math.pi * low / orig
        f_high_edge = 2 * math.pi * high / orig
        assert abs(coef[0] * f_low_edge + coef[1]) < 1e-9
        assert abs(coef[0] * f_high_edge + coef[1] - 1.0) < 1e-9


def pin_freqs_llama3_factor_one(o):
    """factor = 1 reduces llama3 scaling to plain frequencies."""
    f = o.rope_freqs(128, O.PLAIN, 5e5)
    g = o.rope_freqs(128, O.LLAMA3, 5e5, 1.0, 1.0, 4.0, 8192)
    assert np.allclose(f, g, rtol=1e-15, atol=0)


def pin_freqs_linear(o):
    """Linear scaling divides every frequency by the factor (ALGENTA Decoder
    families: gemma3 linear global scaling; UAII P0.2): g_i * factor equals
    exp(-2i ln(theta) / d), and the rotation angle at position p is that of
    plain RoPE at position p / factor.  Factor 1 is plain RoPE; and when
    every wavelength is past original/low, llama3 scaling degenerates to the
    same division, so the two branches agree there."""
    for d, theta, factor in ((64, 1e4, 2.0), (128, 1e6, 8.0), (256, 1e6, 40.0)):
        g = o.rope_freqs(d, O.LINEAR, theta, factor)
        i = np.arange(d // 2)
        assert np.allclose(g * factor, np.exp(-2.0 * i * math.log(theta) / d), rtol=1e-13,
                           atol=0)
        one = o.rope_freqs(d, O.LINEAR, theta, 1.0)
        assert np.array_equal(one, o.rope_freqs(d, O.PLAIN, theta))
        # llama3 with a tiny original context: every lambda > orig / low.
        l3 = o.rope_freqs(d, O.LLAMA3, theta, factor, 1.0, 4.0, 1e-3)
        assert np.array_equal(l3, g)
        x = _rng(17, d).standard_normal(d)
        p = 37
        y = o.rope_apply(x, O.NEOX, g, p)
        # plain rotation by angle (p / factor) * f_i written out
        z = x.copy()
        t = (p / factor) * np.exp(-2.0 * i * math.log(theta) / d)
        h = d // 2
        z[:h] = x[:h] * np.cos(t) - x[h:] * np.sin(t)
        z[h:] = x[:h] * np.sin(t) + x[h:] * np.cos(t)
        assert np.allclose(y, z, rtol=1e-12, atol=1e-13)


def _turns(d, theta, orig):
    """Turns each rotary pair makes over the original context: orig / wavelength."""
    f = np.exp(-2.0 * np.arange(d // 2) * math.log(theta) / d)
    return f, orig * f / (2.0 * math.pi)


YARN_CASES = (  # (d, theta, factor, beta_slow, beta_fast, original context)
    (64, 150000.0, 32.0, 1.0, 32.0, 4096),     # gpt-oss (LLAMAY Architectures)
    (128, 10000.0, 16.0, 1.0, 32.0, 4096),
    (256, 1e6, 4.0, 2.0, 64.0, 32768),
)


def pin_freqs_yarn_bands_by_turns(o):
    """YaRN keeps the frequency of every pair that turns at least beta_fast
    times over the original context and divides by the factor every pair that
    turns at most beta_slow times; the pairs between are blended, with a
    divisor strictly inside (1, factor).  Integer pair indices make this hold
    with and without rounding of the band edges."""
    for d, theta, factor, a, b, orig in YARN_CASES:
        f, turns = _turns(d, theta, orig)
        for trunc in (False, True):
            g = o.rope_freqs(d, O.YARN, theta, factor, a, b, orig, trunc)
            keep, scaled = turns >= b, turns <= a
            assert np.allclose(g[keep], f[keep], rtol=1e-14, atol=0), (d, trunc)
            assert np.allclose(g[scaled], f[scaled] / factor, rtol=1e-14, atol=0), (d, trunc)
            mid = ~(keep | scaled)
            assert mid.sum() >= 2
            div = f[mid] / g[mid]
            assert np.all((div > 1.0 + 1e-9) & (div < factor - 1e-9)), (d, trunc)


def pin_freqs_yarn_ramp_in_index(o):
    """Between the band edges the weight t of the divided frequency,
    g = (1 - t) f + t f / factor, is affine in the pair index (constant first
    differences); with rounded edges t steps by 1 / (whole number of pairs)."""
    for d, theta, factor, a, b, orig in YARN_CASES:
        f, turns = _turns(d, theta, orig)
        for trunc in (False, True):
            g = o.rope_freqs(d, O.YARN, theta, factor, a, b, orig, trunc)
            t = (1.0 - g / f) / (1.0 - 1.0 / factor)
            inside = np.nonzero((t > 1e-12) & (t < 1.0 - 1e-12))[0]
            assert np.array_equal(inside, np.arange(inside[0], inside[-1] + 1))
            step = np.diff(t[inside])
            assert np.allclose(step, step[0], rtol=1e-9, atol=1e-13), (d, trunc)
            if trunc:
                n = 1.0 / step[0]
                assert abs(n - round(n)) < 1e-9, (d, n)
                # first blended pair sits one step above 0
                assert abs(t[inside[0]] - step[0]) < 1e-12


def pin_yarn_factor_one_and_attention_factor(o):
    """Factor 1 gives plain frequencies and attention factor 1; the attention
    factor is 1 + 0.1 ln(factor) (gpt-oss, factor 32: 1.3465735902799727),
    and at position 0 (no rotation) the producer scales q and k by it."""
    d = 64
    assert np.allclose(o.rope_freqs(d, O.YARN, 150000.0, 1.0, 1.0, 32.0, 4096, False),
                       o.rope_freqs(d, O.PLAIN, 150000.0), rtol=1e-15, atol=0)
    assert o.yarn_attn_factor(1.0) == 1.0
    assert abs(o.yarn_attn_factor(32.0) - 1.3465735902799727) < 1e-15
    rng = _rng(78)
    qi = rng.standard_normal((1, 2, d)).astype(np.float32)
    ki = rng.standard_normal((1, 1, d)).astype(np.float32)
    ck = np.zeros((1, 1, 4, d), np.float32)
    cv = np.zeros((1, 1, 4, d), np.float32)
    rope = dict(pairing=O.NEOX, scaling=O.YARN, theta=150000.0, factor=32.0, low=1.0,
                high=32.0, orig=4096.0, truncate=False)
    qo = o.kv_produce(rope=rope, norm=None, q_in=qi, k_in=ki, v_in=ki,
                      positions=np.array([0], np.int32), k_dtype=O.F32, v_dtype=O.F32,
                      cache_k=ck, cache_v=cv)
    m = 1.0 + 0.1 * math.log(32.0)
    assert np.allclose(qo[0], qi[0].astype(np.float64) * m, rtol=1e-15, atol=0)
    assert np.array_equal(ck[0, 0, 0], (ki[0, 0].astype(np.float64) * m).astype(np.float32))
    assert np.array_equal(cv[0, 0, 0], ki[0, 0])      # values are not rotated or scaled
    # an explicit attention factor replaces the default
    qo2 = o.kv_produce(rope=dict(rope, attn_factor=2.0), norm=None, q_in=qi, k_in=ki, v_in=ki,
                       positions=np.array([0], np.int32), k_dtype=O.F32, v_dtype=O.F32,
                       cache_k=ck, cache_v=cv)
    assert np.allclose(qo2[0], 2.0 * qi[0].astype(np.float64), rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# RoPE rotation  (UAII P0.2; LLAMAY Architectures; FREETOKEN Changes)
# ---------------------------------------------------------------------------

def pin_rope_unit_vectors(o):
    """Closed forms with unit vectors: with d = 4 the frequencies are (1, theta^-1/2).
    NeoX pairs (0, 2), (1, 3); interleaved pairs (0, 1), (2, 3).  The first
    unit vector turns by angle p toward its partner: e_a -> cos p e_a + sin p e_b
    (the rotation direction is a convention, fixed here by construction)."""
    g = o.rope_freqs(4, O.PLAIN, 100.0)
    assert np.allclose(g, [1.0, 0.1], rtol=1e-15, atol=0)
    p = 3
    c, s = math.cos(p), math.sin(p)
    e0 = np.array([1.0, 0, 0, 0])
    assert np.allclose(o.rope_apply(e0, O.NEOX, g, p), [c, 0, s, 0], atol=1e-15)
    assert np.allclose(o.rope_apply(e0, O.INTERLEAVED, g, p), [c, s, 0, 0], atol=1e-15)
    e3 = np.array([0, 0, 0, 1.0])
    c1, s1 = math.cos(0.1 * p), math.sin(0.1 * p)
    assert np.allclose(o.rope_apply(e3, O.NEOX, g, p), [0, -s1, 0, c1], atol=1e-15)
    assert np.allclose(o.rope_apply(e3, O.INTERLEAVED, g, p), [0, 0, -s1, c1], atol=1e-15)


def pin_rope_identity_at_zero(o):
    x = _rng(21).standard_normal(128)
    g = o.rope_freqs(128, O.LLAMA3, 5e5, 8.0, 1.0, 4.0, 8192)
    for pairing in (O.NEOX, O.INTERLEAVED):
        assert np.array_equal(o.rope_apply(x, pairing, g, 0), x)


def _pairs(d, pairing):
    if pairing == O.NEOX:
        return [(i, i + d // 2) for i in range(d // 2)]
    return [(2 * i, 2 * i + 1) for i in range(d // 2)]


def pin_rope_pair_norms(o):
    """Each rotated pair keeps its Euclidean norm."""
    d = 64
    x = _rng(22).standard_normal(d)
    g = o.rope_freqs(d, O.PLAIN, 1e4)
    for pairing in (O.NEOX, O.INTERLEAVED):
        y = o.rope_apply(x, pairing, g, 4097)
        for a, b in _pairs(d, pairing):
            assert abs(math.hypot(y[a], y[b]) - math.hypot(x[a], x[b])) < 1e-13


def pin_rope_relative_position(o):
    """q.k after rotation depends only on the position difference."""
    d = 128
    q, k = _rng(23).standard_normal((2, d))
    g = o.rope_freqs(d, O.LLAMA3, 5e5, 8.0, 1.0, 4.0, 8192)
    for pairing in (O.NEOX, O.INTERLEAVED):
        a = o.rope_apply(q, pairing, g, 100) @ o.rope_apply(k, pairing, g, 37)
        b = o.rope_apply(q, pairing, g, 100 + 5000) @ o.rope_apply(k, pairing, g, 37 + 5000)
        assert abs(a - b) < 1e-10 * max(1.0, abs(a)), (a, b)


def pin_rope_group_law(o):
    """Rotating by p1 then p2 equals rotating by p1 + p2."""
    d = 64
    x = _rng(24).standard_normal(d)
    g = o.rope_freqs(d, O.PLAIN, 1e4)
    for pairing in (O.NEOX, O.INTERLEAVED):
        y = o.rope_apply(o.rope_apply(x, pairing, g, 123), pairing, g, 456)
        assert np.allclose(y, o.rope_apply(x, pairing, g, 579), atol=1e-11)


def pin_rope_neox_interleaved_permutation(o):
    """FREETOKEN Changes: interleaved rotary equals NeoX rotary up to a
    permutation of each head's rows.  With pi mapping NeoX index i -> 2i and
    i + d/2 -> 2i + 1: RoPE_interleaved(pi x) = pi RoPE_neox(x)."""
    d = 128
    x = _rng(25).standard_normal(d)
    g = o.rope_freqs(d, O.LLAMA3, 5e5, 8.0, 1.0, 4.0, 8192)
    perm = np.empty(d, dtype=np.int64)
    for i in range(d // 2):
        perm[2 * i], perm[2 * i + 1] = i, i + d // 2   # (pi x)[2i] = x[i]
    for p in (1, 777, 8191):
        a = o.rope_apply(x[perm], O.INTERLEAVED, g, p)
        b = o.rope_apply(x, O.NEOX, g, p)[perm]
        assert np.allclose(a, b, atol=1e-14), p


# ---------------------------------------------------------------------------
# Storage codecs  (UAII P0.1 BF16; LLAMAY The KV cache, in three precisions)
# ---------------------------------------------------------------------------

def pin_bf16_crafted(o):
    """Round to nearest, ties to even (values from tests/golden/bf16_rounding.json)."""
    for case in _golden("bf16_rounding.json")["cases"]:
        x = float.fromhex(case["x"])
        got = o.bf16_from_double(x)
        assert got == int(case["bits"], 16), (case, hex(got))


def pin_bf16_roundtrip_exhaustive(o):
    """Every non-NaN bf16 pattern decodes to a value that re-encodes to itself."""
    enc, dec = o.lib.oracle_bf16_from_double, o.lib.oracle_bf16_to_double
    for bits in range(0, 1 << 16, 1):
        if (bits & 0x7F80) == 0x7F80 and (bits & 0x7F):
            continue  # NaN payloads
        assert enc(dec(bits)) == bits, hex(bits)


def pin_bf16_nearest_brute_force(o):
    """Random doubles: the encoded value is at least as close as its two
    neighbours (brute force over the adjacent bf16 patterns)."""
    xs = _rng(31).standard_normal(3000) * np.exp2(_rng(32).integers(-130, 120, 3000))
    for x in xs:
        bits = o.bf16_from_double(x)
        v = o.bf16_to_double(bits)
        for nb in (bits - 1, bits + 1):
            if (nb & 0x7FFF) >= 0x7F80 or nb < 0 or nb > 0xFFFF:
                continue
            if (nb ^ bits) & 0x8000:
                continue
            assert abs(x - v) <= abs(x - o.bf16_to_double(nb)), (x, hex(bits))


def pin_quantizer_crafted(o):
    """vq8 quantiser: absmax 127 makes the scale exactly 1.0f, so codes are the
    values rounded half away from zero (tests/golden/vq8_quantizer.json)."""
    for case in _golden("vq8_quantizer.json")["cases"]:
        v = np.array(case["v"], dtype=np.float32)
        codes, scale = o.quantize_v(v)
        assert scale == np.float32(case["scale"]), (case, scale)
        assert codes.tolist() == case["codes"], (case, codes.tolist())


def pin_quantizer_near_ties(o):
    """vq8 quantiser at non-power-of-two scales, with values next to a
    half-way point (k + 1/2) * scale (tests/golden/vq8_near_ties.json, from
    exact rational arithmetic in make_vq8_near_ties.py).  Each vector holds
    values whose code changes if the quotient is taken as v * (1/scale)
    instead of the f32 division v / scale, and values whose f32 quotient is
    exactly a half-way point although the exact quotient is not, so that a
    quotient kept in double precision would round the other way."""
    doc = _golden("vq8_near_ties.json")
    n_recip = n_double = 0
    for case in doc["cases"]:
        v = np.array(case["v"], dtype=np.float32)
        codes, scale = o.quantize_v(v)
        assert scale == np.float32(case["scale"]), (scale, case["scale"])
        assert codes.tolist() == case["codes"], (codes.tolist(), case["codes"])
        n_recip += case["n_recip_sensitive"]
        n_double += case["n_double_sensitive"]
    assert n_recip >= 10 and n_double >= 5


def pin_quantizer_properties(o):
    """Zero vector -> scale 0 and codes 0; the absmax element maps to +-127;
    |code| <= 127; |v - code * scale| <= scale / 2 (plus one f32 rounding);
    scale is the IEEE f32 quotient absmax / 127."""
    codes, scale = o.quantize_v(np.zeros(64, np.float32))
    assert scale == 0.0 and not codes.any()
    rng = _rng(33)
    for t in range(300):
        d = (64, 128, 256)[t % 3]
        v = (rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        codes, scale = o.quantize_v(v)
        a = np.max(np.abs(v))
        assert scale == np.float32(a) / np.float32(127.0)
        assert np.all(np.abs(codes.astype(np.int32)) <= 127)
        assert abs(int(codes[np.argmax(np.abs(v))])) == 127
        err = np.abs(v.astype(np.float64) - codes.astype(np.float64) * np.float64(scale))
        assert np.all(err <= np.float64(scale) * 0.5 * (1 + 2.0 ** -21)), err.max() / scale


# ---------------------------------------------------------------------------
# Attention  (ALGENTA Structural fact requirements: GQA ratio, scale
# 1/sqrt(head_dim); UAII P1.4 sliding window, logit softcap)
# ---------------------------------------------------------------------------

def _cache(B, Hkv, cap, d, seed, kdt=O.F32, vdt=O.F32):
    rng = _rng(seed)
    K = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    return K, V


def pin_attention_zero_query_window(o):
    """q = 0 gives uniform weights, so the output is the mean of the visible
    values.  With position-coded values (v_j[0] = j) that mean is
    (lo + L - 1) / 2, which fixes where the window starts: a window of W keys
    counts the new key, lo = max(0, L - W)."""
    B, H, Hkv, d, cap = 3, 4, 2, 64, 40
    K, _ = _cache(B, Hkv, cap, d, 41)
    V = np.zeros((B, Hkv, cap, d), np.float32)
    V[..., 0] = np.arange(cap, dtype=np.float32)
    V[..., 1] = 1.0
    q = np.zeros((B, H, d))
    lens = np.array([40, 17, 1], np.int32)
    for W in (0, 1, 2, 7, 16, 17, 39, 40, 45):
        out = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                       seq_lens=lens, window=W)
        for b, L in enumerate(lens):
            lo = L - W if (W > 0 and L > W) else 0
            assert np.allclose(out[b, :, 0], (lo + L - 1) / 2.0, rtol=1e-14, atol=1e-14), (W, L)
            assert np.allclose(out[b, :, 1], 1.0, rtol=1e-14)


def pin_attention_constant_values(o):
    """Constant values give that constant, with any window or softcap."""
    B, H, Hkv, d, cap = 2, 8, 2, 64, 50
    K, _ = _cache(B, Hkv, cap, d, 42)
    c = _rng(43).standard_normal(d).astype(np.float32)
    V = np.broadcast_to(c, (B, Hkv, cap, d)).copy()
    q = 3.0 * _rng(44).standard_normal((B, H, d))
    for W, cap_ in ((0, 0.0), (5, 0.0), (0, 2.0), (9, 50.0)):
        out = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                       seq_lens=np.array([50, 23], np.int32), window=W, softcap=cap_)
        assert np.allclose(out, np.broadcast_to(c, out.shape), rtol=1e-13, atol=1e-14)


def pin_attention_two_keys_logistic(o):
    """Two keys: the weights are the logistic function of the score gap.
    q = a e_0, k_0 = x e_0, k_1 = 0 give scores a x / sqrt(d) and 0."""
    d = 64
    K = np.zeros((1, 1, 2, d), np.float32)
    V = np.zeros((1, 1, 2, d), np.float32)
    K[0, 0, 0, 0] = 1.5
    V[0, 0, 0, :] = 2.0
    V[0, 0, 1, :] = -1.0
    for a in (0.0, 1.0, -4.0, 10.0):
        q = np.zeros((1, 1, d))
        q[0, 0, 0] = a
        s = a * 1.5 / math.sqrt(d)
        w0 = 1.0 / (1.0 + math.exp(-s))
        out = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                       seq_lens=np.array([2], np.int32))
        assert np.allclose(out[0, 0], 2.0 * w0 - (1.0 - w0), rtol=1e-14, atol=1e-15), a


def pin_attention_window_limits(o):
    """A window of at least L keys equals full attention; a window of 1 key
    returns the newest value."""
    B, H, Hkv, d, cap = 2, 4, 4, 64, 33
    K, V = _cache(B, Hkv, cap, d, 45)
    q = _rng(46).standard_normal((B, H, d))
    lens = np.array([33, 12], np.int32)
    full = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens)
    for W in (33, 34, 1000):
        w = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                     window=W)
        assert np.array_equal(w, full)
    one = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                   window=1)
    for b, L in enumerate(lens):
        for h in range(H):
            assert np.allclose(one[b, h], V[b, h, L - 1], rtol=1e-15, atol=0)


def pin_attention_softcap(o):
    """Capped scores equal c * tanh(s / c) of the uncapped ones; a huge cap
    leaves the scores unchanged to O(s^3 / c^2); the argmax is unchanged.
    Query head 1 of 4 over 2 kv heads reads kv head 0 (consecutive groups)."""
    H, Hkv, d, cap = 4, 2, 64, 30
    K, _ = _cache(1, Hkv, cap, d, 47)
    K[0, 1] = 0.0
    q = 6.0 * _rng(48).standard_normal(d)
    s0 = o.scores(q=q, cache_k=K, k_dtype=O.F32, n_heads=H, b=0, h=1, L=30)
    assert np.allclose(s0, K[0, 0, :30].astype(np.float64) @ q / 8.0, rtol=1e-12, atol=1e-13)
    for c in (0.5, 5.0, 50.0):
        sc = o.scores(q=q, cache_k=K, k_dtype=O.F32, n_heads=H, b=0, h=1, L=30, softcap=c)
        assert np.allclose(sc, c * np.tanh(s0 / c), rtol=1e-14, atol=1e-15)
        assert np.all(np.abs(sc) <= c)
        assert np.argmax(sc) == np.argmax(s0)
    big = o.scores(q=q, cache_k=K, k_dtype=O.F32, n_heads=H, b=0, h=1, L=30, softcap=1e6)
    assert np.all(np.abs(big - s0) <= np.abs(s0) ** 3 / 3e12 + 1e-12)
    win = o.scores(q=q, cache_k=K, k_dtype=O.F32, n_heads=H, b=0, h=1, L=30, window=4)
    assert np.all(win[:26] == -np.inf) and np.array_equal(win[26:], s0[26:])


def pin_attention_gqa_expansion(o):
    """GQA equals multi-head attention on keys and values repeated G times per
    kv head, with consecutive query heads sharing a kv head (h -> h // G);
    kv-head-constant values expose the map directly."""
    B, H, Hkv, d, cap = 2, 8, 2, 64, 20
    G = H // Hkv
    K, V = _cache(B, Hkv, cap, d, 49)
    q = _rng(50).standard_normal((B, H, d))
    lens = np.array([20, 9], np.int32)
    gqa = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens)
    Ke = np.ascontiguousarray(np.repeat(K, G, axis=1))
    Ve = np.ascontiguousarray(np.repeat(V, G, axis=1))
    mha = o.decode(q=q, cache_k=Ke, cache_v=Ve, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens)
    assert np.array_equal(gqa, mha)
    Vc = np.zeros_like(V)
    for u in range(Hkv):
        Vc[:, u] = u + 1
    out = o.decode(q=q, cache_k=K, cache_v=Vc, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens)
    for h in range(H):
        assert np.allclose(out[:, h], h // G + 1, rtol=1e-14)


def pin_attention_dominant_key(o):
    """q = alpha k_j with large alpha puts (almost) all weight on key j."""
    d = 128
    K, V = _cache(1, 1, 64, d, 51)
    j = 37
    q = (60.0 * K[0, 0, j] / np.linalg.norm(K[0, 0, j])).reshape(1, 1, d)
    out = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                   seq_lens=np.array([64], np.int32))
    assert np.allclose(out[0, 0], V[0, 0, j], atol=1e-6)


def pin_attention_brute_force(o):
    """Tiny shapes against a second formulation: long double, scores by
    explicit loops, no max subtraction, weights normalised at the end."""
    rng = _rng(52)
    for t in range(6):
        B, Hkv, G, d = 2, 2, (1, 2, 4)[t % 3], (64, 128)[t % 2]
        H, cap = Hkv * G, 24
        K = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
        V = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
        q = rng.standard_normal((B, H, d))
        lens = rng.integers(1, cap + 1, B).astype(np.int32)
        W = [0, 3, 30][t % 3]
        cap_c = [0.0, 0.0, 7.0][t % 3]
        out = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                       window=W, softcap=cap_c)
        for b in range(B):
            L = int(lens[b])
            for h in range(H):
                u = h // G
                num = np.zeros(d, dtype=np.longdouble)
                den = np.longdouble(0)
                for j in range(L):
                    if W > 0 and j < L - W:
                        continue
                    s = np.longdouble(0)
                    for i in range(d):
                        s += np.longdouble(q[b, h, i]) * np.longdouble(K[b, u, j, i])
                    s /= np.sqrt(np.longdouble(d))
                    if cap_c > 0:
                        s = np.longdouble(cap_c) * np.tanh(s / np.longdouble(cap_c))
                    e = np.exp(s)
                    den += e
                    num += e * V[b, u, j].astype(np.longdouble)
                ref = (num / den).astype(np.float64)
                assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13), (t, b, h)


def pin_attention_storage_formats(o):
    """bf16 caches give the same result as f32 caches holding the decoded
    bf16 values; vq8 values give the result of f32 values code * scale."""
    B, H, Hkv, d, cap = 2, 4, 2, 64, 30
    rng = _rng(53)
    Kf = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    Vf = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    Kb = (Kf.view(np.uint32) >> 16).astype(np.uint16)
    Vb = (Vf.view(np.uint32) >> 16).astype(np.uint16)
    Kbf = (Kb.astype(np.uint32) << 16).view(np.float32)
    Vbf = (Vb.astype(np.uint32) << 16).view(np.float32)
    q = rng.standard_normal((B, H, d))
    lens = np.array([30, 11], np.int32)
    a = o.decode(q=q, cache_k=Kb, cache_v=Vb, k_dtype=O.BF16, v_dtype=O.BF16, seq_lens=lens)
    b = o.decode(q=q, cache_k=Kbf, cache_v=Vbf, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens)
    assert np.array_equal(a, b)
    codes = rng.integers(-127, 128, (B, Hkv, cap, d)).astype(np.int8)
    scale = np.exp2(-rng.integers(4, 10, (B, Hkv, cap))).astype(np.float32)
    deq = codes.astype(np.float32) * scale[..., None]      # exact: power-of-two scales
    c = o.decode(q=q, cache_k=Kb, cache_v=codes, v_scale=scale, k_dtype=O.BF16, v_dtype=O.I8,
                 seq_lens=lens)
    e = o.decode(q=q, cache_k=Kb, cache_v=deq, k_dtype=O.BF16, v_dtype=O.F32, seq_lens=lens)
    assert np.array_equal(c, e)


def pin_attention_sink_zero_query(o):
    """Attention sink (LLAMAY Architectures: gpt-oss; a per-head logit in the
    softmax denominator only).  With q = 0 every visible score is 0, so the
    weights are 1 / (n + e^sink) for each of the n visible keys and the output
    is mean(v) * n / (n + e^sink); the sink itself contributes no value."""
    B, H, Hkv, d, cap = 2, 4, 2, 64, 40
    K, _ = _cache(B, Hkv, cap, d, 71)
    V = np.zeros((B, Hkv, cap, d), np.float32)
    V[..., 0] = np.arange(cap, dtype=np.float32)
    V[..., 1] = 1.0
    q = np.zeros((B, H, d))
    lens = np.array([40, 9], np.int32)
    sinks = np.array([-3.0, 0.0, 1.5, 4.0])
    for W in (0, 5):
        out = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                       seq_lens=lens, window=W, sinks=sinks)
        for b, L in enumerate(lens):
            lo = L - W if (W > 0 and L > W) else 0
            n = L - lo
            for h in range(H):
                frac = n / (n + math.exp(sinks[h]))
                assert abs(out[b, h, 1] - frac) < 1e-14, (W, b, h)
                assert abs(out[b, h, 0] - frac * (lo + L - 1) / 2.0) < 1e-12, (W, b, h)


def pin_attention_sink_denominator(o):
    """With a sink the output is the sink-free output times Z / (Z + e^sink),
    Z = sum of e^s over the visible (capped) scores, computed here in long
    double from the scores; a very negative sink leaves the output unchanged."""
    B, H, Hkv, d, cap = 1, 4, 2, 64, 33
    K, V = _cache(B, Hkv, cap, d, 72)
    q = 2.0 * _rng(73).standard_normal((B, H, d))
    lens = np.array([33], np.int32)
    sinks = np.array([-1.0, 0.5, 2.0, 6.0])
    for W, c in ((0, 0.0), (12, 0.0), (0, 3.0)):
        base = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                        window=W, softcap=c)
        out = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                       window=W, softcap=c, sinks=sinks)
        gone = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                        window=W, softcap=c, sinks=np.full(H, -1e4))
        assert np.array_equal(gone, base)
        for h in range(H):
            s = o.scores(q=q[0, h], cache_k=K, k_dtype=O.F32, n_heads=H, b=0, h=h, L=33,
                         window=W, softcap=c)
            z = np.sum(np.exp(s[s > -np.inf].astype(np.longdouble)))
            ratio = float(z / (z + np.exp(np.longdouble(sinks[h]))))
            assert np.allclose(out[0, h], base[0, h] * ratio, rtol=1e-12, atol=1e-14), (W, c, h)


def pin_combine_sink(o):
    """The sink belongs to no split: combining the split partials with the
    sink in the combine's denominator equals single-pass attention with the
    sink, and equals a combine with one more split that has o = 0 and
    lse = sink."""
    H, Hkv, d, L = 4, 2, 64, 61
    K, V = _cache(1, Hkv, L, d, 74)
    q = 2.0 * _rng(75).standard_normal((1, H, d))
    sinks = np.array([0.0, 3.0, -2.0, 8.0])
    for W in (0, 20):
        single = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                          seq_lens=np.array([L], np.int32), window=W, sinks=sinks)
        for S in (7, 32, L):
            n = -(-L // S)
            for h in range(H):
                os_, ls = np.zeros((n, d)), np.zeros(n)
                for sg in range(n):
                    os_[sg], ls[sg], _ = o.split_partial(
                        q_bh=q[0, h], cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                        n_heads=H, b=0, h=h, L=L, window=W, softcap=0.0, split_size=S, sigma=sg)
                out, _ = o.combine(os_, ls, sink=sinks[h])
                assert np.allclose(out, single[0, h], rtol=1e-12, atol=1e-13), (W, S, h)
                ext, _ = o.combine(np.vstack([os_, np.zeros((1, d))]), np.append(ls, sinks[h]))
                assert np.allclose(out, ext, rtol=1e-13, atol=1e-15), (W, S, h)


def pin_q8_keys(o):
    """q8 (LLAMAY The KV cache, in three precisions: keys and values both
    quantised): int8 keys with a per-token scale score like f32 keys holding
    code * scale (power-of-two scales keep that product exact in f32)."""
    B, H, Hkv, d, cap = 2, 4, 2, 64, 30
    rng = _rng(76)
    kc = rng.integers(-127, 128, (B, Hkv, cap, d)).astype(np.int8)
    ks = np.exp2(-rng.integers(3, 9, (B, Hkv, cap))).astype(np.float32)
    vc = rng.integers(-127, 128, (B, Hkv, cap, d)).astype(np.int8)
    vs = np.exp2(-rng.integers(3, 9, (B, Hkv, cap))).astype(np.float32)
    kd = kc.astype(np.float32) * ks[..., None]
    vd = vc.astype(np.float32) * vs[..., None]
    q = 3.0 * rng.standard_normal((B, H, d))
    lens = np.array([30, 13], np.int32)
    for W, c in ((0, 0.0), (7, 0.0), (0, 4.0)):
        a = o.decode(q=q, cache_k=kc, k_scale=ks, cache_v=vc, v_scale=vs, k_dtype=O.I8,
                     v_dtype=O.I8, seq_lens=lens, window=W, softcap=c)
        b = o.decode(q=q, cache_k=kd, cache_v=vd, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                     window=W, softcap=c)
        assert np.array_equal(a, b), (W, c)
    s8 = o.scores(q=q[0, 1], cache_k=kc, k_scale=ks, k_dtype=O.I8, n_heads=H, b=0, h=1, L=30)
    sf = o.scores(q=q[0, 1], cache_k=kd, k_dtype=O.F32, n_heads=H, b=0, h=1, L=30)
    assert np.array_equal(s8, sf)


# ---------------------------------------------------------------------------
# Split-K flash decoding  (ALGENTA Kernel path capabilities: split-K decode
# partials; Conformance CLI: decode_attn=splitk_flash_decoding)
# ---------------------------------------------------------------------------

def pin_split_combine_equals_single_pass(o):
    """For any split size, combining the per-split partials with their
    log-sum-exp weights reproduces single-pass attention; empty splits
    (before the window) have lse = -inf and drop out."""
    H, Hkv, d, cap = 4, 2, 64, 77
    K, V = _cache(1, Hkv, cap, d, 54)
    q = 2.0 * _rng(55).standard_normal((1, H, d))
    L = 77
    for W, cap_c in ((0, 0.0), (20, 0.0), (0, 30.0), (33, 5.0)):
        single = o.decode(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                          seq_lens=np.array([L], np.int32), window=W, softcap=cap_c)
        for S in (1, 2, 3, 64, L - 1, L, 2 * L):
            for h in (0, 3):
                n = -(-L // S)
                os_, ls = np.zeros((n, d)), np.zeros(n)
                total = 0
                for sg in range(n):
                    os_[sg], ls[sg], k = o.split_partial(
                        q_bh=q[0, h], cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                        n_heads=H, b=0, h=h, L=L, window=W, softcap=cap_c, split_size=S,
                        sigma=sg)
                    total += k
                    assert (k == 0) == (ls[sg] == -math.inf)
                lo = L - W if (W > 0 and L > W) else 0
                assert total == L - lo
                out, used = o.combine(os_, ls)
                assert used == int(np.sum(ls > -math.inf))
                assert np.allclose(out, single[0, h], rtol=1e-12, atol=1e-13), (W, S, h)


def pin_split_partial_is_local_attention(o):
    """A split's partial is softmax attention over its own keys, and its lse
    is the log of the sum of e^s over those keys."""
    H, Hkv, d, cap = 2, 1, 64, 40
    K, V = _cache(1, Hkv, cap, d, 56)
    q = _rng(57).standard_normal(d)
    s = o.scores(q=q, cache_k=K, k_dtype=O.F32, n_heads=H, b=0, h=0, L=40)
    o1, lse, n = o.split_partial(q_bh=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                                 n_heads=H, b=0, h=0, L=40, window=0, softcap=0.0,
                                 split_size=16, sigma=1)
    assert n == 16
    assert abs(lse - math.log(np.sum(np.exp(s[16:32])))) < 1e-12
    w = np.exp(s[16:32] - lse)
    assert np.allclose(o1, w @ V[0, 0, 16:32].astype(np.float64), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Producer  (UAII P1.2: norm before RoPE; P1.3: absolute positions)
# ---------------------------------------------------------------------------

def pin_produce_writes_one_slot(o):
    """The producer writes exactly slot positions[b] of each (b, kv head)."""
    B, H, Hkv, d, cap = 3, 4, 2, 64, 16
    rng = _rng(61)
    qi, ki, vi = (rng.standard_normal(s).astype(np.float32)
                  for s in ((B, H, d), (B, Hkv, d), (B, Hkv, d)))
    pos = np.array([0, 7, 15], np.int32)
    for kdt, vdt in ((O.F32, O.F32), (O.BF16, O.BF16), (O.BF16, O.I8)):
        ck = np.full((B, Hkv, cap, d), 0x55, dtype={O.F32: np.float32, O.BF16: np.uint16}[kdt])
        cv = np.full((B, Hkv, cap, d), 0x55,
                     dtype={O.F32: np.float32, O.BF16: np.uint16, O.I8: np.int8}[vdt])
        vs = np.full((B, Hkv, cap), 7.0, np.float32)
        ck0, cv0, vs0 = ck.copy(), cv.copy(), vs.copy()
        o.kv_produce(rope=dict(pairing=O.NEOX, scaling=O.PLAIN, theta=1e4), norm=None,
                     q_in=qi, k_in=ki, v_in=vi, positions=pos, k_dtype=kdt, v_dtype=vdt,
                     cache_k=ck, cache_v=cv, v_scale=vs)
        mask = np.zeros((B, Hkv, cap), bool)
        for b in range(B):
            mask[b, :, pos[b]] = True
        assert np.array_equal(ck[~mask], ck0[~mask]) and np.array_equal(cv[~mask], cv0[~mask])
        assert np.array_equal(vs[~mask], vs0[~mask])
        assert not np.array_equal(ck[mask], ck0[mask])


def pin_produce_position_zero(o):
    """At position 0 RoPE is the identity: without QK-norm q' = q and the
    stored key and value are the inputs in the cache's format (f32 exact;
    vq8 codes and scale of the value quantiser)."""
    B, H, Hkv, d, cap = 2, 4, 2, 128, 4
    rng = _rng(62)
    qi = rng.standard_normal((B, H, d)).astype(np.float32)
    ki = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    vi = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    ck = np.zeros((B, Hkv, cap, d), np.float32)
    cv = np.zeros((B, Hkv, cap, d), np.int8)
    vs = np.zeros((B, Hkv, cap), np.float32)
    qo = o.kv_produce(rope=dict(pairing=O.INTERLEAVED, scaling=O.LLAMA3, theta=5e5, factor=8.0),
                      norm=None, q_in=qi, k_in=ki, v_in=vi, positions=np.zeros(B, np.int32),
                      k_dtype=O.F32, v_dtype=O.I8, cache_k=ck, cache_v=cv, v_scale=vs)
    assert np.array_equal(qo, qi.astype(np.float64))
    assert np.array_equal(ck[:, :, 0], ki)
    for b in range(B):
        for u in range(Hkv):
            c, s = o.quantize_v(vi[b, u])
            assert np.array_equal(cv[b, u, 0], c) and vs[b, u, 0] == s


def pin_produce_norm_before_rope(o):
    """The producer normalises, then rotates: with a non-uniform gain the two
    orders differ, and the output matches norm-then-rope."""
    d = 64
    rng = _rng(63)
    qi = rng.standard_normal((1, 1, d)).astype(np.float32)
    ki = rng.standard_normal((1, 1, d)).astype(np.float32)
    w = (1.0 + 0.5 * rng.standard_normal(d)).astype(np.float32)
    g = o.rope_freqs(d, O.PLAIN, 1e4)
    ck = np.zeros((1, 1, 8, d), np.float32)
    cv = np.zeros((1, 1, 8, d), np.float32)
    qo = o.kv_produce(rope=dict(pairing=O.NEOX, scaling=O.PLAIN, theta=1e4),
                      norm=dict(enabled=True, eps=1e-6, offset=0, w_q=w, w_k=w),
                      q_in=qi, k_in=ki, v_in=ki, positions=np.array([5], np.int32),
                      k_dtype=O.F32, v_dtype=O.F32, cache_k=ck, cache_v=cv)
    x = qi[0, 0].astype(np.float64)
    # Norm-then-rope written with numpy (unit rms, then gain, then rotation by
    # the oracle's own pieces is avoided: rotation here uses explicit pairs).
    r = 1.0 / math.sqrt(np.mean(x * x) + 1e-6)
    y = x * r * w
    z = y.copy()
    for i in range(d // 2):
        t = 5 * g[i]
        z[i] = y[i] * math.cos(t) - y[i + d // 2] * math.sin(t)
        z[i + d // 2] = y[i] * math.sin(t) + y[i + d // 2] * math.cos(t)
    assert np.allclose(qo[0, 0], z, rtol=1e-13, atol=1e-14)
    xr = o.rope_apply(x, O.NEOX, g, 5)
    other = xr / math.sqrt(np.mean(xr * xr) + 1e-6) * w
    assert not np.allclose(qo[0, 0], other, rtol=1e-6)


def pin_produce_q8_keys(o):
    """The q8 producer stores, for each key, the quantiser applied to the
    rotated key rounded to f32: the same codes and scale as quantising the
    row an f32-key producer writes for the same inputs."""
    B, H, Hkv, d, cap = 2, 4, 2, 64, 12
    rng = _rng(77)
    qi = rng.standard_normal((B, H, d)).astype(np.float32)
    ki = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    vi = rng.standard_normal((B, Hkv, d)).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    pos = np.array([5, 11], np.int32)
    rope = dict(pairing=O.INTERLEAVED, scaling=O.LLAMA3, theta=5e5, factor=8.0, low=1.0,
                high=4.0, orig=8192.0)
    norm = dict(enabled=True, eps=1e-6, offset=0, w_q=w, w_k=w)
    kf = np.zeros((B, Hkv, cap, d), np.float32)
    vf = np.zeros((B, Hkv, cap, d), np.float32)
    qa = o.kv_produce(rope=rope, norm=norm, q_in=qi, k_in=ki, v_in=vi, positions=pos,
                      k_dtype=O.F32, v_dtype=O.F32, cache_k=kf, cache_v=vf)
    k8 = np.zeros((B, Hkv, cap, d), np.int8)
    v8 = np.zeros((B, Hkv, cap, d), np.int8)
    ks = np.zeros((B, Hkv, cap), np.float32)
    vs = np.zeros((B, Hkv, cap), np.float32)
    qb = o.kv_produce(rope=rope, norm=norm, q_in=qi, k_in=ki, v_in=vi, positions=pos,
                      k_dtype=O.I8, v_dtype=O.I8, cache_k=k8, cache_v=v8, k_scale=ks,
                      v_scale=vs)
    assert np.array_equal(qa, qb)
    for b in range(B):
        for u in range(Hkv):
            codes, sc = o.quantize_v(kf[b, u, pos[b]])
            assert np.array_equal(k8[b, u, pos[b]], codes) and ks[b, u, pos[b]] == sc
            codes, sc = o.quantize_v(vi[b, u])
            assert np.array_equal(v8[b, u, pos[b]], codes) and vs[b, u, pos[b]] == sc
    assert np.count_nonzero(k8) == np.count_nonzero(k8[np.arange(B), :, pos])


# ---------------------------------------------------------------------------
# Chunks of new tokens (prefill): ALGENTA Kernel path capabilities (grouped-FA
# prefill); UAII P1.3 (positions follow the absolute KV index), P1.4 (window,
# softcap)
# ---------------------------------------------------------------------------

def _prefill_matrix(q, K, V, lens, T, G, window, softcap, sinks):
    """Causal attention of a chunk in matrix form (numpy, float64): one
    masked score matrix per (sequence, head), a row-wise softmax with the
    sink as an extra column carrying no value, then P V."""
    B, _, H, d = q.shape
    out = np.zeros(q.shape)
    for b in range(B):
        L = int(lens[b])
        pos = np.arange(L - T, L)
        lo = np.maximum(0, pos + 1 - window) if window > 0 else np.zeros(T, np.int64)
        j = np.arange(L)
        mask = (j[None, :] <= pos[:, None]) & (j[None, :] >= lo[:, None])
        for h in range(H):
            Kb = K[b, h // G, :L].astype(np.float64)
            Vb = V[b, h // G, :L].astype(np.float64)
            S = q[b, :, h].astype(np.float64) @ Kb.T / math.sqrt(d)
            if softcap > 0:
                S = softcap * np.tanh(S / softcap)
            S = np.where(mask, S, -np.inf)
            if sinks is not None:
                S = np.concatenate([S, np.full((T, 1), float(sinks[h]))], axis=1)
                Vx = np.concatenate([Vb, np.zeros((1, d))], axis=0)
            else:
                Vx = Vb
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            out[b, :, h] = (P / P.sum(axis=1, keepdims=True)) @ Vx
    return out


def pin_prefill_matrix_form(o):
    """The chunk's causal attention equals the masked matrix form: query t of
    a chunk of T at the end of L keys sees keys lo_t .. L - T + t, for empty
    and non-empty caches, with window, softcap and sink."""
    B, T, H, Hkv, d, cap = 2, 5, 4, 2, 8, 12
    rng = _rng(91)
    K, V = _cache(B, Hkv, cap, d, 92)
    q = rng.standard_normal((B, T, H, d))
    lens = np.array([9, 5], np.int32)        # 4 cached tokens + 5; an empty cache + 5
    sinks = rng.standard_normal(H)
    for window in (0, 3, 1):
        for softcap in (0.0, 1.5):
            for sk in (None, sinks):
                got = o.prefill(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32,
                                seq_lens=lens, window=window, softcap=softcap, sinks=sk)
                want = _prefill_matrix(q, K, V, lens, T, H // Hkv, window, softcap, sk)
                assert np.allclose(got, want, rtol=0, atol=1e-12), (window, softcap, sk is None)


def pin_prefill_causal(o):
    """Query t never reads a key after its own position: poisoning every
    later cache row leaves its output unchanged (and finite)."""
    B, T, H, Hkv, d, cap = 1, 6, 2, 1, 16, 10
    rng = _rng(93)
    K, V = _cache(B, Hkv, cap, d, 94)
    q = rng.standard_normal((B, T, H, d))
    lens = np.array([10], np.int32)
    full = o.prefill(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens)
    for t in range(T):
        p = 10 - T + t
        Kp, Vp = K.copy(), V.copy()
        Kp[:, :, p + 1:] = np.nan
        Vp[:, :, p + 1:] = np.nan
        got = o.prefill(q=q, cache_k=Kp, cache_v=Vp, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                        triples=[(0, t, h) for h in range(H)])
        assert np.all(np.isfinite(got)) and np.array_equal(got, full[0, t]), t


def pin_prefill_last_token_is_decode(o):
    """The chunk's last query sees exactly what a decode step at L keys sees
    (it is the newest token), for any chunk length."""
    B, H, Hkv, d, cap = 2, 4, 2, 16, 20
    rng = _rng(95)
    K, V = _cache(B, Hkv, cap, d, 96)
    lens = np.array([20, 13], np.int32)
    for T in (1, 4, 13):
        q = rng.standard_normal((B, T, H, d))
        got = o.prefill(q=q, cache_k=K, cache_v=V, k_dtype=O.F32, v_dtype=O.F32, seq_lens=lens,
                        window=6, softcap=2.0)
        want = o.decode(q=np.ascontiguousarray(q[:, -1]), cache_k=K, cache_v=V, k_dtype=O.F32,
                        v_dtype=O.F32, seq_lens=lens, window=6, softcap=2.0)
        assert np.array_equal(got[:, -1], want), T


def pin_chunk_producer(o):
    """The chunk producer writes exactly the T slots start .. start + T - 1 of
    every (b, kv head), and its token t is the single-token producer at
    position start + t (here: with the tokens produced in reverse order)."""
    B, T, H, Hkv, d, cap = 2, 4, 4, 2, 32, 12
    rng = _rng(97)
    qi = rng.standard_normal((B, T, H, d)).astype(np.float32)
    ki = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    vi = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    start = np.array([0, 8], np.int32)
    rope = dict(pairing=O.INTERLEAVED, scaling=O.LLAMA3, theta=5e5, factor=8.0)
    ck = np.full((B, Hkv, cap, d), 0x5555, np.uint16)
    cv = np.full((B, Hkv, cap, d), 0x5555, np.uint16)
    q = o.kv_produce_chunk(rope=rope, norm=None, q_in=qi, k_in=ki, v_in=vi, start_positions=start,
                           k_dtype=O.BF16, v_dtype=O.BF16, cache_k=ck, cache_v=cv)
    written = np.zeros((B, Hkv, cap), bool)
    for b in range(B):
        written[b, :, start[b]:start[b] + T] = True
    assert np.all(ck[~written] == 0x5555) and np.all(cv[~written] == 0x5555)
    ck2 = np.full_like(ck, 0x5555)
    cv2 = np.full_like(cv, 0x5555)
    for t in reversed(range(T)):
        q2 = o.kv_produce(rope=rope, norm=None, q_in=np.ascontiguousarray(qi[:, t]),
                          k_in=np.ascontiguousarray(ki[:, t]), v_in=np.ascontiguousarray(vi[:, t]),
                          positions=start + t, k_dtype=O.BF16, v_dtype=O.BF16, cache_k=ck2,
                          cache_v=cv2)
        assert np.array_equal(q2, q[:, t]), t
    assert np.array_equal(ck, ck2) and np.array_equal(cv, cv2)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
