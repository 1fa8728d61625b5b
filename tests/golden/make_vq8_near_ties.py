"""Writes vq8_near_ties.json: quantiser inputs whose codes depend on the exact
order of IEEE f32 operations in the vq8 quantiser, with their codes.

The quantiser (the vq8 cache of 'llamay - Models and formats', The KV cache,
in three precisions; granularity, absmax scale and tie rule as read where the
page is silent) is a fixed sequence of f32 operations:
    scale = RNE32(a / 127),  t = RNE32(v / scale),  code = round_half_away(t),
clamped to +-127.  This script evaluates that sequence in exact rational
arithmetic (Python fractions, with an explicit round-to-nearest-even to the
f32 grid), so its codes come from neither the oracle nor the GPU path.

It searches, for non-power-of-two scales, values v next to a half-way point
(k + 1/2) * scale where a slightly different operation order would give
another code:
  * 'recip':  v * RNE32(1 / scale) rounds to the other side of k + 1/2;
  * 'double': the f32 quotient is exactly k + 1/2 although the exact
    quotient is not (a quotient kept in double would round the other way).
Each case is one vector holding its absmax element first, so the scale is
fixed, then near-tie values of both kinds.

Run:  python tests/golden/make_vq8_near_ties.py   (deterministic)
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "vq8_near_ties.json")


def rne32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest f32 value, ties to even
    (normal range only: the values here are far from under- and overflow)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    # 2^e <= x < 2^(e+1) after adjusting e
    if Fraction(2) ** e > x:
        e -= 1
    if Fraction(2) ** (e + 1) <= x:
        e += 1
    assert -126 <= e <= 127, x
    quantum = Fraction(2) ** (e - 23)
    m = x / quantum  # in [2^23, 2^24)
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def round_half_away(t: Fraction) -> int:
    a = abs(t)
    n = a.numerator // a.denominator
    if a - n >= Fraction(1, 2):
        n += 1
    return n if t >= 0 else -n


def code_of(v: Fraction, scale: Fraction) -> int:
    c = round_half_away(rne32(v / scale))
    return max(-127, min(127, c))


def f32(x: Fraction) -> float:
    v = float(x)
    assert Fraction(float(np.float32(v))) == x
    return v


def ulp32(x: Fraction) -> Fraction:
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    return Fraction(2) ** (e - 23)


def search(seed: int, want_recip: int, want_double: int):
    rng = np.random.default_rng(seed)
    while True:
        a = Fraction(float(np.float32(abs(rng.standard_normal()) * 10.0 ** rng.uniform(-2, 2))))
        scale = rne32(a / 127)
        if scale.numerator & (scale.numerator - 1) == 0 and scale.denominator & (scale.denominator - 1) == 0:
            continue  # a power of two: every order agrees
        recip = rne32(1 / scale)
        got_r, got_d = [], []
        for k in rng.permutation(126):
            mid = (k + Fraction(1, 2)) * scale
            base = rne32(mid)
            u = ulp32(base)
            for j in range(-3, 4):
                v = base + j * u
                if v <= 0 or v >= a:
                    continue
                sgn = -1 if rng.integers(2) else 1
                vv = sgn * v
                c = code_of(vv, scale)
                c_recip = max(-127, min(127, round_half_away(rne32(vv * recip))))
                exact = vv / scale
                c_double = max(-127, min(127, round_half_away(exact)))  # exact quotient, rounded once
                if c_recip != c and len(got_r) < want_recip:
                    got_r.append((vv, c))
                elif c_double != c and len(got_d) < want_double:
                    got_d.append((vv, c))
            if len(got_r) >= want_recip and len(got_d) >= want_double:
                break
        if len(got_r) >= want_recip and len(got_d) >= want_double:
            vals = [(a, 127)] + got_r + got_d
            return scale, vals, len(got_r), len(got_d)


def main():
    cases = []
    for seed, nr, nd in ((1, 4, 2), (2, 3, 3), (3, 5, 1), (4, 2, 2)):
        scale, vals, nr_, nd_ = search(seed, nr, nd)
        v = [f32(x) for x, _ in vals]
        codes = [c for _, c in vals]
        # Cross-check against numpy's IEEE f32 division (an independent
        # implementation of the same operations).
        s32 = np.float32(np.float32(v[0]) / np.float32(127.0))
        assert Fraction(float(s32)) == scale
        t = np.array(v, np.float32) / s32
        np_codes = np.clip(np.sign(t) * np.floor(np.abs(t).astype(np.float64) + 0.5), -127, 127)
        assert np_codes.astype(int).tolist() == codes, (np_codes, codes)
        cases.append({"v": v, "scale": f32(scale), "codes": codes,
                      "n_recip_sensitive": nr_, "n_double_sensitive": nd_})
    doc = {
        "source": ("vq8 quantiser ('llamay - Models and formats', The KV cache, in three "
                   "precisions), read as IEEE f32 operations: scale = a/127, t = v/scale, "
                   "code = clamp(round_half_away(t), -127, 127). Values near (k+1/2)*scale "
                   "for non-power-of-two scales; codes from exact rational arithmetic with "
                   "round-to-nearest-even to f32 (make_vq8_near_ties.py), cross-checked with "
                   "numpy f32 division. Each vector's first element is its absmax."),
        "cases": cases,
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print("wrote", OUT, [len(c["v"]) for c in cases])


if __name__ == "__main__":
    main()
