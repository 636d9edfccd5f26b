"""Pins for the oracle's codebooks and its nearest-level rule (CPU only).

The NF4 levels are checked against what defines them, not against a retyped
formula: the FORWARD normal CDF (math.erf) must map the positive levels to
probabilities evenly spaced between 1/2 and delta and the negative levels to
probabilities evenly spaced between 1/2 and 1-delta ("quantiles, equal
expected mass per bin": llm-compass "QLoRA", 方法与公式 item 1; auryth.ai
"QLoRA", NF4 box; learn-interview-questions §2).  A second, independent
inverse (mpmath bisection on erfc at 50 digits) reproduces the fp32 bits.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "bit_budget.json")))


def _phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def test_nf4_structure():
    q = oracle.nf4_codebook()
    assert q.dtype == np.float32 and q.size == GOLD["nf4_levels"]["value"]
    assert np.all(np.diff(q.astype(np.float64)) > 0), "levels strictly increasing"
    assert q[0] == -1.0 and q[15] == 1.0, "range normalised to [-1, 1]"
    assert q[7] == 0.0 and np.signbit(q[7]) == False, "exact (positive) zero"
    assert (q > 0).sum() == 8 and (q < 0).sum() == 7


def test_nf4_levels_are_equal_probability_quantiles():
    """Phi(level * Phi^-1(delta)) must be evenly spaced on each side."""
    q = oracle.nf4_codebook().astype(np.float64)
    d = oracle.NF4_DELTA
    # z = Phi^-1(delta) found by bisection on the forward CDF (independent route)
    lo, hi = 0.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if _phi(mid) < d else (lo, mid)
    z = 0.5 * (lo + hi)
    pos = sorted(q[q > 0])[::-1]          # 1.0 first
    neg = sorted(q[q < 0])                # -1.0 first
    for i, v in enumerate(pos):
        want = d - i * (d - 0.5) / 8.0
        assert abs(_phi(v * z) - want) < 2e-8, (i, v)
    for j, v in enumerate(neg):
        want = (1.0 - d) + j * (d - 0.5) / 7.0
        assert abs(_phi(v * z) - want) < 2e-8, (j, v)
    # equal spacing in probability on each side
    pp = np.array([0.5] + [_phi(v * z) for v in sorted(q[q > 0])])
    assert np.allclose(np.diff(pp), (d - 0.5) / 8.0, atol=3e-8)
    pn = np.array([_phi(v * z) for v in sorted(q[q < 0])] + [0.5])
    assert np.allclose(np.diff(pn), (d - 0.5) / 7.0, atol=3e-8)


def test_nf4_bits_match_high_precision_inverse():
    """An mpmath bisection at 50 digits gives the same fp32 bits."""
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    d = mp.mpf(1) - (mp.mpf(1) / 30 + mp.mpf(1) / 32) / 2

    def inv(p):
        lo, hi = mp.mpf(-20), mp.mpf(20)
        for _ in range(200):
            m = (lo + hi) / 2
            if mp.ncdf(m) < p:
                lo = m
            else:
                hi = m
        return (lo + hi) / 2

    z = inv(d)
    vals = [inv(d - i * (d - mp.mpf(1) / 2) / 8) / z for i in range(8)]
    vals += [-inv(d - j * (d - mp.mpf(1) / 2) / 7) / z for j in range(7)]
    vals += [mp.mpf(0)]
    # correctly rounded fp32 of the 50-digit value (via Fraction, no double rounding)
    def rn32(x):
        f = Fraction(mp.nstr(x, 45, min_fixed=-100, max_fixed=100))
        c = np.float32(float(f))
        best = None
        for cand in (np.nextafter(c, np.float32(-2)), c, np.nextafter(c, np.float32(2))):
            err = abs(Fraction(float(cand)) - f)
            if best is None or err < best[0]:
                best = (err, cand)
        return best[1]
    want = np.array(sorted(rn32(v) for v in vals), dtype=np.float32)
    got = oracle.nf4_codebook()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_dq_codebook_is_correctly_rounded_linear():
    q8 = oracle.dq_codebook()
    assert q8.size == 255 and q8[0] == -1.0 and q8[127] == 0.0 and q8[254] == 1.0
    for i in range(255):
        exact = Fraction(i - 127, 127)
        v = q8[i]
        err = abs(Fraction(float(v)) - exact)
        for nb in (np.nextafter(v, np.float32(-2)), np.nextafter(v, np.float32(2))):
            assert err <= abs(Fraction(float(nb)) - exact), i


def _exact_nearest(v, levels):
    fv = Fraction(float(v))
    best, bi = None, None
    for i, l in enumerate(levels):
        d = abs(fv - Fraction(float(l)))
        if best is None or d < best:
            best, bi = d, i
    return bi


@pytest.mark.parametrize("book", ["nf4", "dq"])
def test_nearest_index_matches_exact_rationals(book):
    levels = oracle.nf4_codebook() if book == "nf4" else oracle.dq_codebook()
    g = np.random.default_rng(123)
    vals = list(g.uniform(-1, 1, 400).astype(np.float32))
    vals += [np.float32(x) for x in (0.0, -0.0, 1.0, -1.0, 1e-30, -1e-30, 1e-45)]
    # every exact midpoint that fp32 can hold, and its fp32 neighbours
    for i in range(levels.size - 1):
        mid = (Fraction(float(levels[i])) + Fraction(float(levels[i + 1]))) / 2
        m32 = np.float32(float(mid))
        for v in (np.nextafter(m32, np.float32(-2)), m32, np.nextafter(m32, np.float32(2))):
            vals.append(v)
    vals = np.array(vals, dtype=np.float32)
    got = oracle.nearest_index(vals, levels)
    want = np.array([_exact_nearest(v, levels) for v in vals])
    assert np.array_equal(got, want)


def test_nf4_ties_go_to_lower_index():
    q = oracle.nf4_codebook()
    ties = 0
    for i in range(15):
        mid = (Fraction(float(q[i])) + Fraction(float(q[i + 1]))) / 2
        m32 = np.float32(float(mid))
        if Fraction(float(m32)) == mid:
            ties += 1
            assert oracle.nearest_index(np.array([m32]), q)[0] == i
            assert oracle.nearest_index(np.array([np.nextafter(m32, np.float32(2))]), q)[0] == i + 1
    assert ties == 4   # midpoints 2-3, 6-7, 7-8 and 14-15 are representable


def test_nearest_equals_midpoint_search():
    """Brute-force argmin == search among exact midpoints (side='left' = lower on ties)."""
    q = oracle.nf4_codebook()
    mids = (q[:-1].astype(np.float64) + q[1:].astype(np.float64)) / 2   # exact in fp64
    v = np.random.default_rng(7).uniform(-1, 1, 200_000).astype(np.float32)
    got = oracle.nearest_index(v, q)
    want = np.searchsorted(mids, v.astype(np.float64), side="left")
    assert np.array_equal(got, want)
