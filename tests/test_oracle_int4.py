"""Pins of the uniform INT4 codebook and the generic blockwise quantiser that
the NF4 comparison uses: even spacing and symmetry of the levels, round trip
of the levels, the half-spacing error bound, and the pages' argument for NF4
(on normally distributed blocks NF4 reconstructs with less error and uses its
16 codes more evenly, i.e. with higher entropy)."""
from fractions import Fraction

import numpy as np

import oracle


def test_levels_evenly_spaced_and_symmetric():
    lv = oracle.int4_codebook()
    assert lv.dtype == np.float32 and lv.size == 16
    assert lv[0] == -1.0 and lv[-1] == 1.0
    assert np.array_equal(lv[::-1], -lv)
    for i in range(16):
        exact = Fraction(-1) + Fraction(2 * i, 15)
        assert abs(Fraction(float(lv[i])) - exact) <= Fraction(2) ** -25   # one fp32 rounding of |x| <= 1


def test_levels_round_trip():
    lv = oracle.int4_codebook()
    w = np.tile(lv, 4).astype(np.float32)         # a block of 64 whose absmax is 1
    c, a = oracle.quantize_blocks(w, lv, 64)
    assert a[0] == 1.0
    assert np.array_equal(c, np.tile(np.arange(16), 4))
    what, _ = oracle.dequant_codes(c, a, 64, levels=lv)
    assert np.array_equal(what, w)


def test_error_bound_half_spacing():
    lv = oracle.int4_codebook()
    g = np.random.default_rng(1)
    w = g.normal(size=64 * 500).astype(np.float32)
    c, a = oracle.quantize_blocks(w, lv, 64)
    what, _ = oracle.dequant_codes(c, a, 64, levels=lv)
    per = np.repeat(a, 64)
    assert np.all(np.abs(what - w) <= per * (1.0 / 15.0 + 1e-6))


def test_nf4_default_is_unchanged():
    g = np.random.default_rng(2)
    w = g.normal(size=64 * 40).astype(np.float32)
    c1, a1 = oracle.quantize_nf4(w, 64)
    c2, a2 = oracle.quantize_blocks(w, oracle.nf4_codebook(), 64)
    assert np.array_equal(c1, c2) and np.array_equal(a1, a2)


def test_nf4_beats_uniform_int4_on_gaussian_blocks():
    g = np.random.default_rng(3)
    W = g.standard_normal(64 * 8192).astype(np.float32)
    res = {}
    for name, lv in (("nf4", oracle.nf4_codebook()), ("int4", oracle.int4_codebook())):
        c, a = oracle.quantize_blocks(W, lv, 64)
        w, _ = oracle.dequant_codes(c, a, 64, levels=lv)
        err = np.linalg.norm(w - W) / np.linalg.norm(W)
        h = np.bincount(c, minlength=16) / c.size
        ent = -np.sum(h[h > 0] * np.log2(h[h > 0]))
        res[name] = (err, ent)
    assert res["nf4"][0] < 0.95 * res["int4"][0]
    assert res["nf4"][1] > res["int4"][1] + 0.2
    assert res["nf4"][1] > 3.8          # close to the 4-bit maximum
