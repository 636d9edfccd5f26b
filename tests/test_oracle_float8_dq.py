"""Pins of the oracle's 8-bit-float second-level table (the other reading of
the pages' "8-bit" double quantisation next to the linear code; [AU]
Dubbele Quantisatie box, [LC] 方法与公式 item 2).

The levels are checked against a source other than the oracle's own bit-field
decoding: torch's float8_e4m3fn dtype decodes the same 256 bit patterns.
"""
import math

import numpy as np
import pytest

import oracle


def test_e4m3_values_match_torch_decoding_of_every_bit_pattern():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = bits.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = sorted(set(v for v in vals.tolist() if math.isfinite(v)))
    assert np.array_equal(np.array(finite), oracle.fp8_e4m3_values())


def test_e4m3_structure():
    v = oracle.fp8_e4m3_values()
    assert v.size == 253                                  # 2 x 127 patterns, +-0 once
    assert v[-1] == 448.0 and v[0] == -448.0              # 1.75 * 2^8
    pos = v[v > 0]
    assert pos[0] == 2.0 ** -9                            # smallest subnormal
    assert np.array_equal(v, -v[::-1])                    # symmetric
    assert np.count_nonzero(v == 0.0) == 1
    # every binade 2^-6 .. 2^8 holds 8 evenly spaced values
    for e in range(-6, 8):
        b = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert b.size == 8 and np.allclose(np.diff(b), 2.0 ** (e - 3))


def test_float8_table_levels():
    q = oracle.dq_float8_codebook()
    assert q.dtype == np.float32 and q.size == 253
    assert q[0] == -1.0 and q[-1] == 1.0 and q[126] == 0.0
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    exact = oracle.fp8_e4m3_values() / 448.0
    assert np.array_equal(q, exact.astype(np.float32))     # one rounding from fp64
    assert np.all(np.abs(q.astype(np.float64) - exact) <= np.spacing(np.abs(q)) / 2)


def test_float8_table_round_trip_and_nearest_bound():
    q = oracle.dq_float8_codebook()
    assert np.array_equal(oracle.nearest_index(q, q), np.arange(q.size))
    g = np.random.default_rng(3)
    x = g.uniform(-1, 1, 20000).astype(np.float32)
    idx = oracle.nearest_index(x, q).astype(np.int64)
    err = np.abs(x.astype(np.float64) - q[idx].astype(np.float64))
    # nearest level: never farther than half the gap to the neighbour on either side
    lo = np.clip(np.searchsorted(q, x, side="right") - 1, 0, q.size - 2)
    gap = q[lo + 1].astype(np.float64) - q[lo].astype(np.float64)
    assert np.all(err <= gap / 2 + 1e-12)


def test_double_quant_with_the_float8_table():
    """Codes index the float table, the zero group takes the zero level, and the
    decoded constants stay within s_g times half the local gap (plus fp32
    rounding) of the exact ones."""
    g = np.random.default_rng(5)
    a = np.abs(g.standard_normal(1024)).astype(np.float32) * np.float32(0.02)
    a[512:768] = a[512:768].mean(dtype=np.float32)           # a group that centres near zero
    q = oracle.dq_float8_codebook()
    codes, scales, mu = oracle.double_quant(a, 256, levels=q)
    assert codes.max() <= 252
    ah = oracle.dequant_absmax(codes, scales, mu, 256, levels=q)
    c = (a - mu).astype(np.float64)
    for gi in range(4):
        sl = slice(256 * gi, 256 * (gi + 1))
        n2 = c[sl] / float(scales[gi])
        lo = np.clip(np.searchsorted(q, n2, side="right") - 1, 0, q.size - 2)
        gap = (q[lo + 1].astype(np.float64) - q[lo].astype(np.float64)) * float(scales[gi])
        assert np.all(np.abs(ah[sl] - a[sl]) <= gap / 2 + 4e-7 * np.abs(a[sl]).max() + 1e-9)
    z = np.full(256, 0.5, dtype=np.float32)                    # s_g = 0: all zero code
    cz, sz, _ = oracle.double_quant(z, 256, levels=q)
    assert sz[0] == 0.0 and np.all(cz == 126)


def test_float8_table_keeps_small_constants_next_to_an_outlier():
    """The reason for a float code: in a group whose scale is set by one large
    outlier constant, the linear code's step s_g / 127 is a large fraction of
    the ordinary constants, while the float code keeps their relative error
    small."""
    g = np.random.default_rng(7)
    a = (0.03 + 0.005 * g.standard_normal(256)).astype(np.float32)
    a[17] = np.float32(4.0)                                      # one outlier block
    lin = oracle.double_quant(a, 256)
    f8 = oracle.double_quant(a, 256, levels=oracle.dq_float8_codebook())
    ah_lin = oracle.dequant_absmax(*lin, 256)
    ah_f8 = oracle.dequant_absmax(*f8, 256, levels=oracle.dq_float8_codebook())
    keep = np.arange(256) != 17
    rel_lin = np.abs(ah_lin[keep] - a[keep]) / a[keep]
    rel_f8 = np.abs(ah_f8[keep] - a[keep]) / a[keep]
    assert np.median(rel_f8) < np.median(rel_lin)
