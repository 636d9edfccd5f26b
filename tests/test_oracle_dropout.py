"""Pins of the oracle's LoRA dropout: the Philox4x32-10 generator against the
known-answer vectors published with its definition (Salmon, Moraes, Dror,
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) and, at 64-bit
width, against numpy's own Philox bit generator; the mask against binomial
bounds and its counter-based structure; the dropout output and the layer's
gradients against special cases and exact directional derivatives."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import qlora_workloads as wl

# Philox4x32-10 known-answer vectors (counter words, key words) -> output,
# from the generator's published reference implementation.
KAT_4X32_10 = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT_4X32_10)
def test_philox4x32_known_answers(ctr, key, want):
    assert tuple(oracle.philox(ctr, key, 32)) == want


@pytest.mark.parametrize("key,ctr", [((0, 0), (0, 0, 0, 0)), ((7, 11), (5, 0, 3, 9)),
                                     ((2**64 - 1, 123), (2**63, 1, 2, 3))])
def test_philox_round_function_matches_numpy_at_64_bits(key, ctr):
    """numpy's Philox bit generator is Philox4x64-10; it advances the counter
    by one before producing a block.  The same round function at 64-bit width
    must reproduce it: a swapped multiplier, a missing key bump or a wrong
    output permutation fails here as well as in the 32-bit vectors."""
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    got = [int(x) for x in g.random_raw(8)]
    c = list(ctr)
    for blk in range(2):
        c[0] += 1
        want = oracle.philox(c, key, 64)
        assert got[4 * blk:4 * blk + 4] == want


def test_vectorised_words_equal_scalar_generator():
    groups = np.array([0, 1, 2, 1000, 2**32 - 1, 2**32, 2**40 + 17])
    for seed in (0, 1, 2**33 + 5):
        words = oracle.philox4x32_words(seed, groups)
        for j, gi in enumerate(groups):
            want = oracle.philox((int(gi) & 0xFFFFFFFF, int(gi) >> 32, 0, 0),
                                 (seed & 0xFFFFFFFF, seed >> 32), 32)
            assert [int(x) for x in words[j]] == want


def test_keep_rate_within_binomial_bounds():
    M, K, p = 256, 4096, 0.05
    m = oracle.dropout_mask(M, K, p, seed=77)
    n = m.size
    q = 1.0 - oracle.dropout_threshold(p) / 2.0**32
    sd = np.sqrt(n * q * (1 - q))
    assert abs(m.sum() - n * q) < 6 * sd
    # rows and columns look alike (no structure by position)
    assert abs(m[:, :K // 2].mean() - m[:, K // 2:].mean()) < 6 * np.sqrt(q * (1 - q) / (n / 2))


def test_threshold_and_scale():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.5) == 2**31
    assert oracle.dropout_threshold(0.05) == int(Fraction(0.05) * 2**32)   # floor of the exact product
    s = oracle.dropout_scale(0.05)
    exact = 1 / (1 - Fraction(0.05))
    assert abs(Fraction(float(s)) - exact) <= Fraction(2) ** -24 * exact   # one fp32 rounding
    assert oracle.dropout_scale(0.5) == np.float32(2.0)


def test_p_zero_keeps_everything_unchanged():
    X = wl.activations(3, 1, 16, 256)
    m = oracle.dropout_mask(16, 256, 0.0, seed=5)
    assert m.all()
    assert np.array_equal(oracle.dropout_apply(X, m, 0.0), X)


def test_mask_is_counter_based():
    """Each element's draw depends only on (seed, index): any row subset is a
    slice of the full mask, and another seed gives another mask."""
    M, K = 40, 96
    full = oracle.dropout_mask(M, K, 0.3, seed=9)
    rows = np.array([0, 7, 39, 13])
    assert np.array_equal(oracle.dropout_mask(M, K, 0.3, seed=9, rows=rows), full[rows])
    assert not np.array_equal(oracle.dropout_mask(M, K, 0.3, seed=10), full)


def test_dropout_apply_values():
    """Kept: bf16(fp32(x * scale)) -- checked with exact rational arithmetic
    for a few values; dropped: +0."""
    p = 0.05
    xs = np.array([1.0, -3.5, 0.0078125, 1.5e-3], dtype=np.float32)
    bits = wl.round_to_bf16_bits(xs)
    keep = np.array([True, True, True, False])
    got = oracle.dropout_apply(bits, keep, p)
    s = Fraction(float(oracle.dropout_scale(p)))
    for j in range(3):
        x = Fraction(float(oracle.bf16_bits_to_f64(bits[j:j + 1])[0]))
        prod32 = Fraction(float(np.float32(float(x * s))))   # fp32 rounding of the exact product
        # bf16 candidates around prod32: the result is the nearer one
        v = oracle.bf16_bits_to_f64(got[j:j + 1])[0]
        step = Fraction(2) ** (int(np.frexp(float(prod32))[1]) - 8)
        assert abs(Fraction(float(v)) - prod32) <= step / 2
    assert got[3] == 0


def _layer(X, keep, W, A, B, s):
    return X @ W.T + s * ((X * keep) @ A.T) @ B.T


def test_forward_backward_all_kept_is_the_plain_layer():
    g = np.random.default_rng(4)
    M, K, N, r = 12, 64, 40, 8
    X, W = g.normal(size=(M, K)), g.normal(size=(N, K))
    A, B, dY = g.normal(size=(r, K)), g.normal(size=(N, r)), g.normal(size=(M, N))
    keep = np.ones((M, K), bool)
    Y, T = oracle.forward_dropout(X, X, W, A, B, 16.0, r)
    Y0, T0 = oracle.forward(X, W, A, B, 16.0, r)
    assert np.allclose(Y, Y0, rtol=1e-13, atol=1e-12) and np.allclose(T, T0, rtol=1e-13, atol=1e-12)
    got = oracle.backward_dropout(dY, X, keep, 0.0, W, A, B, 16.0, r)
    want = oracle.backward(dY, X, W, A, B, 16.0, r)
    for a, b in zip(got, want):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-12)


def test_gradients_are_exact_directional_derivatives():
    """The layer is linear in X, in A and in B separately (mask fixed), so the
    inner product of each gradient with a direction V equals <dY, f(. + V) -
    f(.)> up to fp64 rounding."""
    g = np.random.default_rng(5)
    M, K, N, r, p, alpha = 10, 64, 24, 4, 0.25, 8.0
    X, W = g.normal(size=(M, K)), g.normal(size=(N, K))
    A, B, dY = g.normal(size=(r, K)), g.normal(size=(N, r)), g.normal(size=(M, N))
    mask = g.random((M, K)) > p
    sc = float(oracle.dropout_scale(p))
    keep = mask * sc
    s = oracle.lora_scale(alpha, r)
    Xd = X * keep
    dX, dA, dB = oracle.backward_dropout(dY, Xd, mask, p, W, A, B, alpha, r)
    Y, _ = oracle.forward_dropout(X, Xd, W, A, B, alpha, r)
    assert np.allclose(Y, _layer(X, keep, W, A, B, s), rtol=1e-12, atol=1e-12)
    for grad, which in ((dX, 0), (dA, 1), (dB, 2)):
        V = g.normal(size=grad.shape)
        args = [X, A, B]
        args2 = list(args)
        args2[which] = args[which] + V
        f0 = _layer(args[0], keep, W, args[1], args[2], s)
        f1 = _layer(args2[0], keep, W, args2[1], args2[2], s)
        lhs, rhs = np.sum(grad * V), np.sum(dY * (f1 - f0))
        assert abs(lhs - rhs) <= 1e-9 * (abs(rhs) + 1.0)


def test_pack_mask_bit_order():
    m = np.zeros(70, bool)
    m[[0, 5, 31, 32, 69]] = True
    w = oracle.pack_mask(m)
    assert w.dtype == np.uint32 and w.size == 3
    assert int(w[0]) == (1 | 1 << 5 | 1 << 31) and int(w[1]) == 1 and int(w[2]) == 1 << 5
