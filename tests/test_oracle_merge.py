"""Pins of the oracle's adapter merge W_merged = bf16(W_hat + s B A) and of
its fp64 -> bf16 rounding, against facts fixed outside the oracle: the
special case B = 0, a closed form for constant adapters, hand-worked
rounding ties, and torch's own bf16 conversion."""
import numpy as np
import pytest

import oracle
import qlora_workloads as wl


def test_zero_up_projection_gives_the_dequantised_base():
    rng = np.random.default_rng(1)
    W = rng.normal(0, 0.02, (64, 128)).astype(np.float32)
    c4, am = oracle.quantize_nf4(W, 64)
    c8, sc, mu = oracle.double_quant(am, 256)
    _, wb = oracle.dequant_nf4(oracle.pack_nibbles(c4), c8, sc, mu, 64, 128)
    Wh = oracle.bf16_bits_to_f64(wb)
    A = rng.normal(0, 1, (16, 128))
    m = oracle.merge(Wh, A, np.zeros((64, 16)), 32.0, 16)
    assert np.array_equal(oracle.f64_to_bf16_bits(m), wb)


@pytest.mark.parametrize("alpha,r", [(32.0, 16), (16.0, 8), (48.0, 24), (4.0, 16)])
def test_constant_adapters_closed_form(alpha, r):
    """A = a (all entries), B = b: (B A)[n, k] = r a b, so the merged weight
    (alpha / r exact in fp32 for these pairs)
    is W + (alpha / r) r a b = W + alpha a b.  A dropped scale, alpha in place
    of alpha / r, or a transposed product all break this."""
    N, K, a, b = 24, 40, 0.25, -0.5
    W = np.random.default_rng(2).integers(-8, 8, (N, K)) / 16.0
    m = oracle.merge(W, np.full((r, K), a), np.full((N, r), b), alpha, r)
    assert m.shape == (N, K)
    assert np.array_equal(m, W + alpha * a * b)


def test_rounding_ties_to_even():
    # bf16 has 8 significant bits: the spacing just above 1 is 2^-7.
    x = np.array([1.0 + 2.0 ** -8,        # tie between 1 and 1 + 2^-7: even is 1
                  1.0 + 3 * 2.0 ** -8,    # tie between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
                  1.0 + 2.0 ** -8 + 2.0 ** -30,   # just above the tie: up
                  -(2.0 + 2.0 ** -7),     # tie at magnitude 2 (spacing 2^-6): even is 2
                  0.75])
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.0, 0.75])
    got = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(x))
    assert np.array_equal(got, want)


def test_rounding_matches_torch_bf16():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).normal(0, 0.05, 4096).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(oracle.f64_to_bf16_bits(x), ref.view(np.uint16))
