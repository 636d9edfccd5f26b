"""Pins for the oracle's blockwise NF4 quantisation, double quantisation and
dequantisation (CPU only).

What pins what:
* round trip: blocks made of exact codebook multiples come back unchanged;
* the reconstruction error bound half-gap * absmax (no double quant) and the
  extra |a - a_hat| <= s_g / 254 with it;
* the pages' bit budget (golden/bit_budget.json) from the real buffer sizes;
* the mean against math.fsum (exact whenever the fp64 sum is exact);
* bf16 rounding against torch's own float32 -> bfloat16 conversion;
* the nibble order on a hand-written example.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import qlora_workloads as wl

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "bit_budget.json")))


def test_pack_order_hand_example():
    codes = np.array([1, 2, 3, 4, 15, 0], dtype=np.uint8)
    assert list(oracle.pack_nibbles(codes)) == [0x12, 0x34, 0xF0]
    assert list(oracle.unpack_nibbles(np.array([0xAB], np.uint8))) == [0xA, 0xB]


def test_absmax_hand_example():
    w = np.zeros(128, np.float32)
    w[3], w[70], w[100] = -2.5, 1.25, -1.5
    assert list(oracle.absmax_blocks(w, 64)) == [2.5, 1.5]


@pytest.mark.parametrize("a", [np.float32(1.0), np.float32(0.03125), np.float32(0.0173)])
def test_round_trip_codebook_multiples(a):
    q = oracle.nf4_codebook()
    g = np.random.default_rng(1)
    idx = g.integers(0, 16, size=(4, 64)).astype(np.uint8)
    idx[:, 0], idx[:, 1] = 0, 15            # +-a present: absmax is exactly a
    w = (q[idx] * a).astype(np.float32)
    codes, am = oracle.quantize_nf4(w, 64)
    assert np.all(am == a)
    assert np.array_equal(codes.reshape(4, 64), idx)
    # dequant without double quant reproduces the same fp32 values
    w_hat = (q[codes] * np.repeat(am, 64)).astype(np.float32).reshape(4, 64)
    assert np.array_equal(w_hat, w)


def test_zero_block_gives_zero_code():
    w = np.zeros((2, 64), np.float32)
    w[1, 5] = 0.25
    codes, am = oracle.quantize_nf4(w, 64)
    assert am[0] == 0 and np.all(codes[:64] == 7)
    assert codes[64 + 5] == 15


def test_rejects_non_finite():
    w = np.zeros(64, np.float32)
    w[3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_nf4(w)


def test_reconstruction_error_bound_without_dq():
    q = oracle.nf4_codebook().astype(np.float64)
    half_gap = np.diff(q).max() / 2
    assert abs(half_gap - 0.15190) < 1e-4       # widest gap is between levels 0 and 1
    w = wl.weight(0, 2, 0, wl.Linear("w", 256, 1024, 16, 32.0))
    codes, am = oracle.quantize_nf4(w, 64)
    w_hat = (oracle.nf4_codebook()[codes] * np.repeat(am, 64)).astype(np.float64)
    err = np.abs(w.reshape(-1).astype(np.float64) - w_hat)
    bound = half_gap * np.repeat(am, 64).astype(np.float64) * (1 + 1e-6)
    assert np.all(err <= bound)
    # local bound: each element within half of the gap around its own level
    lo = np.concatenate([[0.0], np.diff(q) / 2])[codes]
    hi = np.concatenate([np.diff(q) / 2, [0.0]])[codes]
    n = w.reshape(-1).astype(np.float64) / np.repeat(am, 64)
    assert np.all(n - q[codes] <= hi + 1e-6) and np.all(q[codes] - n <= lo + 1e-6)


def test_double_quant_mean_and_bounds():
    w = wl.weight(0, 2, 0, wl.Linear("w", 512, 4096, 16, 32.0))
    _, am = oracle.quantize_nf4(w, 64)
    codes, scales, mu = oracle.double_quant(am, 256)
    assert codes.dtype == np.uint8 and codes.max() <= 254
    assert scales.size == am.size // 256
    # the fp64 sum is exact for these magnitudes, so the fixed order equals fsum
    assert mu == np.float32(math.fsum(am.astype(np.float64)) / am.size)
    a_hat = oracle.dequant_absmax(codes, scales, mu, 256)
    s_rep = np.repeat(scales, 256).astype(np.float64)
    err = np.abs(a_hat.astype(np.float64) - am.astype(np.float64))
    assert np.all(err <= s_rep / 254 + 4 * np.spacing(np.abs(am)).astype(np.float64))
    # the largest |centred| constant in each group is represented exactly up to rounding
    c = (am - mu).astype(np.float32).reshape(-1, 256)
    jmax = np.abs(c).argmax(axis=1)
    assert np.all(np.isin(codes.reshape(-1, 256)[np.arange(c.shape[0]), jmax], [0, 254]))


def test_double_quant_fixed_order_partial_group():
    a = np.linspace(0.01, 0.05, 300).astype(np.float32)      # one full + one partial group
    codes, scales, mu = oracle.double_quant(a, 256)
    assert scales.size == 2 and codes.size == 300
    s = 0.0
    for grp in (a[:256], a[256:]):
        t = 0.0
        for v in grp.astype(np.float64):
            t += v
        s += t
    assert mu == np.float32(s / 300)


def test_double_quant_zero_group():
    a = np.full(256, 0.02, np.float32)           # all equal: centred values are 0
    codes, scales, mu = oracle.double_quant(a, 256)
    assert mu == np.float32(0.02) and scales[0] == 0 and np.all(codes == 127)
    assert np.all(oracle.dequant_absmax(codes, scales, mu) == np.float32(0.02))


def test_bit_budget_matches_pages():
    """The pages' 0.5 -> 0.13 bit overhead and 0.37 / ~0.4 bit saving, from buffer sizes."""
    N, K = 512, 4096
    w = wl.weight(0, 2, 0, wl.Linear("w", N, K, 16, 32.0))
    codes4, am = oracle.quantize_nf4(w, GOLD["blocksize_example"]["value"])
    packed = oracle.pack_nibbles(codes4)
    codes8, scales, mu = oracle.double_quant(am, 256)
    numel = N * K
    bits_plain = (packed.nbytes + am.nbytes) * 8 / numel
    bits_dq = (packed.nbytes + codes8.nbytes + scales.nbytes + 4) * 8 / numel
    assert abs(bits_plain - 4 - GOLD["overhead_fp32_constants_bits_per_param"]["value"]) < 1e-9
    assert abs(bits_dq - 4 - GOLD["overhead_after_double_quant_bits_per_param"]["value"]) < 0.01
    saving = bits_plain - bits_dq
    assert abs(saving - GOLD["saving_bits_per_param_li"]["value"]) < 0.01
    assert abs(saving - GOLD["saving_bits_per_param_ag"]["value"]) < 0.05
    assert abs(bits_dq / 8 - GOLD["storage_bytes_per_param_nf4"]["value"]) < 0.02
    assert abs(oracle.bits_per_param(numel) - bits_dq) < 1e-9


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(5)
    x = np.concatenate([g.standard_normal(100_000).astype(np.float32) * 1e-2,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.0e38], np.float32)])
    # add exact ties (low 16 bits == 0x8000)
    ties = (g.integers(0, 2**15, 1000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32)
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x)]
    ours = oracle.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_dequant_round_trip_and_bound():
    N, K = 64, 512
    w = wl.weight(3, 2, 0, wl.Linear("w", N, K, 16, 32.0))
    codes4, am = oracle.quantize_nf4(w, 64)
    packed = oracle.pack_nibbles(codes4)
    c8, sc, mu = oracle.double_quant(am, 256)
    w_hat, wb = oracle.dequant_nf4(packed, c8, sc, mu, N, K)
    a_hat = oracle.dequant_absmax(c8, sc, mu)
    q = oracle.nf4_codebook()
    # per element: w_hat = fp32(Q4[code] * a_hat)
    assert np.array_equal(w_hat.reshape(-1), (q[codes4] * np.repeat(a_hat, 64)).astype(np.float32))
    # total error <= half gap * absmax + |a - a_hat|
    err = np.abs(w.reshape(-1).astype(np.float64) - w_hat.reshape(-1))
    bound = (0.1519 * np.repeat(am, 64) + np.abs(np.repeat(am - a_hat, 64))) * 1.0001
    assert np.all(err <= bound + 1e-12)
    # bf16 bits are the RNE of w_hat
    torch = pytest.importorskip("torch")
    tb = torch.from_numpy(w_hat).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wb, tb)
