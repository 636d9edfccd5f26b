"""The kernels compute the 8-bit double-quantisation level Q8[i] = (i - 127)/127
(correctly rounded to fp32, as the oracle's linear code fixes it) without a
division: q0 = x * fl(1/127), then q = fma(fma(-q0, 127, x), fl(1/127), q0).
This checks, in exact rational arithmetic with round-to-nearest-even, that the
form equals the correctly rounded quotient for every byte value (the oracle's
255 levels and the unused code 255), and
that the plain product x * fl(1/127) alone would not (so the correction step
is needed)."""
from fractions import Fraction

import numpy as np

import oracle


def _rne_f32(v: Fraction) -> np.float32:
    """Nearest fp32 to an exact rational (ties to even); |v| in [2^-126, 2^127)."""
    if v == 0:
        return np.float32(0.0)
    sign, a = (-1, -v) if v < 0 else (1, v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    q = a / ulp
    n, rem = divmod(q.numerator, q.denominator)
    rem = Fraction(rem, q.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n * ulp))


def _fma(a, b, c) -> np.float32:
    return _rne_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def test_corrected_reciprocal_equals_quotient_for_all_codes():
    inv = _rne_f32(Fraction(1, 127))
    assert inv == np.float32(1.0) / np.float32(127.0)
    table = oracle.dq_codebook()
    plain_mismatch = 0
    for i in range(256):
        x = np.float32(i - 127)
        want = _rne_f32(Fraction(i - 127, 127))
        if i < table.size:            # the code has 255 levels; 255 is never stored
            assert want == table[i], i
        q0 = _rne_f32(Fraction(float(x)) * Fraction(float(inv)))
        plain_mismatch += int(q0 != want)
        q = _fma(r := _fma(-q0, np.float32(127.0), x), inv, q0)
        assert q == want, (i, r)
    assert plain_mismatch > 0
