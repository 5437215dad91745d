"""The exact-rounding helper of the operation-order pins against the IEEE
arithmetic of numpy (binary32 / binary64 multiply, divide, add and sqrt are
correctly rounded there), on seeded operands and on hand-picked ties."""
from fractions import Fraction

import numpy as np

from exact_fp import f32, fl32, fl64, rne_int, sqrt64


def test_fl32_matches_numpy_float32_ops():
    g = np.random.default_rng(5)
    for _ in range(3000):
        a, b = (g.standard_normal(2) * g.uniform(1e-3, 1e3)).astype(np.float32)
        assert Fraction(float(a * b)) == fl32(f32(a) * f32(b))
        assert Fraction(float(a / b)) == fl32(f32(a) / f32(b))
        assert Fraction(float(a + b)) == fl32(f32(a) + f32(b))


def test_fl64_and_sqrt64_match_numpy_float64_ops():
    g = np.random.default_rng(6)
    for _ in range(3000):
        x = float(abs(g.standard_normal())) * 10.0 ** g.uniform(-30, 30)
        y = float(g.standard_normal())
        assert Fraction(float(np.sqrt(np.float64(x)))) == sqrt64(Fraction(x))
        assert Fraction(1.0 / x) == fl64(1 / Fraction(x))
        assert Fraction(x * y) == fl64(Fraction(x) * Fraction(y))
    for v in (4.0, 2.0, 0.25, 1e-300, 2.0 ** 1000):
        assert sqrt64(Fraction(v)) == Fraction(float(np.sqrt(v)))


def test_ties_go_to_even():
    one = Fraction(1)
    ulp = Fraction(1, 2 ** 23)
    assert fl32(one + ulp / 2) == one                 # tie, 1 is even
    assert fl32(one + 3 * ulp / 2) == one + 2 * ulp   # tie, 1 + ulp is odd
    assert fl32(Fraction(2 ** 24 + 1)) == 2 ** 24
    assert fl32(Fraction(2 ** 24 + 3)) == 2 ** 24 + 4
    assert [rne_int(Fraction(v, 2)) for v in (-5, -3, -1, 1, 3, 5)] == [-2, -2, 0, 0, 2, 2]
    tiny = Fraction(1, 2 ** 149)                      # smallest binary32 subnormal
    assert fl32(tiny / 2) == 0 and fl32(3 * tiny / 2) == 2 * tiny
