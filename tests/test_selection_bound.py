"""The error bound behind the selection kernel's decision band, checked in exact arithmetic (no GPU).

The kernel scales each pooled fp64 vector by a power of two so that every |x~_d| < 1/4, splits it into four
int8 limbs 7 bits apart (x~ = a1 2^-8 + a2 2^-15 + a3 2^-22 + a4 2^-29 + r), and approximates x~ . y~ by the
ten exact integer limb products with n + m <= 5; it relies on an error below 1.5 * 2^-30 per entry, hence
|t - x~ . y~| < 1.5 * 2^-23 for D <= 128, which sets the band of 56 key units. This test restates that split from its description in exact rational
arithmetic and checks the bound on random vectors and on vectors built to stress it (every entry just below
1/4 in magnitude, entries whose limb remainders sit on rounding ties, signs that line the errors up).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

BOUND = Fraction(3, 2) * Fraction(1, 2 ** 23)
BOUND_PER_D = Fraction(3, 2) * Fraction(1, 2 ** 30)


def scaled(x):
    """x~ = x 2^-(F+2) with max |x| = f 2^F, f in [1/2, 1); exact."""
    mx = float(np.max(np.abs(x)))
    if mx == 0.0:
        return [Fraction(0)] * len(x)
    _, F = math.frexp(mx)
    return [Fraction(float(v)) / Fraction(2) ** (F + 2) for v in x]


def limbs(xs):
    """Four limbs per entry, each the remainder rounded to the nearest integer (ties to even), 7 bits apart."""
    out = []
    for v in xs:
        y = v * 256
        a = []
        for n in range(4):
            q = round(y)                      # Fraction rounds half to even
            a.append(int(q))
            y = (y - q) * 128
        out.append(a)
    return out


def approx_terms(xl, yl):
    """Per entry d, the ten limb products with n + m <= 5 (1-based), exactly; their sum over d is t."""
    out = []
    for a, b in zip(xl, yl):
        t = Fraction(0)
        for n in range(4):
            for m in range(4):
                if n + m <= 3:                # 0-based n + m <= 3  <=>  1-based n + m <= 5
                    t += Fraction(a[n] * b[m], 2 ** (16 + 7 * (n + m)))
        out.append(t)
    return out


def check(x, y):
    xs, ys = scaled(x), scaled(y)
    assert all(abs(v) < Fraction(1, 4) for v in xs + ys)
    xl, yl = limbs(xs), limbs(ys)
    assert all(abs(a) <= 64 for row in xl + yl for a in row)
    terms = approx_terms(xl, yl)
    for td, u, v in zip(terms, xs, ys):
        assert abs(td - u * v) < BOUND_PER_D
    exact = sum(a * b for a, b in zip(xs, ys))
    err = abs(sum(terms) - exact)
    assert err < BOUND, (float(err), float(BOUND))
    return err


@pytest.mark.parametrize("D", [64, 128])
def test_random_vectors(D):
    rng = np.random.Generator(np.random.PCG64(7 + D))
    worst = Fraction(0)
    for _ in range(40):
        scale = 2.0 ** rng.integers(-30, 4)
        x = rng.standard_normal(D) * scale
        y = rng.standard_normal(D) * 2.0 ** rng.integers(-30, 4)
        worst = max(worst, check(x, y))
    assert worst < BOUND / 8                  # typical errors sit far inside the bound


@pytest.mark.parametrize("D", [64, 128])
def test_entries_just_below_a_quarter(D):
    # every entry at the top of its binade: |x~| = 1/4 - ulp, remainders as large as the split allows
    v = math.nextafter(0.5, 0.0)
    for sx in (1.0, -1.0):
        x = np.full(D, v) * sx
        y = np.full(D, v)
        y[::2] *= -1
        check(x, y)
        check(x, np.full(D, v))


@pytest.mark.parametrize("D", [64, 128])
def test_remainders_on_rounding_ties(D):
    # entries whose scaled value is k + 1/2 units of some limb, so every rounding step ties
    rng = np.random.Generator(np.random.PCG64(99 + D))
    for _ in range(10):
        base = rng.integers(-63, 64, size=D).astype(np.float64)
        x = (base + 0.5) * 2.0 ** -8 + (rng.integers(-63, 64, size=D) + 0.5) * 2.0 ** -15
        x[0] = 0.2499                          # fixes the scale exponent: max |x| in [1/8, 1/4)
        y = (rng.integers(-63, 64, size=D) + 0.5) * 2.0 ** -22 + 0.24 * np.sign(rng.standard_normal(D))
        check(x * 2.0 ** -1, y * 2.0 ** 3)    # other binades: the split rescales them alike


def test_aligned_worst_case_signs():
    # choose y's signs to match the signs of x's dropped terms, so the per-entry errors add up
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.uniform(-0.5, 0.5, 128)
    x[0] = math.nextafter(0.5, 0.0)
    xs = scaled(x)
    xl = limbs(xs)
    rem = [v - sum(Fraction(a, 2 ** (8 + 7 * n)) for n, a in enumerate(row)) for v, row in zip(xs, xl)]
    y = np.array([math.nextafter(0.5, 0.0) * (1.0 if r >= 0 else -1.0) for r in rem])
    check(x, y)
