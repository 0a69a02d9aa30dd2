"""The dequantize kernel builds its table (q/127 or q/255, then the softsign
inverse y / (2 - |y|), dequantize() on page "code/flashsim/quantization.py")
with multiplies and FMAs only: a Markstein correction of q R for the
quotient by a constant, and a Newton reciprocal of 2 - |y| followed by the
same correction for the softsign inverse.  This test
evaluates every rounding of those sequences exactly (rational arithmetic,
fp32 round-to-nearest-even; an FMA rounds once) for every code of the
signed and unsigned specs, with the constants read from the kernel source,
and requires the correctly rounded quotient each time, which is what
dequantize() computes in fp32.  (The GPU codec tests compare the kernel's
tables with the oracle on every code as well; the step kernels load
compile-time constants of the same entries.)"""
import os
import re
from fractions import Fraction as Fr

import numpy as np

SRC = os.path.join(os.path.dirname(__file__), "..", "bit_companded_adam_amd", "csrc",
                   "flashopt_kernels.hip")


def rn(x: Fr) -> Fr:
    """x rounded to the nearest fp32 value, ties to even (normal range and
    subnormals; the values here are far from overflow)."""
    if x == 0:
        return Fr(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    ulp = Fr(2) ** (max(e, -126) - 23)
    q = a / ulp
    f, rem = divmod(q.numerator, q.denominator)
    rem = Fr(rem, q.denominator)
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and f % 2 == 1):
        f += 1
    return sign * f * ulp


def fma(a, b, c):
    return rn(a * b + c)


def _constants():
    src = open(SRC).read()
    lin0 = float.fromhex(re.search(r"kRecipLin0 = (0x[0-9a-fp.+-]+)f;", src).group(1))
    lin1 = float.fromhex(re.search(r"kRecipLin1 = (0x[0-9a-fp.+-]+)f;", src).group(1))
    steps = int(re.search(r"kRecipSteps = (\d+);", src).group(1))
    return Fr(lin0), Fr(lin1), steps


def _quotient(q: Fr, d: Fr) -> Fr:
    r = rn(1 / d)                       # the constant 1/D, rounded once at compile time
    y0 = rn(q * r)
    return fma(fma(-d, y0, q), r, y0)


def _softsign_inverse(y: Fr, lin0: Fr, lin1: Fr, steps: int) -> Fr:
    den = rn(2 - abs(y))
    h = rn(den / 2)                     # exact: den is a normal number
    x = fma(-lin1, h, lin0)
    for _ in range(steps):
        x = fma(x, fma(-h, x, Fr(1)), x)
    x = rn(x / 2)
    z0 = rn(y * x)
    return fma(fma(-den, z0, y), x, z0)


def test_constants_are_the_rounded_fractions():
    lin0, lin1, steps = _constants()
    assert lin0 == rn(Fr(48, 17)) and lin1 == rn(Fr(32, 17))
    assert steps >= 1


def test_quotients_by_127_and_255_are_correctly_rounded():
    for d, codes in ((127, range(-128, 128)), (255, range(256))):
        for c in codes:
            assert _quotient(Fr(c), Fr(d)) == rn(Fr(c, d)), (c, d)


def test_softsign_inverse_is_correctly_rounded():
    lin0, lin1, steps = _constants()
    for c in range(-128, 128):
        y = rn(Fr(c, 127))
        want = rn(y / rn(2 - abs(y)))
        assert _softsign_inverse(y, lin0, lin1, steps) == want, c


def test_a_planted_error_is_caught():
    """A sequence without the correction step (y0 = q R alone) is wrong on
    some codes, so the checks above can fail."""
    bad = [c for c in range(256) if rn(Fr(c) * rn(Fr(1, 255))) != rn(Fr(c, 255))]
    assert bad
    lin0, lin1, _ = _constants()
    wrong = [c for c in range(-128, 128)
             if _softsign_inverse(rn(Fr(c, 127)), lin0, lin1, 0) != rn(rn(Fr(c, 127)) / rn(2 - abs(rn(Fr(c, 127)))))]
    assert wrong


def test_fp32_rounding_helper_matches_numpy():
    rng = np.random.default_rng(5)
    for x in rng.standard_normal(200):
        assert rn(Fr(float(x))) == Fr(float(np.float32(x)))
