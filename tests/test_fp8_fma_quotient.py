"""The blockwise fp8 quantisers take RN(v / s) as one FMA correction of
RN(v * RN(1 / s)): with rs = RN(1/s) and q = RN(v rs), RN(q + RN(v - q s) rs)
is the rounded quotient (Markstein's theorem on FMA-based division) unless
the residual v - q s underflows.  The kernels use it for |v| >= 2^-100 with
rs finite, and divide otherwise.  Checked here in exact rational arithmetic
on float32 values: random and structured scales and values, values next to
e4m3 rounding midpoints, scales with all-ones and all-zeros mantissas, and
magnitudes near the guard.  CPU only."""
from fractions import Fraction

import numpy as np


def rn32(x: Fraction) -> float:
    """x rounded to the nearest float32, ties to even (integer arithmetic)."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    e = max(e, -126)
    q = x / Fraction(2) ** (e - 23)
    n, r = divmod(q.numerator, q.denominator)
    rem = Fraction(r, q.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(np.float32(n * 2.0 ** (e - 23)))


def f32(x) -> float:
    return float(np.float32(x))


def fma_quotient(v: float, s: float) -> float:
    rs = rn32(Fraction(1) / Fraction(s))
    q = f32(np.float32(v) * np.float32(rs))
    if v == 0.0:
        return q
    r = rn32(Fraction(v) - Fraction(q) * Fraction(s))
    return rn32(Fraction(q) + Fraction(r) * Fraction(rs))


def _cases(rng, n):
    for t in range(n):
        kind = t % 5
        if kind == 0:      # amax / 448 scales, values inside the block's range
            amax = f32(abs(rng.standard_normal()) * 2.0 ** int(rng.integers(-40, 40)) + 1e-30)
            s = f32(np.float32(amax) / np.float32(448.0))
            v = f32(rng.uniform(-1, 1) * amax)
        elif kind == 1:    # random float32 bit patterns
            s = float(np.uint32(rng.integers(0x00800000, 0x7E800000)).view(np.float32))
            v = float(np.uint32(rng.integers(0, 0x7F000000)).view(np.float32)) * (1 if rng.random() < .5 else -1)
            if not 1e-37 < abs(v / s) < 1e38:
                continue
        elif kind == 2:    # scale mantissas near all ones or all zeros
            m = 0x7FFFFF - int(rng.integers(0, 16)) if rng.random() < .5 else int(rng.integers(0, 16))
            s = float(np.uint32((int(rng.integers(60, 190)) << 23) | m).view(np.float32))
            v = f32(s * f32(rng.uniform(-448, 448)))
        elif kind == 3:    # next to an e4m3 rounding midpoint of v / s
            s = f32(rng.uniform(1e-3, 1e3))
            mid = f32(int(rng.integers(-448, 448)) + 0.5 * 2.0 ** int(rng.integers(-3, 1)))
            v = float(np.nextafter(np.float32(mid * s), np.float32(np.inf if rng.random() < .5 else -np.inf)))
        else:              # small magnitudes just above the guard, tiny scales
            s = f32(2.0 ** rng.uniform(-120, 0))
            v = f32(2.0 ** rng.uniform(-100, -60)) * (1 if rng.random() < .5 else -1)
        if abs(v) < 2.0 ** -100 and v != 0.0:
            continue
        if abs(rn32(Fraction(1) / Fraction(s))) == float("inf"):
            continue
        yield v, s


def test_fma_quotient_is_the_rounded_quotient():
    rng = np.random.default_rng(2024)
    n = 0
    for v, s in _cases(rng, 4000):
        assert fma_quotient(v, s) == rn32(Fraction(v) / Fraction(s)), (v, s)
        n += 1
    assert n > 3000


def test_signed_zero_is_kept():
    assert np.signbit(fma_quotient(-0.0, 0.125)) and not np.signbit(fma_quotient(0.0, 0.125))


def test_guard_is_needed_below_it():
    """Below 2^-100 the residual underflows and one correction is not enough:
    a value the kernels therefore divide."""
    v, s = -4.822013750781985e-38, 0.03394550457596779
    v, s = f32(v), f32(s)
    assert abs(v) < 2.0 ** -100
    assert fma_quotient(v, s) != rn32(Fraction(v) / Fraction(s))
