"""The oracle's fixed fp32 exponential and silu, pinned bit for bit to their
stated programs.

The programs (the library header and the oracle's comments state them): the
Cody & Waite range reduction (Cody & Waite, "Software Manual for the
Elementary Functions", 1980) with n = rint(fp32(x * fp32(1/ln 2))), ln 2 split
into its first 15 significant bits and the fp32 rounding of the rest, the
degree-7 Taylor polynomial with fp32-rounded 1/i! coefficients by Horner's
rule with fused multiply-adds, then p * 2^n; inputs clamped to [-104, 89].
silu(g) = g / (1 + exp(-g)).

Here each step is evaluated in exact rational arithmetic and rounded once to
binary32 (round to nearest, ties to even, subnormals kept), as IEEE 754
defines each operation, with ln 2 from Python's decimal module to 60 digits.
A different program in the oracle (another polynomial degree, a non-fused
Horner step, other constants, a different rounding of n) changes some of the
10^4 results.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle

getcontext().prec = 60
LN2 = Fraction(str(Decimal(2).ln()))
F32_MAX = Fraction((2 ** 24 - 1) * 2 ** 104)


def rnd32(q: Fraction) -> Fraction:
    """The binary32 value nearest to q (ties to even; subnormals; overflow -> inf)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                  # 2^e <= a < 2^(e+1)
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    M = m.numerator // m.denominator
    rem = m - M
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and M % 2 == 1):
        M += 1
    v = M * quantum
    if v > F32_MAX:
        return Fraction(sign) * Fraction(10) ** 400   # stands for +-inf
    return sign * v


def to_f32(q: Fraction) -> np.float32:
    if abs(q) > F32_MAX:
        return np.float32(np.inf if q > 0 else -np.inf)
    return np.float32(float(q))                # exact: q is a binary32 value


def rint_even(q: Fraction) -> Fraction:
    f = q.numerator // q.denominator
    rem = q - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return Fraction(f)


L2E = rnd32(1 / LN2)
HI = Fraction(math.floor(LN2 * 2 ** 15), 2 ** 15)          # 15 significant bits: 2^-1 .. 2^-15
LO = rnd32(LN2 - HI)
COEF = [rnd32(Fraction(1, math.factorial(i))) for i in range(8)]


def exp_program(x: float) -> np.float32:
    xq = Fraction(float(np.float32(x)))
    xq = min(max(xq, Fraction(-104)), Fraction(89))
    n = rint_even(rnd32(xq * L2E))
    r = rnd32(-n * HI + xq)                     # fused: one rounding
    r = rnd32(-n * LO + r)
    p = COEF[7]
    for i in range(6, -1, -1):
        p = rnd32(p * r + COEF[i])              # fused multiply-add
    return to_f32(rnd32(p * Fraction(2) ** int(n)))


def silu_program(g: float) -> np.float32:
    gq = Fraction(float(np.float32(g)))
    ex = exp_program(float(-gq))
    if np.isinf(ex):
        return np.float32(-0.0) if gq < 0 else np.float32(0.0)
    den = rnd32(1 + Fraction(float(ex)))
    return to_f32(rnd32(gq / den))


def test_constants_are_the_stated_ones():
    assert HI * 2 ** 15 == int(HI * 2 ** 15) and HI < LN2 < HI + Fraction(1, 2 ** 15)
    # n * HI is exact in fp32 for |n| < 2^9 (15 + 9 bits)
    assert all(rnd32(n * HI) == n * HI for n in range(-200, 200))
    assert float(L2E) == float(np.float32(1 / math.log(2)))


def _points(n=10_000):
    rng = np.random.default_rng(7)
    pts = [rng.uniform(-110.0, 95.0, n // 2).astype(np.float32),
           rng.uniform(-1.0, 1.0, n // 4).astype(np.float32),
           # inputs near the rounding boundaries of n = rint(x / ln 2)
           ((np.arange(-150, 130) + 0.5) * math.log(2)).astype(np.float32),
           np.array([0.0, -0.0, 1e-30, -1e-30, 89.0, 88.72, -87.33, -103.9, -104.0, -1000.0, 200.0],
                    np.float32)]
    pts = np.concatenate(pts)
    return pts[:n]


def test_exp_p_is_the_stated_program_bit_for_bit():
    xs = _points()
    got = oracle.exp_p(xs).astype(np.float32)
    want = np.array([exp_program(float(x)) for x in xs], dtype=np.float32)
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, "first mismatches: %s" % [(float(xs[i]), float(got[i]), float(want[i])) for i in bad[:5]]


def test_silu_p_is_the_stated_program_bit_for_bit():
    rng = np.random.default_rng(11)
    gs = np.concatenate([rng.uniform(-40.0, 40.0, 9_000).astype(np.float32),
                         rng.standard_normal(1_000).astype(np.float32)])
    got = oracle.silu_p(gs).astype(np.float32)
    want = np.array([silu_program(float(g)) for g in gs], dtype=np.float32)
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, "first mismatches: %s" % [(float(gs[i]), float(got[i]), float(want[i])) for i in bad[:5]]


def _variant(x, fused=True, degree=7, hi_bits=15):
    xq = Fraction(float(np.float32(x)))
    xq = min(max(xq, Fraction(-104)), Fraction(89))
    hi = Fraction(math.floor(LN2 * 2 ** hi_bits), 2 ** hi_bits)
    lo = rnd32(LN2 - hi)
    n = rint_even(rnd32(xq * L2E))
    r = rnd32(-n * hi + xq)
    r = rnd32(-n * lo + r)
    p = COEF[degree]
    for i in range(degree - 1, -1, -1):
        p = rnd32(p * r + COEF[i]) if fused else rnd32(rnd32(p * r) + COEF[i])
    return to_f32(rnd32(p * Fraction(2) ** int(n)))


@pytest.mark.parametrize("kw", [dict(fused=False), dict(degree=6), dict(hi_bits=14)],
                         ids=["unfused_horner", "degree6", "ln2_split_14_bits"])
def test_the_pin_separates_plausible_other_programs(kw):
    # each of these mistakes, made in the oracle, would change some of the
    # pinned points (a check of the pin's power, on a subset of its points)
    xs = _points()[::5]
    diff = sum(int(_variant(float(x), **kw) != exp_program(float(x))) for x in xs)
    assert diff > 0
