"""The step kernels' fp32 decision of stochastic rounding equals the exact definition.

For rows on the refit fast path with inv <= 2^100 the kernels decide
floor(h*inv + z + K/2^16) in fp32 with the rounding mode set toward -infinity (RD):
A = 2^16 inv, v = RD(h*A + (2^23 + K)) by one fma, f = RD(v*2^-16 + (1.5*2^23 + z - 128))
by another, code = f - 1.5*2^23.  This models that arithmetic with exact rationals (each
operation the value of its exact result rounded down to fp32) and checks it against the
definition over codes across the whole range, zero points far beyond the code range (0 for
the symmetric grid), scales from 2^-60 to 2^60 and up to the 2^100 bound, and values aimed
at code boundaries, exactly on them included.  It also checks that rounding to nearest in
the same two operations would be wrong at such boundaries, which is what the mode switch
is for.  Host arithmetic only; no GPU.
"""
import math
import random
from fractions import Fraction

import numpy as np

MAGIC = 1.5 * 2.0 ** 23


def round32(x: Fraction, down: bool) -> float:
    """x rounded to fp32 (toward -infinity, or to nearest with ties to even), subnormals
    included."""
    if x == 0:
        return 0.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = x / Fraction(2) ** (e - 23)  # signed, in ulps
    n = math.floor(q)
    if not down:
        r = q - n
        if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
            n += 1
    return float(n) * 2.0 ** (e - 23)


def f32(x: float) -> float:
    return float(np.float32(x))


def decide(h, inv, z, K, down=True):
    """The code the kernels' two fp32 operations give (before the clamp)."""
    A = f32(inv * 65536.0)
    assert A == inv * 65536.0
    kf = float(np.array([K | 0x4B000000], np.uint32).view(np.float32)[0])
    assert kf == 2.0 ** 23 + K
    mz = f32(f32(MAGIC + z) - 128.0)
    assert mz == MAGIC + z - 128  # exact
    v = round32(Fraction(h) * Fraction(A) + Fraction(kf), down)
    f = round32(Fraction(v) / 65536 + Fraction(mz), down)
    return f - MAGIC


def exact_code(h, inv, z, K):
    return math.floor(Fraction(h) * Fraction(inv) + z + Fraction(K, 65536))


def test_fp32_decision_matches_the_definition():
    rng = random.Random(7)
    on_boundary = nearest_wrong = 0
    for i in range(6000):
        bits = rng.choice([4, 8])
        sym = rng.random() < 0.25
        qa = (1 << bits) - 1
        lo, hi = (-(qa // 2), qa // 2) if sym else (0, qa)
        z = 0 if sym else rng.choice([rng.randint(-255, 255), rng.randint(-(2 ** 20), 2 ** 20)])
        inv_exp = rng.randint(-60, 60) if i % 10 else rng.randint(90, 99)
        inv = f32(rng.uniform(0.5, 2.0) * 2.0 ** inv_exp)
        K = rng.randint(0, 65535)
        if rng.random() < 0.5:
            # aim h*inv + z + K/2^16 at an integer code, exactly or just beside it
            c = rng.randint(lo - 1, hi + 1)
            t = c - z - K / 65536.0 + rng.choice([0.0, 0.0, 1e-7, -1e-7, 2.0 ** -30, -(2.0 ** -30)])
        else:
            t = rng.uniform(lo - z - 0.5, hi - z + 0.5)
        t = min(max(t, lo - z - 0.5), hi - z + 0.5)  # the fast path's range of h*inv
        h = f32(t / inv)
        want = exact_code(h, inv, z, K)
        got = decide(h, inv, z, K)
        assert min(max(got, lo), hi) == min(max(want, lo), hi), (h, inv, z, K)
        x = Fraction(h) * Fraction(inv) + z + Fraction(K, 65536)
        if x == math.floor(x) or (x - math.floor(x)) * 2 ** 24 < 1 or (math.ceil(x) - x) * 2 ** 24 < 1:
            on_boundary += 1
            near = decide(h, inv, z, K, down=False)
            nearest_wrong += min(max(near, lo), hi) != min(max(want, lo), hi)
    # the boundary cases are exercised, and rounding to nearest would get some of them wrong
    assert on_boundary > 100 and nearest_wrong > 0, (on_boundary, nearest_wrong)
