"""The step kernels' fp32 decision of stochastic rounding equals the exact definition.

For asymmetric rows on the refit fast path with |z| <= 255 the kernels decide
floor(h*inv + z + K/2^16) in fp32: A = 2^16 inv, Kz = K + 2^16 z (built as
(2^23 + K) + (2^16 z - 2^23)), v = fma(h, A, Kz), y = v/2^16, code = floor(y); an
entry whose v is a multiple of 2^16 is decided in double instead.  This models that
arithmetic with exact rationals (each fp32 operation the correctly rounded value of its
exact result) and checks it against the definition, over codes across the whole range,
zero points in [-255, 255], scales from 2^-60 to 2^60 and values aimed at code
boundaries.  Host arithmetic only; no GPU.
"""
import math
import random
from fractions import Fraction

import numpy as np


def rn32(x: Fraction) -> float:
    """x rounded to the nearest fp32 (ties to even), subnormals included."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = a / Fraction(2) ** (e - 23)
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n) * 2.0 ** (e - 23)


def f32(x: float) -> float:
    return float(np.float32(x))


def decide_fp32(h, inv, z, K):
    """(code before the clamp, whether the entry goes to the double decision)"""
    A = f32(inv * 65536.0)
    zk = f32(z * 65536.0 - 8388608.0)
    kf = float(np.array([K | 0x4B000000], np.uint32).view(np.float32)[0])
    Kz = f32(kf + zk)
    assert Kz == K + 65536 * z  # exact
    v = rn32(Fraction(h) * Fraction(A) + Fraction(Kz))
    y = f32(v / 65536.0)
    m = math.floor(y)
    return m, y == m


def exact_code(h, inv, z, K):
    return math.floor(Fraction(h) * Fraction(inv) + z + Fraction(K, 65536))


def test_fp32_decision_matches_the_definition():
    rng = random.Random(7)
    edges = wrong_at_edges = 0
    for _ in range(6000):
        bits = rng.choice([4, 8])
        qa = (1 << bits) - 1
        z = rng.randint(-255, 255)
        inv = f32(rng.uniform(0.5, 2.0) * 2.0 ** rng.randint(-60, 60))
        K = rng.randint(0, 65535)
        if rng.random() < 0.5:
            # aim h*inv + z + K/2^16 at an integer code, exactly or just beside it
            c = rng.randint(-1, qa + 1)
            t = c - z - K / 65536.0 + rng.choice([0.0, 0.0, 1e-7, -1e-7, 2.0 ** -30, -(2.0 ** -30)])
        else:
            t = rng.uniform(-z - 0.5, qa - z + 0.5)
        t = min(max(t, -z - 0.5), qa - z + 0.5)  # the fast path's range of h*inv
        h = f32(t / inv)
        m, edge = decide_fp32(h, inv, z, K)
        want = exact_code(h, inv, z, K)
        if edge:
            edges += 1
            wrong_at_edges += m != want
            continue  # decided in double, which is exact
        assert min(max(m, 0), qa) == min(max(want, 0), qa), (h, inv, z, K)
    # the double decision is needed: some multiples of 2^16 hide a code one lower
    assert edges > 100 and wrong_at_edges > 0
