"""The delta kernels' u accumulation with codes read as subnormal doubles rounds exactly as
the plain accumulation does.

For unsigned codes the kernels form sum_i kap_i*c_ij as fma(kap_i*2^P, c*2^-1074, acc) with
acc started at -zt*2^-(1074-P) and scale the finished column sum back by 2^(1074-P).  The
claim is that every rounding then equals the plain fma(kap_i, c, acc) rounding, one power of
two lower, for every finite input.  This checks it with exact rational arithmetic (each fma
is the correctly rounded value of an exact sum) over kap drawn across the whole fp32 range,
including subnormal fp32 factors, for the scalar rule (kap = k*s) and the KDA rule
(kap = (k*alpha)*s rounded once).  Host arithmetic only; no GPU.
"""
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "mamba_decode_amd", "csrc", "ssq_delta.hip")
m = re.search(r"kSubScale = 0x1p(\d+), kSubUnscale = 0x1p(\d+);", open(SRC).read())
P, UNSCALE = int(m.group(1)), int(m.group(2))


def fma(a: float, b: float, c: float) -> float:
    """Correctly rounded a*b + c (int / int true division rounds correctly, subnormals too)."""
    x = Fraction(a) * Fraction(b) + Fraction(c)
    return x.numerator / x.denominator


def rand_f32(rng, n, emin=-149, emax=127):
    """fp32 values with uniformly drawn binary exponents (subnormals included), random sign."""
    e = rng.integers(emin, emax + 1, n)
    mant = rng.integers(0, 1 << 23, n)
    v = np.where(e < -126, mant * 2.0 ** -149, (1.0 + mant / 2.0 ** 23) * np.ldexp(1.0, np.maximum(e, -126)))
    v = np.where(rng.random(n) < 0.5, -v, v).astype(np.float32)
    assert np.all(np.isfinite(v))
    return v


def accumulate(kaps, zs, codes):
    """(plain, scaled) column sums over 32 row groups of 4 rows, as the kernels order them."""
    plain_parts, scaled_parts = [], []
    for g in range(kaps.shape[0]):
        zt = 0.0
        for r in range(4):
            zt = fma(float(kaps[g, r]), float(zs[g, r]), zt)
        up, us = -zt, -zt * 2.0 ** -UNSCALE
        assert us * 2.0 ** UNSCALE == up
        for r in range(4):
            kap = float(kaps[g, r])
            up = fma(kap, float(codes[g, r]), up)
            us = fma(kap * 2.0 ** P, math.ldexp(int(codes[g, r]), -1074), us)
            assert us * 2.0 ** UNSCALE == up, (g, r, kap, int(codes[g, r]))
        plain_parts.append(up)
        scaled_parts.append(us)
    ap, asc = 0.0, 0.0
    for a, b in zip(plain_parts, scaled_parts):
        ap += a
        asc += b
    return ap, asc


def test_scaling_constants_leave_room():
    # kap < 2^384 (three fp32 factors) stays finite after the 2^P scaling, and a multiple of
    # 2^-447 stays in the normal range after the 2^-(1074-P) scaling
    assert 384 + P < 1024
    assert -447 - UNSCALE >= -1022
    assert P - 1074 == -UNSCALE


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("ranges", ["unit", "wide"])
def test_scaled_accumulation_equals_plain(kda, bits, ranges):
    rng = np.random.default_rng(1000 * bits + 10 * kda + (ranges == "wide"))
    for case in range(6):
        n = 32 * 4
        if ranges == "unit":
            k = rand_f32(rng, n, -12, 0)
            s = rand_f32(rng, n, -16, -2)
            a = rand_f32(rng, n, -3, -1)
        else:
            k = rand_f32(rng, n)
            s = rand_f32(rng, n)
            a = rand_f32(rng, n)
        kd = k.astype(np.float64) * a.astype(np.float64) if kda else k.astype(np.float64)
        kaps = (kd * s.astype(np.float64)).reshape(32, 4)  # one rounding for KDA, exact otherwise
        qa = (1 << bits) - 1
        codes = rng.integers(0, qa + 1, (32, 4))
        zs = rng.integers(0, qa + 1, (32, 4)).astype(np.float64)
        if case == 0:
            codes[:] = qa  # largest products
        if case == 1:
            codes[::2] = 0  # zero codes: the subnormal operand is +0
        plain, scaled = accumulate(kaps, zs, codes)
        assert scaled * 2.0 ** UNSCALE == plain


def test_extreme_factors():
    """Every factor at the ends of the fp32 range at once."""
    tiny, huge = np.float32(2.0 ** -149), np.float32(np.finfo(np.float32).max)
    for k, a, s in [(tiny, tiny, tiny), (huge, huge, huge), (tiny, huge, tiny), (huge, tiny, huge)]:
        kap = float(np.float64(k) * np.float64(a) * np.float64(s))
        kaps = np.full((32, 4), kap)
        kaps[1::2] = -kap
        codes = np.arange(128).reshape(32, 4) % 256
        zs = np.full((32, 4), 7.0)
        plain, scaled = accumulate(kaps, zs, codes)
        assert scaled * 2.0 ** UNSCALE == plain
