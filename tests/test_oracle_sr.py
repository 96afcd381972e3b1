"""Pins of the oracle's stochastic rounding (CPU only).

Stochastic rounding of the state is the alternative to round-to-nearest that
the "ssm-state-quantization" README tests in Findings 9.  The pages name it
only, so the plain textbook definition is used: the code is floor(v + U) for
the exact real v = h*inv + z and a uniform U in [0, 1), i.e. the row rounds up
with probability equal to the fractional part of v; the grid (scale and zero
point) is the one round-to-nearest refits.  U is a 16-bit uniform, a multiple of
2^-16: counter ctr = (step*rows + row)*N + n takes bits 16k .. 16k+15 (k = ctr
mod 4) of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) output number
ctr/4 + 1 for the state's seed, four uniforms per output.

The pins: the generator's published output sequence and how its outputs split
into uniforms; the uniforms' distribution; hand-worked rows; every code is
floor(v + U) computed in exact rational arithmetic, down to values a hair below
zero; the mean code over many draws is the exact value up to the 2^-16 grid of U
(unbiasedness); values on the grid are kept; and the decode step, scan and delta
step draw the uniforms of the rows and tokens they update.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

F64 = np.float64
QUANT = ["int8_sym", "int8_asym", "int4_sym", "int4_asym"]


def test_splitmix64_published_sequence():
    # the first outputs of SplitMix64 started at state 0, as printed by the
    # generator's reference implementation
    assert oracle.splitmix64(0, 1) == 0xE220A8397B1DCDAF
    assert oracle.splitmix64(0, 2) == 0x6E789E6AA1B965F4
    assert oracle.splitmix64(0, 3) == 0x06C45D188009454F
    # counters 0..3 take the four 16-bit pieces of output number 1, low piece first;
    # counters 4..7 those of output number 2, and so on
    pieces = [0xCDAF, 0x7B1D, 0xA839, 0xE220, 0x65F4, 0xA1B9, 0x9E6A, 0x6E78, 0x454F, 0x8009, 0x5D18, 0x06C4]
    for ctr, piece in enumerate(pieces):
        assert oracle.sr_uniform(0, 0, 1, 0, 12, ctr) == piece / 2.0 ** 16


def test_uniforms_are_16_bit_and_uniform():
    n = 1 << 16
    u = oracle.sr_row_uniforms(7, 3, 1000, 11, n).astype(F64)
    assert u[12345] == oracle.sr_uniform(7, 3, 1000, 11, n, 12345)
    assert np.all(u >= 0.0) and np.all(u < 1.0)
    assert np.array_equal(u * 2.0 ** 16, np.floor(u * 2.0 ** 16))  # 16-bit fractions
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / n)
    counts = np.bincount((u * 16).astype(int), minlength=16)
    chi2 = ((counts - n / 16) ** 2 / (n / 16)).sum()
    assert chi2 < 60.0  # 15 degrees of freedom: p < 1e-6 above 60


def test_uniforms_follow_the_flat_counter():
    # token `step`, row r, entry n use counter (step*rows + r)*N + n: consecutive
    # tokens and rows continue one flat sequence, and different seeds differ
    rows, N = 5, 8
    assert oracle.sr_uniform(1, 1, rows, 0, N, 0) == oracle.sr_uniform(1, 0, rows, rows, N, 0)
    assert oracle.sr_uniform(1, 0, rows, 1, N, 0) == oracle.sr_uniform(1, 0, rows, 0, N, N)
    assert oracle.sr_uniform(1, 0, rows, 0, N, 0) != oracle.sr_uniform(1, 1, rows, 0, N, 0)
    assert oracle.sr_uniform(1, 0, rows, 0, N, 0) != oracle.sr_uniform(2, 0, rows, 0, N, 0)


def _grid16(u):
    return np.round(np.asarray(u, F64) * 65536) / 65536


def test_hand_worked_rows():
    # asymmetric 2-bit grid over [0, 3]: s = 1, z = 0, so v = h
    h = np.array([0.0, 3.0, 1.25, 1.25, 2.5, 2.5], np.float32)
    U = _grid16([0.9, 0.9, 0.74, 0.76, 0.49, 0.51])
    code2, s2, z2 = _q(h, 2, 1, U)
    assert (s2, z2) == (1.0, 0.0)
    # floor(v + U): 0.9 -> 0, 3.9 -> 3, 1.99 -> 1, 2.01 -> 2, 2.99 -> 2, 3.01 -> 3
    assert code2.tolist() == [0, 3, 1, 2, 2, 3]
    # symmetric 2-bit grid: amax 2, step 2, v = h/2 in [-1, 1]
    h = np.array([-2.0, 2.0, -1.0, -1.0, 0.5, 0.5], np.float32)
    U = _grid16([0.3, 0.3, 0.49, 0.51, 0.74, 0.76])
    code3, s3, z3 = _q(h, 2, 0, U)
    assert (s3, z3) == (2.0, 0.0)
    # v = -1, 1, -0.5, -0.5, 0.25, 0.25 -> floor(v + U)
    assert code3.tolist() == [-1, 1, -1, 0, 0, 1]
    # symmetric 8-bit grid with amax 127: s = 1, v = h.  A value a hair below zero
    # rounds down to -1 only when U = 0; a hair below 3 reaches 3 once U >= 2^-16
    h = np.array([127.0, -1e-30, -1e-30, -1e-30, np.nextafter(np.float32(3), np.float32(0)),
                  np.nextafter(np.float32(3), np.float32(0)), -127.0], np.float32)
    U = np.array([0.0, 0.0, 2.0 ** -16, 1 - 2.0 ** -16, 0.0, 2.0 ** -16, 0.0])
    code8, s8, z8 = _q(h, 8, 0, U)
    assert (s8, z8) == (1.0, 0.0)
    assert code8.tolist() == [127, -1, 0, 0, 2, 3, -127]
    with pytest.raises(ValueError):
        oracle.quantize_row_sr(np.ones(4, np.float32), "int8_sym", np.full(4, 0.3))  # off the 2^-16 grid


def _q(h, bits, asym, U):
    h = np.ascontiguousarray(h, np.float32)
    n = h.shape[0]
    code = np.empty(n, np.int32)
    s = np.empty(1, np.float32)
    z = np.empty(1, np.float32)
    oracle.lib().orc_quantize_row_sr(oracle._f(h), n, bits, asym, oracle._i(code), oracle._f(s),
                                     oracle._f(z), None, oracle._f(np.ascontiguousarray(U, np.float32)))
    return code, float(s[0]), float(z[0])


def _rows():
    h = synth.init_state(21, 1, 24, 128)
    r = synth.normal(21, 98, 0, np.arange(4 * 128)).reshape(4, 128)
    tiny = 1e-12 * r[:1]  # values a hair either side of zero
    # the last row's offset is huge against its spread: |z| ~ 2^29
    return np.concatenate([h, 10.0 + 1e-2 * r, -3.0 + 1e-3 * r, tiny, 1000.0 + 1e-4 * r[:1]]).astype(np.float32)


def _floor_exact(h, inv, z, U):
    """floor(h*inv + z + U) per entry, in exact rational arithmetic."""
    fi = Fraction(float(inv))
    return np.array([math.floor(Fraction(float(a)) * fi + int(z) + Fraction(float(u))) for a, u in zip(h, U)],
                    np.int64)


@pytest.mark.parametrize("fmt", QUANT)
def test_codes_bracket_the_exact_value_and_keep_the_grid(fmt):
    bits, asym = oracle.FORMATS[fmt]
    lo, hi = (0, (1 << bits) - 1) if asym else (-((1 << (bits - 1)) - 1), (1 << (bits - 1)) - 1)
    for i, h in enumerate(_rows()):
        U = oracle.sr_row_uniforms(5, 2, 99, i, 128)
        c_rtn, s_rtn, z_rtn = oracle.quantize_row_sr(h, fmt, None)
        c, s, z = oracle.quantize_row_sr(h, fmt, U)
        assert (s, z) == (s_rtn, z_rtn)          # the grid does not depend on the rounding
        assert s >= np.finfo(np.float32).tiny  # no degenerate row here
        inv = np.float32(1.0) / np.float32(s)
        ref = np.clip(_floor_exact(h, inv, z, U), lo, hi)
        assert np.array_equal(c, ref), (fmt, i)


@pytest.mark.parametrize("fmt", QUANT)
def test_stochastic_rounding_is_unbiased(fmt):
    # one row drawn 4096 times with fresh uniforms: entry v rounds up with probability
    # floor(2^16 frac(v))/2^16, within 2^-16 of frac(v); the mean code follows it
    h = synth.init_state(23, 1, 1, 128)[0].astype(np.float32)
    c0, s, z = oracle.quantize_row_sr(h, fmt, None)
    inv = np.float32(1.0) / np.float32(s)
    v = h.astype(F64) * F64(inv) + F64(z)
    bits, asym = oracle.FORMATS[fmt]
    hi = (1 << bits) - 1 if asym else (1 << (bits - 1)) - 1
    inside = (v > (0 if asym else -hi)) & (v < hi)  # no clamping in play
    draws = 4096
    total = np.zeros(128, F64)
    for t in range(draws):
        U = oracle.sr_row_uniforms(3, t, 1, 0, 128)
        total += oracle.quantize_row_sr(h, fmt, U)[0]
    mean = total / draws
    frac = v - np.floor(v)
    p_up = np.floor(frac * 65536) / 65536
    assert np.all(np.abs(np.floor(v) + p_up - v) < 2.0 ** -16)
    sd = np.sqrt(p_up * (1 - p_up) / draws)
    assert np.all(np.abs(mean - (np.floor(v) + p_up))[inside] <= 5 * sd[inside] + 1e-12)


@pytest.mark.parametrize("fmt", QUANT)
def test_values_on_the_grid_are_kept(fmt):
    # a dequantized row lies on its own grid: stochastic rounding returns its codes
    h = synth.init_state(25, 1, 4, 128).astype(np.float32)
    code, s, z = oracle.quantize_rows(h, fmt)
    r = oracle.dequantize_rows(code, s, z)
    for i in range(4):
        U = oracle.sr_row_uniforms(9, 0, 4, i, 128)
        c_rtn, s_rtn, z_rtn = oracle.quantize_row_sr(r[i], fmt, None)
        c_sr, s_sr, z_sr = oracle.quantize_row_sr(r[i], fmt, U)
        if np.array_equal(c_rtn, code[i]):  # the row's extremes survived dequantization
            assert np.array_equal(c_sr, c_rtn)


def _uniforms(seed, step, rows, ids, N=128):
    return np.stack([oracle.sr_row_uniforms(seed, step, rows, r, N) for r in ids])


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_sym"])
def test_decode_step_and_scan_draw_their_rows_uniforms(fmt):
    B, H, G, P, T, N = 1, 2, 1, 4, 3, 128
    rows = B * H * P
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(13, 0, B, T, H, G, P, N)
    init = synth.init_state(13, 0, rows, N)
    seed, step0 = 77, 5
    # decode steps by hand: the pre-rounding rows quantized with the uniforms of (row, step)
    st = oracle.make_state(fmt, rows, N, init)
    ref = st.copy()
    for t in range(T):
        y, hpre, _ = oracle.mamba2_step(st, x[:, t], dt[:, t], A, Bm[:, t], Cm[:, t], D, diag=True,
                                        sr=(seed, step0 + t))
        U = _uniforms(seed, step0 + t, rows, range(rows))
        for r in range(rows):
            c, s, z = oracle.quantize_row_sr(hpre[r], fmt, U[r])
            assert np.array_equal(st.code[r], c) and st.scale[r] == s and st.zero[r] == z
    # the scan uses step0 + t for token t
    ysc = oracle.mamba2_scan(ref, x, dt, A, Bm, Cm, D, sr=(seed, step0))
    assert np.array_equal(ref.code, st.code) and np.array_equal(ref.scale, st.scale)
    assert np.isfinite(ysc).all()


def test_rows_scan_uses_the_state_row_ids():
    B, H, G, P, T, N = 1, 2, 1, 4, 2, 128
    rows = B * H * P
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(14, 0, B, T, H, G, P, N)
    init = synth.init_state(14, 0, rows, N)
    full = oracle.make_state("int8_asym", rows, N, init)
    oracle.mamba2_scan(full, x, dt, A, Bm, Cm, D, sr=(3, 11))
    ids = np.array([5, 2], np.int64)
    sub = oracle.make_state("int8_asym", 2, N, init[ids])
    hh = ids // P
    xr = np.ascontiguousarray(x[0][:, hh, ids % P].T)
    dtr = np.ascontiguousarray(dt[0][:, hh].T)
    Br = np.ascontiguousarray(np.repeat(Bm[0][None, :, 0], 2, axis=0))
    Cr = np.ascontiguousarray(np.repeat(Cm[0][None, :, 0], 2, axis=0))
    oracle.mamba2_rows_scan(sub, xr, dtr, A[hh], Br, Cr, D[hh], sr=(3, 11), rows=rows, row_id=ids)
    assert np.array_equal(sub.code, full.code[ids]) and np.array_equal(sub.scale, full.scale[ids])


def test_delta_step_draws_key_row_uniforms():
    B, H, dk = 1, 2, 128
    rows = B * H * dk
    q, k, v, al, be = synth.delta_inputs(15, 0, B, H, dk, 128)
    st = oracle.make_state("int8_asym", rows, 128, synth.init_state(15, 0, rows, 128))
    o, Spre, _ = oracle.delta_step(st, q, k, v, al, be, B, H, diag=True, sr=(8, 4))
    U = _uniforms(8, 4, rows, range(rows))
    for r in range(0, rows, 17):
        c, s, z = oracle.quantize_row_sr(Spre[r], "int8_asym", U[r])
        assert np.array_equal(st.code[r], c) and st.scale[r] == s and st.zero[r] == z
