"""Pins of the oracle's DAMP-style two-tier delta state (CPU only).

"Mamba state quantization for inference", section "Mixed precision spends bits on
persistent channels": a Hadamard transform along each key channel's value dimension,
the protected key channels in FP16 and the rest in INT8 with scale and zero point,
the protected channels permuted to be contiguous, and one fused kernel that
reconstructs, runs the recurrence in FP32, refits and writes back.  Readings: Hs =
H_128/16 (Sylvester order; Hs symmetric, Hs Hs = I/2); the protected channels are key
channels 0..15 (16 of 128, the pages' main layout) after the model's offline
permutation; the stored matrix is S Hs row by row, and the step runs in those
coordinates with v rotated in and o rotated out.

Pins: the half rounding against numpy's float16; the rotation's entries and its
inverse; the step's pre-rounding matrix against the dense delta rule applied to the
reconstructed state; the stored half rows exactly the rounded pre-rounding values;
the int8 rows within half a step; the readout against the un-rotated new state; the
storage cost; stochastic rounding of the int8 rows.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.test_oracle_pins import delta_rounding_bound

F64 = np.float64
NHI = oracle.DAMP_NHI


def block_rel(got, ref, axis=-1):
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    rms = np.sqrt(np.mean(ref * ref, axis=axis, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))


def hadamard_s():
    """H_128 / 16 by Sylvester's construction, in float64."""
    Hm = np.array([[1.0]])
    while Hm.shape[0] < 128:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm / 16.0


def test_round_half_matches_numpy_float16():
    x = synth.normal(5, 97, 0, np.arange(20000)).astype(np.float32)
    scales = np.float32(2.0) ** np.arange(-30, 20, 0.37).astype(np.float32)
    vals = np.concatenate([(x[:, None] * scales[None, :20]).ravel(), x * 70000, x * 1e-6,
                           np.float32([0.5 + 2 ** -12, 2049.0, 2051.0, 65504.0, 65519.0, 65520.0, 6e-8,
                                       -3e-8, 2 ** -25, 2 ** -24 + 2 ** -26])]).astype(np.float32)
    got = np.array([oracle.round_half(float(v)) for v in vals], np.float32)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).astype(np.float32)
    assert np.array_equal(got, ref)


def test_rotation_is_sylvester_hadamard_over_16():
    Hs = hadamard_s()
    assert np.allclose(Hs @ Hs, np.eye(128) / 2)
    # a unit row rotates into row c of Hs; ones in the first NHI rows are stored as half, exactly
    S = np.zeros((1, 1, 128, 128), np.float32)
    S[0, 0, np.arange(128), np.arange(128)] = 1.0
    st = oracle.damp_from_fp32(S, 1, 1)
    rot = st.rotated()[0].astype(F64)
    assert np.array_equal(rot[:NHI], Hs[:NHI])
    # the int8 rows hold the +-1/16 pattern as two codes: 0 and the row's top code (254 or
    # 255: -mn*inv lands on the tie 127.5 up to the rounding of inv)
    top = st.code.max(axis=1, keepdims=True)
    assert np.all(top >= 254) and np.array_equal(st.code, np.where(Hs[NHI:] > 0, top, 0))
    assert np.all(np.abs(rot[NHI:] - Hs[NHI:]) <= st.scale.astype(F64)[:, None] * 0.5 * (1 + 2.0 ** -18))


def _state(seed, Bsz, H):
    S0 = synth.init_state(seed, 0, Bsz * H * 128, 128).reshape(Bsz, H, 128, 128)
    return oracle.damp_from_fp32(S0, Bsz, H), S0


@pytest.mark.parametrize("readout", ["post", "pre"])
def test_step_is_the_delta_rule_in_rotated_coordinates(readout):
    Bsz, H = 2, 2
    st, _ = _state(51, Bsz, H)
    Hs = hadamard_s()
    before = st.rotated().astype(F64)
    q, k, v, al, be = synth.delta_inputs(51, 0, Bsz, H, 128, 128)
    o, Spre = oracle.damp_step(st, q, k, v, al, be, Bsz, H, readout=readout, diag=True)
    for m in range(Bsz * H):
        b, hh = divmod(m, H)
        S = 2.0 * before[m] @ Hs                      # the state in original coordinates
        kk = k[b, hh].astype(F64)
        Snew = F64(al[b, hh]) * (np.eye(128) - F64(be[b, hh]) * np.outer(kk, kk)) @ S \
            + F64(be[b, hh]) * np.outer(kk, v[b, hh].astype(F64))
        assert block_rel(Spre[m], Snew @ Hs) < 1e-5
        # entry by entry: one fp32 step of the rule in rotated coordinates from the stored
        # matrix, v rotated in (rounded once)
        vt = Hs @ v[b, hh].astype(F64)
        Sstar, bound = delta_rounding_bound(before[m], k[b, hh], vt, be[b, hh], alpha=al[b, hh],
                                            v_err=2.0 ** -24 * np.abs(vt))
        assert np.allclose(Sstar, Snew @ Hs, rtol=1e-9, atol=1e-9)
        assert np.all(np.abs(Spre[m].astype(F64) - Sstar) <= bound)
        stored = st.rotated()[m].astype(F64)
        # half rows are the rounded pre-rounding values; int8 rows within half a step
        assert np.array_equal(stored[:NHI], Spre[m][:NHI].astype(np.float16).astype(F64))
        sc = st.scale[m * (128 - NHI):(m + 1) * (128 - NHI)].astype(F64)
        err = np.abs(stored[NHI:] - Spre[m][NHI:].astype(F64))
        assert np.all(err <= sc[:, None] * 0.5 * (1 + 2.0 ** -18) + 2.0 ** -22 * np.abs(Spre[m][NHI:]))
        # the readout, rotated back
        src = Spre[m].astype(F64) if readout == "pre" else stored
        oref = (2.0 * src @ Hs).T @ q[b, hh].astype(F64)
        assert block_rel(o[b, hh], oref) < 1e-5


def test_storage_is_under_ten_bits_per_value():
    # 16 half rows + 112 int8 rows with a 4-byte scale and zero point each, per 128 x 128 matrix
    bits = (NHI * 128 * 16 + (128 - NHI) * (128 * 8 + 64)) / (128 * 128)
    assert bits == pytest.approx(9.4375)
    assert bits < 9.875  # the pages' layout, with 9-bit low-tier values


def test_stochastic_rounding_of_the_int8_rows():
    Bsz, H = 1, 2
    st, _ = _state(52, Bsz, H)
    q, k, v, al, be = synth.delta_inputs(52, 0, Bsz, H, 128, 128)
    nlo = 128 - NHI
    rows = Bsz * H * nlo
    o, Spre = oracle.damp_step(st, q, k, v, al, be, Bsz, H, diag=True, sr=(9, 3))
    for m in range(Bsz * H):
        for li in range(0, nlo, 11):
            U = oracle.sr_row_uniforms(9, 3, rows, m * nlo + li, 128)
            c, s, z = oracle.quantize_row_sr(Spre[m][NHI + li], "int8_asym", U)
            r = m * nlo + li
            assert np.array_equal(st.code[r], c) and st.scale[r] == s and st.zero[r] == z
