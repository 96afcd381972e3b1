"""Pins of the oracle's KDA-style step: the delta rule with a decay per key channel (CPU only).

"Mamba state quantization for inference" names Kimi Delta Attention next to Gated
DeltaNet (one dk x dv matrix per head, read by the query, written by decay and a
delta-rule correction) and reports that DAMP finds persistence differing across KDA
key channels.  The pages give no formula; the reading taken is the channel-wise gate:
S' = (I - beta k k^T) Diag(alpha) S + beta k v^T with alpha in (0, 1)^dk, o = S'^T q.

Pins: the dense fp64 form; equal channel decays reduce to the scalar-decay delta rule;
alpha = beta = 1 with a unit key writes v at k; beta = 0 is a pure per-row decay that
keeps every code; the quantized state is within half a step of the fp32 update of the
same start; stochastic rounding draws the uniforms of each key row.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.test_oracle_pins import delta_rounding_bound

F64 = np.float64
U = 2.0 ** -24


def block_rel(got, ref, axis=-1):
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    rms = np.sqrt(np.mean(ref * ref, axis=axis, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))


def _dense(S, k, v, a, b):
    """(I - b k k^T) Diag(a) S + b k v^T in fp64."""
    k = k.astype(F64)
    return (np.eye(len(k)) - F64(b) * np.outer(k, k)) @ (a.astype(F64)[:, None] * S) \
        + F64(b) * np.outer(k, v.astype(F64))


@pytest.mark.parametrize("dk,dv", [(4, 4), (8, 8), (8, 4)])
def test_kda_fp32_matches_dense_form(dk, dv):
    Bsz, H, T = 2, 2, 3
    S0 = synth.init_state(31, 0, Bsz * H * dk, dv)
    st = oracle.make_state("fp32", Bsz * H * dk, dv, S0)
    S = S0.astype(F64).reshape(Bsz, H, dk, dv)
    for t in range(T):
        q, k, v, _, be = synth.delta_inputs(31, 0, Bsz, H, dk, dv, t=t)
        al = synth.kda_alpha(31, 0, Bsz, H, dk, t=t)
        o = oracle.kda_step(st, q, k, v, al, be, Bsz, H)
        for b in range(Bsz):
            for hh in range(H):
                S[b, hh] = _dense(S[b, hh], k[b, hh], v[b, hh], al[b, hh], be[b, hh])
                assert block_rel(o[b, hh], S[b, hh].T @ q[b, hh].astype(F64)) < 1e-5
        assert block_rel(st.h.reshape(Bsz, H, dk, dv), S, axis=(2, 3)) < 1e-5


def test_equal_channel_decays_reduce_to_the_scalar_rule():
    Bsz, H, dk, dv = 2, 3, 16, 32
    S0 = synth.init_state(32, 0, Bsz * H * dk, dv)
    q, k, v, al, be = synth.delta_inputs(32, 0, Bsz, H, dk, dv)
    a_vec = np.repeat(al[..., None], dk, axis=-1)
    s1 = oracle.make_state("fp32", Bsz * H * dk, dv, S0)
    s2 = oracle.make_state("fp32", Bsz * H * dk, dv, S0)
    o1 = oracle.kda_step(s1, q, k, v, a_vec, be, Bsz, H)
    o2 = oracle.delta_step(s2, q, k, v, al, be, Bsz, H)
    assert block_rel(s1.h, s2.h) < 1e-6 and block_rel(o1, o2) < 1e-6


def test_kda_writes_v_at_unit_key():
    Bsz, H, dk, dv = 2, 2, 16, 8
    st = oracle.make_state("fp32", Bsz * H * dk, dv, synth.init_state(33, 0, Bsz * H * dk, dv))
    q, k, v, _, be = synth.delta_inputs(33, 0, Bsz, H, dk, dv)
    oracle.kda_step(st, k, k, v, np.ones((Bsz, H, dk), np.float32), np.ones_like(be), Bsz, H)
    S = st.h.reshape(Bsz, H, dk, dv).astype(F64)
    assert block_rel(np.einsum("bhij,bhi->bhj", S, k.astype(F64)), v.astype(F64)) < 1e-5


@pytest.mark.parametrize("fmt", ["int8_asym", "int8_sym", "int4_asym"])
def test_kda_zero_beta_decays_each_row(fmt):
    bits, asym = oracle.FORMATS[fmt]
    Bsz, H, dk, dv = 2, 2, 32, 128
    rows = Bsz * H * dk
    st = oracle.make_state(fmt, rows, dv, synth.init_state(34, 0, rows, dv))
    top = (1 << bits) - 1 if asym else (1 << (bits - 1)) - 1
    full = (st.code.max(axis=1) == top) if asym else np.ones(rows, bool)
    code0, z0, s0 = st.code.copy(), st.zero.copy(), st.scale.copy()
    q, k, v, _, be = synth.delta_inputs(34, 0, Bsz, H, dk, dv)
    al = synth.kda_alpha(34, 0, Bsz, H, dk)
    be[:] = 0
    oracle.kda_step(st, q, k, v, al, be, Bsz, H)
    assert np.array_equal(st.code[full], code0[full]) and np.array_equal(st.zero[full], z0[full])
    a_r = al.reshape(-1).astype(F64)
    assert np.all(np.abs(st.scale[full] / (a_r[full] * s0[full]) - 1) <= 8 * U)


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym"])
def test_kda_quantized_state_within_half_step(fmt):
    Bsz, H, dk, dv = 2, 2, 16, 128
    rows = Bsz * H * dk
    st = oracle.make_state(fmt, rows, dv, synth.init_state(35, 0, rows, dv))
    S_start = st.dequant().astype(F64).reshape(Bsz, H, dk, dv)
    q, k, v, _, be = synth.delta_inputs(35, 0, Bsz, H, dk, dv)
    al = synth.kda_alpha(35, 0, Bsz, H, dk)
    o, Spre, _ = oracle.kda_step(st, q, k, v, al, be, Bsz, H, diag=True)
    Spre4 = Spre.reshape(Bsz, H, dk, dv).astype(F64)
    for b in range(Bsz):
        for hh in range(H):
            ref = _dense(S_start[b, hh], k[b, hh], v[b, hh], al[b, hh], be[b, hh])
            # within the rounding of one fp32 step from the dequantized start
            Sstar, bound = delta_rounding_bound(S_start[b, hh], k[b, hh], v[b, hh], be[b, hh], a_vec=al[b, hh])
            assert np.allclose(Sstar, ref, rtol=1e-12, atol=1e-12)
            assert np.all(np.abs(Spre4[b, hh] - ref) <= bound)
    deq = st.dequant().astype(F64)
    assert np.all(np.abs(deq - Spre.astype(F64))
                  <= st.scale.astype(F64)[:, None] * 0.5 * (1 + 2.0 ** -18) + 4 * U * np.abs(Spre))
    oref = np.einsum("bhij,bhi->bhj", deq.reshape(Bsz, H, dk, dv), q.astype(F64))
    assert block_rel(o, oref) < 1e-6


def test_kda_stochastic_rounding_draws_key_row_uniforms():
    B, H, dk = 1, 2, 128
    rows = B * H * dk
    q, k, v, _, be = synth.delta_inputs(36, 0, B, H, dk, 128)
    al = synth.kda_alpha(36, 0, B, H, dk)
    st = oracle.make_state("int8_asym", rows, 128, synth.init_state(36, 0, rows, 128))
    o, Spre, _ = oracle.kda_step(st, q, k, v, al, be, B, H, diag=True, sr=(4, 9))
    for r in range(0, rows, 13):
        c, s, z = oracle.quantize_row_sr(Spre[r], "int8_asym", oracle.sr_row_uniforms(4, 9, rows, r, 128))
        assert np.array_equal(st.code[r], c) and st.scale[r] == s and st.zero[r] == z
