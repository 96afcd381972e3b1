"""The oracle's parallel drivers return exactly what the single calls return: each worker
runs the same C entry point on a disjoint slice of sequences or rows (CPU only)."""
import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_sym", "fp32"])
def test_parallel_mamba2_drivers_equal_single_calls(fmt):
    B, H, G, P, N, T = 5, 6, 2, 8, 128, 17
    rows = B * H * P
    init = synth.init_state(3, 0, rows, N)
    x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(3, 0, B, H, G, P, N)
    s1 = oracle.make_state(fmt, rows, N, init)
    s2 = s1.copy()
    y1, h1, v1 = oracle.mamba2_step(s1, x, dt, A, Bm, Cm, D, diag=True)
    y2, h2, v2 = oracle.mamba2_step_par(s2, x, dt, A, Bm, Cm, D, diag=True, k=3)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)
    if fmt == "fp32":
        assert np.array_equal(s1.h, s2.h)
    else:
        assert np.array_equal(s1.code, s2.code) and np.array_equal(s1.scale, s2.scale)
        assert np.array_equal(s1.zero, s2.zero) and np.array_equal(v1, v2)
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(3, 0, B, T, H, G, P, N)
    s1 = oracle.make_state(fmt, rows, N, init)
    s2 = s1.copy()
    assert np.array_equal(oracle.mamba2_scan(s1, x, dt, A, Bm, Cm, D, readout="pre"),
                          oracle.mamba2_scan_par(s2, x, dt, A, Bm, Cm, D, readout="pre", k=4))
    sample = np.arange(0, rows, 5)
    xr, dtr, Br, Cr, Ar, Dr = synth.mamba2_rows_scan_inputs(3, 0, B, T, H, G, P, N, sample)
    s1 = oracle.make_state(fmt, len(sample), N, init[sample])
    s2 = s1.copy()
    assert np.array_equal(oracle.mamba2_rows_scan(s1, xr, dtr, Ar, Br, Cr, Dr),
                          oracle.mamba2_rows_scan_par(s2, xr, dtr, Ar, Br, Cr, Dr, k=4))
    if fmt != "fp32":
        assert np.array_equal(s1.code, s2.code)


@pytest.mark.parametrize("fmt", ["int8_asym", "fp32"])
def test_parallel_delta_driver_equals_single_call(fmt):
    B, H = 3, 2
    init = synth.init_state(4, 0, B * H * 128, 128)
    s1 = oracle.make_state(fmt, B * H * 128, 128, init)
    s2 = s1.copy()
    q, k, v, al, be = synth.delta_inputs(4, 0, B, H, 128, 128)
    r1 = oracle.delta_step(s1, q, k, v, al, be, B, H, diag=True)
    r2 = oracle.delta_step_par(s2, q, k, v, al, be, B, H, diag=True, k=2)
    for a, b in zip(r1, r2):
        assert (a is None and b is None) or np.array_equal(a, b)


def test_scan_inputs_drawn_in_blocks_equal_one_draw():
    a = synth.mamba2_scan_inputs(1, 3, 4, 700, 24, 1, 64, 128)
    b = synth.mamba2_scan_inputs(1, 3, 4, 700, 24, 1, 64, 128, threads=4)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_parallel_kda_damp_prefill_drivers_equal_single_calls():
    B, H = 3, 2
    init = synth.init_state(4, 0, B * H * 128, 128)
    s1 = oracle.make_state("int8_asym", B * H * 128, 128, init)
    s2 = s1.copy()
    q, k, v, al, be = synth.delta_inputs(4, 0, B, H, 128, 128)
    ak = synth.kda_alpha(4, 0, B, H, 128)
    assert np.array_equal(oracle.kda_step(s1, q, k, v, ak, be, B, H), oracle.kda_step_par(s2, q, k, v, ak, be, B, H, k=2))
    assert np.array_equal(s1.code, s2.code) and np.array_equal(s1.scale, s2.scale)
    d1 = oracle.damp_from_fp32(init.reshape(B, H, 128, 128), B, H)
    d2 = oracle.damp_from_fp32_par(init.reshape(B, H, 128, 128), B, H, k=2)
    assert np.array_equal(d1.code, d2.code) and np.array_equal(d1.hi, d2.hi) and np.array_equal(d1.scale, d2.scale)
    assert np.array_equal(oracle.damp_step(d1, q, k, v, al, be, B, H), oracle.damp_step_par(d2, q, k, v, al, be, B, H, k=3))
    assert np.array_equal(d1.code, d2.code) and np.array_equal(d1.hi, d2.hi)
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(4, 0, 4, 40, 3, 1, 16, 128)
    p1 = oracle.make_state("int8_asym", 4 * 3 * 16, 128)
    p2 = p1.copy()
    assert np.array_equal(oracle.mamba2_prefill(p1, x, dt, A, Bm, Cm, D, chunk=8),
                          oracle.mamba2_prefill_par(p2, x, dt, A, Bm, Cm, D, chunk=8, k=3))
    assert np.array_equal(p1.code, p2.code)


def test_parallel_stochastic_decode_draws_each_rows_own_uniforms():
    B, H, G, P, N = 4, 3, 1, 16, 128
    rows = B * H * P
    init = synth.init_state(6, 0, rows, N)
    x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(6, 0, B, H, G, P, N)
    s1 = oracle.make_state("int4_asym", rows, N, init)
    s2 = s1.copy()
    y1 = oracle.mamba2_step(s1, x, dt, A, Bm, Cm, D, sr=(11, 5))
    y2 = oracle.mamba2_step_par(s2, x, dt, A, Bm, Cm, D, sr=(11, 5), k=3)
    assert np.array_equal(y1, y2) and np.array_equal(s1.code, s2.code)
