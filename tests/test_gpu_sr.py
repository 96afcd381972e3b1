"""GPU parity of stochastic rounding (ssq_set_rounding) against the CPU oracle, through the C ABI.

Both sides draw the same uniforms (SplitMix64 at counter (token*rows + row)*128 + n) and
take the round-up decision frac(v) >= 1 - U exactly, so codes, scales and zero points
must match bit for bit; y and o within 1e-5.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mamba_decode_amd as ssq
    from tests import parity as par

QFORMATS = ["int8_sym", "int8_asym", "int4_sym", "int4_asym"]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _same_state(g, ost, where):
    assert np.array_equal(g["code"], ost.code), where
    assert np.array_equal(g["scale"].view(np.uint32), ost.scale.view(np.uint32)), where
    if "zero" in g and g["zero"] is not None and ost.zero is not None:
        assert np.array_equal(g["zero"].view(np.uint32), ost.zero.view(np.uint32)), where


def _init(seed, rows):
    from tests.test_gpu_mamba2 import init_rows
    return init_rows(seed, 0, rows)


@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("fmt", QFORMATS)
def test_decode_step_stochastic_teacher_forced(fmt, readout):
    B, H, G, P, T = 2, 6, 2, 32, 4
    rows = B * H * P
    seed, step0 = 1234567, 40
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    ost = oracle.make_state(fmt, rows, 128, _init(61, rows))
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G))
    ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    for t in range(T):
        say(f"stochastic decode fmt={fmt} readout={readout} t={t}")
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(61, 1, B, H, G, P, 128, t=t)
        par.write_gpu_state(gst, ost)
        y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
        ssq.ssq_decode_step(gst, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y, ro)
        yo = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, readout=readout, sr=(seed, step0 + t))
        _same_state(par.read_gpu_state(gst, fmt), ost, f"t={t}")
        assert par.block_rel(y.cpu().numpy(), yo, axis=2) <= 1e-5, t
        assert ssq.ssq_get_rounding(gst) == (ssq.SSQ_ROUND_STOCHASTIC, seed, step0 + t + 1)


def _rows_with_zero_points(zs, qa, per, n_rows, seed):
    """Rows spanning [-z/qa, 1 - z/qa] (range 1, so the grid's zero point is z), `per` rows for
    each z, the remaining rows seeded random."""
    rng = np.random.default_rng(seed)
    rows = synth.init_state(seed, 0, n_rows, 128).astype(np.float64)
    k = 0
    for z in zs:
        for _ in range(per):
            u = rng.permutation(np.linspace(0.0, 1.0, 128))
            rows[k] = -z / qa + u
            k += 1
    return rows.astype(np.float32)


@pytest.mark.parametrize("fmt", ["int4_asym", "int8_asym"])
def test_decode_stochastic_zero_points_around_the_fp32_bound(fmt):
    """Asymmetric rows decide stochastic rounding in fp32 while |z| <= 255 and take the
    general path beyond; rows with zero points on both sides of that bound and at it.  x = 0
    keeps each row's zero point through the step (the update only decays the row)."""
    qa = 15 if fmt == "int4_asym" else 255
    zs = [-300, -256, -255, -254, -40, 0, 3, 127, 200, 254, 255, 256, 300, 1000]
    B, H, G, P = 1, 4, 1, 64
    rows = B * H * P
    seed, step0 = 4242, 3
    init = _rows_with_zero_points(zs, qa, 12, rows, 64)
    ost = oracle.make_state(fmt, rows, 128, init)
    assert set(zs) <= set(np.unique(ost.zero).astype(int))
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G))
    ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    for t in range(3):
        say(f"stochastic decode around |z| = 255 fmt={fmt} t={t}")
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(64, 1, B, H, G, P, 128, t=t)
        x[:] = 0.0
        par.write_gpu_state(gst, ost)
        y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
        ssq.ssq_decode_step(gst, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
        yo = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, sr=(seed, step0 + t))
        _same_state(par.read_gpu_state(gst, fmt), ost, f"t={t}")
        assert par.block_rel(y.cpu().numpy(), yo, axis=2) <= 1e-5, t


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym", "int8_sym"])
def test_scan_stochastic_equals_steps_and_oracle(fmt):
    B, H, G, P, T = 2, 4, 1, 16, 20
    rows = B * H * P
    seed, step0 = 99, 7
    init = _init(62, rows)
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(62, 0, B, T, H, G, P, 128)
    say(f"stochastic scan fmt={fmt}")
    g1 = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G), init)
    ssq.ssq_set_rounding(g1, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    y1 = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_scan(g1, T, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y1)
    assert ssq.ssq_get_rounding(g1)[2] == step0 + T
    g2 = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G), init)
    ssq.ssq_set_rounding(g2, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    for t in range(T):
        y = torch.empty(x[:, t].shape, dtype=torch.float32, device="cuda")
        ssq.ssq_decode_step(g2, par.dev(x[:, t]), par.dev(dt[:, t]), par.dev(A), par.dev(Bm[:, t]),
                            par.dev(Cm[:, t]), par.dev(D), y)
    s1, s2 = par.read_gpu_state(g1, fmt), par.read_gpu_state(g2, fmt)
    for k in s1:
        if s1[k] is not None:
            assert np.array_equal(s1[k].view(np.uint32) if s1[k].dtype == np.float32 else s1[k],
                                  s2[k].view(np.uint32) if s2[k].dtype == np.float32 else s2[k]), k
    ost = oracle.make_state(fmt, rows, 128, init)
    yo = oracle.mamba2_scan(ost, x, dt, A, Bm, Cm, D, sr=(seed, step0))
    _same_state(s1, ost, "scan")
    assert par.block_rel(y1.cpu().numpy(), yo, axis=(1, 3)) <= 1e-5


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_sym"])
def test_delta_step_stochastic(fmt):
    B, H = 2, 3
    rows = B * H * 128
    seed, step0 = 5, 1000
    init = synth.init_state(63, 0, rows, 128)
    ost = oracle.make_state(fmt, rows, 128, init)
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_DELTA, fmt, B, H, 128, 128), init)
    ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    for t in range(2):
        say(f"stochastic delta fmt={fmt} t={t}")
        q, k, v, al, be = synth.delta_inputs(63, t, B, H, 128, 128)
        par.write_gpu_state(gst, ost)
        o = torch.empty(v.shape, dtype=torch.float32, device="cuda")
        ssq.ssq_delta_step(gst, par.dev(q), par.dev(k), par.dev(v), par.dev(al), par.dev(be), o)
        oo = oracle.delta_step(ost, q, k, v, al, be, B, H, sr=(seed, step0 + t))
        _same_state(par.read_gpu_state(gst, fmt), ost, f"t={t}")
        assert par.block_rel(o.cpu().numpy(), oo, axis=2) <= 1e-5


def test_370m_layer_stochastic_sampled_rows():
    """The 370m-shaped int4 layer (batch 256 x 32 heads x 64), one stochastic step, in the bench's
    launch configuration; the oracle follows 512 sampled rows with their state row ids."""
    fmt, B, H, P = "int4_asym", 256, 32, 64
    rows = B * H * P
    seed, step0 = 2024, 3
    sample = np.unique(np.linspace(0, rows - 1, 512).astype(np.int64))
    say("370m layer stochastic")
    init = synth.init_state(2, 0, rows, 128, threads=8)
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P), init)
    ost = oracle.make_state(fmt, len(sample), 128, init[sample])
    del init
    ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(2, 0, B, H, 1, P, 128, t=0)
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_decode_step(gst, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
    xr, dtr, Br, Cr, Ar, Dr = synth.mamba2_rows_scan_inputs(2, 0, B, 1, H, 1, P, 128, sample)
    yo = oracle.mamba2_rows_scan(ost, xr, dtr, Ar, Br, Cr, Dr, sr=(seed, step0), rows=rows, row_id=sample)
    g = par.read_gpu_state(gst, fmt)
    assert np.array_equal(g["code"][sample], ost.code)
    assert np.array_equal(g["scale"][sample], ost.scale) and np.array_equal(g["zero"][sample], ost.zero)
    assert par.block_rel(y.cpu().numpy().reshape(-1)[sample], yo[:, 0]) <= 1e-5


def test_rounding_mode_errors_and_reset():
    gq = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, "int8_asym", 1, 2, 16))
    gf = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, "fp32", 1, 2, 16))
    assert ssq.ssq_get_rounding(gq) == (ssq.SSQ_ROUND_NEAREST, 0, 0)
    with pytest.raises(ssq.SsqError) as e:
        ssq.ssq_set_rounding(gq, 7, 1, 1)
    assert e.value.status == ssq.SSQ_ERR_INVALID_ARG
    with pytest.raises(ssq.SsqError) as e:
        ssq.ssq_set_rounding(gf, ssq.SSQ_ROUND_STOCHASTIC, 1, 1)
    assert e.value.status == ssq.SSQ_ERR_UNSUPPORTED
    ssq.ssq_set_rounding(gf, ssq.SSQ_ROUND_NEAREST, 0, 0)
    ssq.ssq_set_rounding(gq, ssq.SSQ_ROUND_STOCHASTIC, 11, 22)
    assert ssq.ssq_get_rounding(gq) == (ssq.SSQ_ROUND_STOCHASTIC, 11, 22)
    # a rejected call (T = 0) does not advance the token
    buf = torch.zeros(4096, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    rc = ssq.lib.ssq_scan(gq.handle, 0, p, p, p, p, p, p, p, 0, None)
    assert rc == ssq.SSQ_ERR_INVALID_ARG
    assert ssq.ssq_get_rounding(gq)[2] == 22
    ssq.ssq_set_rounding(gq, ssq.SSQ_ROUND_NEAREST, 0, 0)
    assert ssq.ssq_get_rounding(gq) == (ssq.SSQ_ROUND_NEAREST, 0, 0)


@pytest.mark.parametrize("mag_exp", [-118, -95, -60, 100])
@pytest.mark.parametrize("fmt", ["int4_asym", "int8_asym", "int8_sym"])
def test_decode_stochastic_far_from_unit_scale(fmt, mag_exp):
    """Rows scaled by 2^mag_exp, a fifth of their entries exactly zero, x = 0 (the state only
    decays): scales whose reciprocal is far above and below 2^16 and reaches past 2^100, where
    the fp32 decision's A = 2^16 inv would leave the fp32 range, with exact-zero entries."""
    B, H, G, P, T = 2, 4, 1, 32, 3
    rows = B * H * P
    seed, step0 = 424242 + mag_exp, 7
    init = synth.init_state(70, 0, rows, 128).astype(np.float64) * 2.0 ** mag_exp
    init[:, ::5] = 0.0
    ost = oracle.make_state(fmt, rows, 128, init.astype(np.float32))
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G))
    ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    for t in range(T):
        say(f"stochastic decode far from unit scale fmt={fmt} mag=2^{mag_exp} t={t}")
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(71, 0, B, H, G, P, 128, t=t)
        x = np.zeros_like(x)
        par.write_gpu_state(gst, ost)
        y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
        ssq.ssq_decode_step(gst, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
        yo = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, sr=(seed, step0 + t))
        _same_state(par.read_gpu_state(gst, fmt), ost, f"t={t}")
        assert par.block_rel(y.cpu().numpy(), yo, axis=2) <= 1e-5, t
