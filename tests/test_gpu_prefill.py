"""GPU parity of the chunked prefill (ssq_prefill) against the CPU oracle, through the C ABI."""
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


def _run(gst, T, chunk, ins, readout):
    x, dt, Bm, Cm, A, D = ins
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_prefill(gst, T, chunk, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D),
                    y, readout)
    return y.cpu().numpy()


def _same(g, ost, where):
    assert np.array_equal(g["code"], ost.code), where
    assert np.array_equal(g["scale"].view(np.uint32), ost.scale.view(np.uint32)), where
    assert np.array_equal(g["zero"].view(np.uint32), ost.zero.view(np.uint32)), where


@pytest.mark.parametrize("chunk", [1, 5, 64])
@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("fmt", QFORMATS)
def test_prefill_matches_oracle(fmt, readout, chunk):
    B, H, G, P, T = 2, 4, 2, 32, 24
    rows = B * H * P
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    from tests.test_gpu_mamba2 import init_rows
    init = init_rows(71, 0, rows)
    ins = synth.mamba2_scan_inputs(71, 0, B, T, H, G, P, 128)
    x, dt, Bm, Cm, A, D = ins
    say(f"prefill fmt={fmt} readout={readout} chunk={chunk}")
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G), init)
    yg = _run(gst, T, chunk, ins, ro)
    ost = oracle.make_state(fmt, rows, 128, init)
    yo = oracle.mamba2_prefill(ost, x, dt, A, Bm, Cm, D, chunk=chunk, readout=readout)
    _same(par.read_gpu_state(gst, fmt), ost, "final state")
    assert par.block_rel(yg, yo, axis=(1, 3)) <= 1e-5


def test_fp32_prefill_is_the_scan():
    B, H, G, P, T = 2, 4, 1, 16, 12
    rows = B * H * P
    init = synth.init_state(72, 0, rows, 128)
    ins = synth.mamba2_scan_inputs(72, 0, B, T, H, G, P, 128)
    x, dt, Bm, Cm, A, D = ins
    g1 = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, "fp32", B, H, P, 128, G), init)
    y1 = _run(g1, T, 4, ins, ssq.SSQ_READ_POST_QUANT)
    g2 = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, "fp32", B, H, P, 128, G), init)
    y2 = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_scan(g2, T, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y2)
    assert np.array_equal(y1, y2.cpu().numpy())
    assert np.array_equal(par.read_gpu_state(g1, "fp32")["h"], par.read_gpu_state(g2, "fp32")["h"])


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym"])
def test_prefill_stochastic_chunk_ends(fmt):
    B, H, G, P, T, chunk = 2, 4, 1, 16, 20, 6
    rows = B * H * P
    seed, step0 = 31, 500
    init = synth.init_state(73, 0, rows, 128)
    ins = synth.mamba2_scan_inputs(73, 0, B, T, H, G, P, 128)
    x, dt, Bm, Cm, A, D = ins
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G), init)
    ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    yg = _run(gst, T, chunk, ins, ssq.SSQ_READ_POST_QUANT)
    assert ssq.ssq_get_rounding(gst)[2] == step0 + T
    ost = oracle.make_state(fmt, rows, 128, init)
    yo = oracle.mamba2_prefill(ost, x, dt, A, Bm, Cm, D, chunk=chunk, sr=(seed, step0))
    _same(par.read_gpu_state(gst, fmt), ost, "final state")
    assert par.block_rel(yg, yo, axis=(1, 3)) <= 1e-5


def test_prefill_130m_heads_long_prompt():
    """130m-shaped heads (24 x 64 x 128) of two sequences over a 512-token prompt in chunks of 64,
    int8 asymmetric, from the zero state, then decode steps continue from the packed state."""
    B, H, G, P, T, chunk, fmt = 2, 24, 1, 64, 512, 64, "int8_asym"
    rows = B * H * P
    ins = synth.mamba2_scan_inputs(74, 0, B, T, H, G, P, 128)
    x, dt, Bm, Cm, A, D = ins
    say("prefill 130m heads T=512")
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G))
    yg = _run(gst, T, chunk, ins, ssq.SSQ_READ_POST_QUANT)
    ost = oracle.make_state(fmt, rows, 128)
    yo = oracle.mamba2_prefill(ost, x, dt, A, Bm, Cm, D, chunk=chunk)
    g = par.read_gpu_state(gst, fmt)
    assert (g["code"] != ost.code).mean() <= 1e-4
    assert par.block_rel(yg, yo, axis=(1, 3)) <= 1e-3
    # decode continues from the prefilled state on both sides
    xs, dts, Bs, Cs, As, Ds = synth.mamba2_step_inputs(74, 1, B, H, G, P, 128, t=0)
    par.write_gpu_state(gst, ost)
    y = torch.empty(xs.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_decode_step(gst, par.dev(xs), par.dev(dts), par.dev(As), par.dev(Bs), par.dev(Cs), par.dev(Ds), y)
    yo1 = oracle.mamba2_step(ost, xs, dts, As, Bs, Cs, Ds)
    assert par.block_rel(y.cpu().numpy(), yo1, axis=2) <= 1e-5
