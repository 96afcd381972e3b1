"""Every row at full size, and the long scans at their own shapes, against the oracle.

The oracle runs on K host workers (the process's CPU affinity, at most 16), each one
single-threaded on a disjoint slice of sequences or rows; the wall time of each oracle
run is printed with K.

* Mamba-2 370m-shaped decode layer (batch 256 x 32 heads x 64 x 128, int4 asymmetric,
  seeded random state with 5% x20 outlier rows): every one of the 524,288 rows.
* Mamba-2 8B-shaped decode layer (batch 256 x 128 heads x 64 x 128), int8 symmetric and
  int4 asymmetric, two steps from a zero state: every one of the 2,097,152 rows.
* int4 decode layers of 1,048,576 and 2,097,152 rows (the sizes at which a wave takes 16
  and 32 iterations), both int4 formats and both readouts, from a seeded random state:
  every row.
* Delta-rule layer (batch 256 x 32 heads of 128 x 128, int8 asymmetric, seeded random
  state): every one of the 8,192 matrices.
* Mamba-2 130m-shaped layer (batch 32 x 24 heads x 64 x 128, 2048 tokens, state rounded
  every token), int8 symmetric, int8 asymmetric and the fp32 control: every row and every
  token of one layer.
* Mamba-2 8B-shaped scan (batch 8 x 128 heads x 64 x 128, 8192 tokens), int8 symmetric and
  int4 asymmetric: the GPU scans the whole layer; the oracle follows 4,096 rows, four in
  every (sequence, head).

Decode steps are compared under the contract (codes bit-exact except near-boundary flips,
scales and zero points bit-exact outside rows holding one; y within the contract's 1e-3 of
its head for quantized states, and every row's y within the error bound of an fp32 sum of
its 128 readout terms).  Scans run
free, so they are compared on y and the dequantized state (1e-3; 1e-5 for the fp32
control), with the number of differing codes reported.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mamba_decode_amd as ssq
    from tests import parity as par

K = oracle.workers()
THREADS = K


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def oracle_timed(label, fn, *a, **kw):
    t0 = time.perf_counter()
    r = fn(*a, **kw)
    say(f"  oracle {label}: {time.perf_counter() - t0:.2f} s on {K} host workers")
    return r


def m2desc(fmt, B, H, P, G=1):
    return ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G)


def run_step(gst, x, dt, A, Bm, Cm, D, readout="post"):
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    ssq.ssq_decode_step(gst, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y, readout=ro)
    return y.cpu().numpy()


def _decode_every_row(fmt, B, H, P, init_seed, steps, seed, readout="post"):
    rows = B * H * P
    if init_seed is not None:
        say(f"  drawing the fp32 state of {rows} rows")
        init = synth.init_state(init_seed, 0, rows, 128, threads=THREADS)
        gst = par.new_gpu_state(m2desc(fmt, B, H, P), init)
        ost = oracle.make_state(fmt, rows, 128, init)
        del init
        g = par.read_gpu_state(gst, fmt)
        assert np.array_equal(g["code"], ost.code), "initial codes differ"
        assert np.array_equal(g["scale"].view(np.uint32), ost.scale.view(np.uint32)), "initial scales differ"
        assert np.array_equal(g["zero"], ost.zero), "initial zero points differ"
    else:
        gst = par.new_gpu_state(m2desc(fmt, B, H, P))
        ost = oracle.make_state(fmt, rows, 128)
    for t in range(steps):
        say(f"  {fmt} step {t}: {rows} rows")
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(seed, 0, B, H, 1, P, 128, t=t)
        yg = run_step(gst, x, dt, A, Bm, Cm, D, readout)
        yo, hpre, vq = oracle_timed(f"decode step of {rows} rows", oracle.mamba2_step_par, ost, x, dt, A, Bm, Cm, D,
                                    readout=readout, diag=True)
        g = par.read_gpu_state(gst, fmt)
        flips = par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, f"{fmt} step {t}")
        err = par.block_rel(yg, yo, axis=2)
        # y against the exact readout of the new row: within the error of an fp32 sum of its 128
        # terms for every row, and within the contract's head-relative tolerance for quantized y
        crow = np.broadcast_to(Cm[:, :, None, :], (B, H, P, 128)).reshape(rows, 128)
        terms = hpre if readout == "pre" else ost.dequant()  # the row the readout sums over
        ratio = par.y_within_sum_bound(yg, yo, crow, terms, (D[None, :, None] * x).astype(np.float32))
        say(f"  {fmt} step {t}: {flips} codes at a rounding boundary differ, y max relative error {err:.2e}, "
            f"largest error / fp32-sum bound {ratio:.3f}")
        assert ratio <= 1.0
        assert err <= 1e-3
        if flips:
            par.write_gpu_state(gst, ost)  # teacher forcing: the next step starts from the oracle's state


def test_370m_decode_layer_every_row():
    """The bench's headline layer in the launch configuration it times, every row compared."""
    say("370m decode layer, int4 asymmetric, every row")
    _decode_every_row("int4_asym", 256, 32, 64, init_seed=2, steps=1, seed=2)


@pytest.mark.parametrize("fmt", ["int8_sym", "int4_asym"])
def test_8b_decode_layer_every_row(fmt):
    say(f"8B decode layer, {fmt}, every row")
    _decode_every_row(fmt, 256, 128, 64, init_seed=None, steps=2, seed=4)


@pytest.mark.parametrize("fmt,readout,B,H,P", [("int4_sym", "post", 128, 128, 64), ("int4_asym", "post", 128, 128, 64),
                                               ("int4_sym", "post", 256, 128, 64), ("int4_asym", "pre", 256, 128, 64),
                                               ("int4_sym", "pre", 128, 128, 64), ("int4_asym", "post", 131100, 1, 16)])
def test_int4_decode_long_waves_every_row(fmt, readout, B, H, P):
    """int4 layers large enough for the step to give each wave 16 (1,048,576 rows) or 32
    (2,097,152 rows) iterations on a 256-CU part, both readouts, from a seeded random state,
    every row compared for two teacher-forced steps.  131,100 sequences of one 16-row head
    make 131,100 iterations: 4,096 waves of 32 and 28 left over for the one-iteration launch."""
    say(f"int4 decode, {fmt}, {readout} readout, batch {B} x {H} heads x {P}, every row")
    _decode_every_row(fmt, B, H, P, init_seed=7, steps=2, seed=9, readout=readout)


def test_delta_layer_every_matrix():
    B, H, fmt = 256, 32, "int8_asym"
    rows = B * H * 128
    say(f"delta layer, {fmt}, every one of {B * H} matrices")
    init = synth.init_state(3, 0, rows, 128, threads=THREADS)
    gst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_DELTA, fmt, B, H, 128, 128), init)
    ost = oracle.make_state(fmt, rows, 128, init)
    del init
    q, k, v, al, be = synth.delta_inputs(3, 0, B, H, 128, 128)
    o = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_delta_step(gst, par.dev(q), par.dev(k), par.dev(v), par.dev(al), par.dev(be), o)
    og = o.cpu().numpy()
    oo, _, vq = oracle_timed(f"delta step of {B * H} matrices", oracle.delta_step_par, ost, q, k, v, al, be, B, H,
                             diag=True)
    g = par.read_gpu_state(gst, fmt)
    flips = par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, "delta layer")
    err = par.block_rel(og, oo, axis=2)
    say(f"  delta layer: {flips} codes at a rounding boundary differ, o max relative error {err:.2e}")
    assert err <= 1e-5


def _compare_free_scan(fmt, g, ost, yg, yo, axis_y):
    ey = par.block_rel(yg, yo, axis=axis_y)
    if fmt == "fp32":
        es = par.block_rel(g["h"], ost.h, axis=1)
        say(f"  {fmt}: y max relative error {ey:.2e}, state {es:.2e}")
        assert ey <= 1e-5 and es <= 1e-5
        return
    diff = int((g["code"] != ost.code).sum())
    deq = oracle.dequantize_rows(g["code"], g["scale"], g["zero"])
    es = par.block_rel(deq, ost.dequant(), axis=1)
    say(f"  {fmt}: {diff} of {g['code'].size} final codes differ; y max relative error {ey:.2e}, "
        f"dequantized state {es:.2e}")
    assert ey <= 1e-3 and es <= 1e-3
    assert diff <= 1e-4 * g["code"].size


@pytest.mark.parametrize("fmt", ["int8_sym", "int8_asym", "fp32"])
def test_130m_scan_layer_every_row(fmt):
    """One layer of the 130m-shaped stack at its own shape: batch 32, 2048 tokens, every row
    and every token's y compared (the free run from a zero state)."""
    B, H, G, P, T = 32, 24, 1, 64, 2048
    rows = B * H * P
    say(f"130m scan layer, {fmt}: {rows} rows x {T} tokens")
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(1, 0, B, T, H, G, P, 128, threads=THREADS)
    gst = par.new_gpu_state(m2desc(fmt, B, H, P))
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_scan(gst, T, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
    yg = y.cpu().numpy()
    del y
    g = par.read_gpu_state(gst, fmt)
    ost = oracle.make_state(fmt, rows, 128)
    yo = oracle_timed(f"scan of {rows} rows x {T} tokens", oracle.mamba2_scan_par, ost, x, dt, A, Bm, Cm, D)
    _compare_free_scan(fmt, g, ost, yg, yo, axis_y=(1, 3))


@pytest.mark.parametrize("fmt", ["int8_sym", "int4_asym"])
def test_8b_scan_layer_own_shape(fmt):
    """The 8B-shaped layer at batch 8 over 8192 tokens: the GPU scans all 65,536 rows; the
    oracle follows four rows of every (sequence, head), 4,096 rows.  Rows are independent and a
    row reads only its own x and its head's dt, A, D, B and C, so the oracle scans the same
    sequences and heads with just those four rows per head (x sliced along the head dimension)."""
    B, H, G, P, T = 8, 128, 1, 64, 8192
    psel = np.array([0, 21, 42, 63])
    say(f"8B scan layer, {fmt}: {B * H * P} rows x {T} tokens")
    t0 = time.perf_counter()
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(4, 0, B, T, H, G, P, 128, threads=THREADS)
    say(f"  inputs drawn in {time.perf_counter() - t0:.1f} s")
    gst = par.new_gpu_state(m2desc(fmt, B, H, P))
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_scan(gst, T, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
    torch.cuda.synchronize()
    say("  GPU scan done")
    yg = y[:, :, :, torch.from_numpy(psel).cuda()].cpu().numpy()  # [B][T][H][4]
    del y
    xs = np.ascontiguousarray(x[:, :, :, psel])
    del x
    g = par.read_gpu_state(gst, fmt)
    rows = (np.arange(B * H)[:, None] * P + psel[None, :]).ravel()  # (b, h, p) in the oracle's order
    g = {k: v[rows] for k, v in g.items()}
    ost = oracle.make_state(fmt, len(rows), 128)
    yo = oracle_timed(f"scan of {len(rows)} rows x {T} tokens", oracle.mamba2_scan_par, ost, xs, dt, A, Bm, Cm, D)
    _compare_free_scan(fmt, g, ost, yg, yo, axis_y=(1, 3))
