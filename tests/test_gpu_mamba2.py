"""GPU parity of the Mamba-2 path (ssq_alloc_state, ssq_decode_step, ssq_scan, ssq_dequant)
against the CPU oracle, through the C ABI, on seeded synthetic inputs.

Shapes: small cases that span several waves and a ragged tail of rows, the
benchmark layers at full size checked on sampled rows, and long scans.
"""
import math
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

FORMATS = ["fp32", "int8_sym", "int8_asym", "int4_sym", "int4_asym"]
QFORMATS = FORMATS[1:]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def m2desc(fmt, B, H, P, G=1):
    return ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, G)


def special_rows(n_each=4, N=128):
    """Rows that exercise the refit's corners: zero, constant, huge offset (slow path), tiny, outliers."""
    z = synth.normal(77, 98, 0, np.arange(16 * N)).reshape(16, N)
    rows = [np.zeros((n_each, N)),
            np.full((n_each, N), 3.25), np.full((n_each, N), -0.5),
            1e4 + 1e-4 * z[:n_each],          # |z| ~ 2.5e10 at int8: slow path
            -7.0 + 1e-5 * z[n_each:2 * n_each],
            1e-30 * z[:n_each],
            np.where(np.arange(N) == 5, 1e3, z[:n_each])]
    return np.concatenate(rows).astype(np.float32)


def init_rows(seed, layer, nrows, N=128, special=True):
    h = synth.init_state(seed, layer, nrows, N)
    if special:
        sp = special_rows()
        k = min(len(sp), nrows)
        idx = np.linspace(0, nrows - 1, k).astype(int)
        h[idx] = sp[:k]
    return h


def assert_same_y(y_scan, y_step, fmt):
    """y of a scan against y of the same tokens as decode steps: bit for bit in every format
    (the scan sums an int8 row's readout in the decode step's order although it spreads the
    row over 4 lanes instead of 8)."""
    a = np.asarray(y_scan, np.float32).view(np.uint32)
    b = np.asarray(y_step, np.float32).view(np.uint32)
    assert np.array_equal(a, b), f"{fmt}: {int((a != b).sum())} of {a.size} y differ"


def run_step(gst, x, dt, A, Bm, Cm, D, readout):
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_decode_step(gst, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y,
                        readout)
    return y.cpu().numpy()


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", FORMATS)
def test_init_quantize_and_dequant_bit_exact(fmt):
    B, H, P = 3, 5, 32
    rows = B * H * P
    init = init_rows(31, 0, rows)
    say(f"init fmt={fmt} rows={rows}")
    gst = par.new_gpu_state(m2desc(fmt, B, H, P), init)
    g = par.read_gpu_state(gst, fmt)
    ost = oracle.make_state(fmt, rows, 128, init)
    out = torch.empty(rows * 128, dtype=torch.float32, device="cuda")
    ssq.ssq_dequant(gst, out)
    deq = out.cpu().numpy().reshape(rows, 128)
    if fmt == "fp32":
        assert np.array_equal(g["h"], init)
        assert np.array_equal(deq, init)
        return
    assert np.array_equal(g["code"], ost.code)
    assert np.array_equal(g["scale"].view(np.uint32), ost.scale.view(np.uint32))
    if fmt.endswith("asym"):
        assert np.array_equal(g["zero"].view(np.uint32), ost.zero.view(np.uint32))
    assert np.array_equal(deq.view(np.uint32), ost.dequant().view(np.uint32))


@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_decode_step_teacher_forced(fmt, readout):
    """Each step starts from the oracle's state on both sides; codes, scales, zero points and y
    are compared after every step."""
    B, H, G, P, T = 3, 6, 2, 32, 6
    rows = B * H * P
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    ost = oracle.make_state(fmt, rows, 128, init_rows(41, 1, rows))
    gst = par.new_gpu_state(m2desc(fmt, B, H, P, G))
    flips = 0
    for t in range(T):
        say(f"teacher-forced fmt={fmt} readout={readout} t={t}")
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(41, 1, B, H, G, P, 128, t=t)
        par.write_gpu_state(gst, ost)
        yg = run_step(gst, x, dt, A, Bm, Cm, D, ro)
        yo, _, vq = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, readout=readout, diag=True)
        g = par.read_gpu_state(gst, fmt)
        if fmt == "fp32":
            assert np.array_equal(g["h"], ost.h), t
        else:
            flips += par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, f"t={t}")
        assert par.block_rel(yg, yo, axis=2) <= 1e-5, t
    say(f"  flipped codes: {flips}")


@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("shape", [(1, 5, 1, 16), (3, 7, 7, 48), (2, 9, 3, 80)])
@pytest.mark.parametrize("fmt", FORMATS)
def test_decode_ragged_wave_tails(fmt, shape, readout):
    """Row counts that leave part of a wave's iterations to the one-iteration tail launch
    (80, 1,008 and 1,440 rows: an int4 or fp32 wave-iteration takes 16 rows and a wave 8 of
    them, an int8 wave-iteration 8 rows and a wave 4), groups shared by 1, 1 or 3 heads."""
    B, H, G, P = shape
    rows = B * H * P
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    say(f"ragged fmt={fmt} shape={shape} readout={readout}")
    ost = oracle.make_state(fmt, rows, 128, init_rows(43, 2, rows))
    gst = par.new_gpu_state(m2desc(fmt, B, H, P, G))
    for t in range(2):
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(43, 2, B, H, G, P, 128, t=t)
        par.write_gpu_state(gst, ost)
        yg = run_step(gst, x, dt, A, Bm, Cm, D, ro)
        yo, _, vq = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, readout=readout, diag=True)
        g = par.read_gpu_state(gst, fmt)
        if fmt == "fp32":
            assert np.array_equal(g["h"], ost.h), t
        else:
            par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, f"t={t}")
        assert par.block_rel(yg, yo, axis=2) <= 1e-5, t


def test_config0_free_running_and_scan_equivalence():
    """Single Mamba-2 layer, batch 1, 24 heads x 64 x 128, T = 64, int8 asymmetric, state from 0,
    seed 0: 64 decode steps against the oracle, and one 64-token scan that must equal them bit for bit."""
    B, H, G, P, T, fmt = 1, 24, 1, 64, 64, "int8_asym"
    rows = B * H * P
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(0, 0, B, T, H, G, P, 128)
    ost = oracle.make_state(fmt, rows, 128)
    y_orc = oracle.mamba2_scan(ost, x, dt, A, Bm, Cm, D)
    gst = par.new_gpu_state(m2desc(fmt, B, H, P))
    ys = []
    for t in range(T):
        ys.append(run_step(gst, x[:, t], dt[:, t], A, Bm[:, t], Cm[:, t], D, ssq.SSQ_READ_POST_QUANT))
    y_step = np.stack(ys, axis=1)
    g = par.read_gpu_state(gst, fmt)
    say(f"config0: code mismatches {(g['code'] != ost.code).sum()}")
    assert (g["code"] != ost.code).mean() <= 1e-4
    assert par.block_rel(y_step, y_orc, axis=(1, 3)) <= 1e-3
    assert par.block_rel(par.oracle.dequantize_rows(g["code"], g["scale"], g["zero"]), ost.dequant()) <= 1e-3
    # scan == T x decode, bit for bit
    gsc = par.new_gpu_state(m2desc(fmt, B, H, P))
    y_scan = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_scan(gsc, T, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y_scan)
    gs = par.read_gpu_state(gsc, fmt)
    assert np.array_equal(gs["code"], g["code"]) and np.array_equal(gs["scale"], g["scale"])
    assert np.array_equal(gs["zero"], g["zero"])
    assert_same_y(y_scan.cpu().numpy(), y_step, fmt)


@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_scan_equals_repeated_steps_and_oracle(fmt, readout):
    B, H, G, P, T = 2, 4, 4, 16, 24
    rows = B * H * P
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    init = init_rows(51, 2, rows)
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(51, 2, B, T, H, G, P, 128)
    say(f"scan fmt={fmt} readout={readout}")
    g1 = par.new_gpu_state(m2desc(fmt, B, H, P, G), init)
    y1 = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_scan(g1, T, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y1, ro)
    g2 = par.new_gpu_state(m2desc(fmt, B, H, P, G), init)
    y2 = np.stack([run_step(g2, x[:, t], dt[:, t], A, Bm[:, t], Cm[:, t], D, ro) for t in range(T)], axis=1)
    s1, s2 = par.read_gpu_state(g1, fmt), par.read_gpu_state(g2, fmt)
    for k in s1:
        assert np.array_equal(s1[k].view(np.uint32) if s1[k].dtype == np.float32 else s1[k],
                              s2[k].view(np.uint32) if s2[k].dtype == np.float32 else s2[k]), k
    assert_same_y(y1.cpu().numpy(), y2, fmt)
    ost = oracle.make_state(fmt, rows, 128, init)
    yo = oracle.mamba2_scan(ost, x, dt, A, Bm, Cm, D, readout=readout)
    if fmt == "fp32":
        assert np.array_equal(s1["h"], ost.h)
    else:
        assert (s1["code"] != ost.code).mean() <= 1e-4
    assert par.block_rel(y2, yo, axis=(1, 3)) <= 1e-5


@pytest.mark.parametrize("fmt", ["int8_sym", "int4_asym"])
def test_8b_decode_256_steps(fmt):
    """8B-shaped decode at batch 256 for 256 steps, free-running from a zero state (8 of the 128
    heads: every row is independent, and the full 128 heads run in the test above).  The oracle
    follows 256 sampled rows; after 256 rounded steps y stays within 1e-3 and at most 1e-4 of the
    codes differ."""
    B, H, P, T, seed = 256, 8, 64, 256, 6
    rows = B * H * P
    sample = np.unique(np.linspace(0, rows - 1, 256).astype(np.int64))
    say(f"8b decode {fmt}: {T} steps at batch {B}")
    gst = par.new_gpu_state(m2desc(fmt, B, H, P))
    ost = oracle.make_state(fmt, len(sample), 128)
    xr, dtr, Br, Cr, Ar, Dr = synth.mamba2_rows_scan_inputs(seed, 0, B, T, H, 1, P, 128, sample)
    yo = oracle.mamba2_rows_scan(ost, xr, dtr, Ar, Br, Cr, Dr)
    yg = np.empty((len(sample), T), np.float32)
    for t in range(T):
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(seed, 0, B, H, 1, P, 128, t=t)
        yg[:, t] = run_step(gst, x, dt, A, Bm, Cm, D, ssq.SSQ_READ_POST_QUANT).reshape(-1)[sample]
    assert par.block_rel(yg, yo, axis=1) <= 1e-3
    g = par.read_gpu_state(gst, fmt)
    mism = (g["code"][sample] != ost.code).mean()
    say(f"  code mismatch fraction after {T} steps: {mism}")
    assert mism <= 1e-4
    deq_g = oracle.dequantize_rows(g["code"][sample], g["scale"][sample], g["zero"][sample])
    assert par.block_rel(deq_g, ost.dequant(), axis=1) <= 1e-3


@pytest.mark.parametrize("fmt", QFORMATS)
def test_exact_ties_take_the_even_code_on_the_fast_path(fmt):
    """Rows whose new values sit exactly halfway between two codes, through ssq_decode_step's
    fast path: from a zero state with dt*A = -2^-30 (so lambda rounds to 1) and w = dt*x a
    power of two, the new row is w*B exactly; B holds the grid's two ends (0 and 2^b - 1, or
    -Qs and Qs) and values j + 1/2 in between, so the refit gives step w and those entries
    round from an exact tie.  Both sides must take the even code; x's sign and exponent vary
    by row (2^-20 .. 2^20)."""
    B, H, P, N = 2, 2, 64, 128
    rows = B * H * P
    bits, asym = oracle.FORMATS[fmt]
    top = (1 << bits) - 1 if asym else (1 << (bits - 1)) - 1
    rng = np.random.default_rng(5)
    Bm = np.empty((B, 1, N), np.float32)
    for b in range(B):
        j = rng.integers(0, top, N).astype(np.float64)
        vals = j + 0.5 if asym else (j - top // 2) + 0.5 * np.sign(rng.standard_normal(N))
        if not asym:
            vals = np.clip(vals, -top + 0.5, top - 0.5)
        vals[:8] = np.floor(vals[:8])  # a few entries on the grid itself
        vals[8], vals[9] = (0.0, float(top)) if asym else (-float(top), float(top))
        Bm[b, 0] = vals
    assert np.all(np.float32(Bm) == Bm)
    dt = np.full((B, H), 2.0 ** -30, np.float32)
    A = np.full(H, -1.0, np.float32)
    D = np.zeros(H, np.float32)
    e = rng.integers(-20, 21, (B, H, P))
    x = (np.where(rng.random((B, H, P)) < 0.5, -1.0, 1.0) * 2.0 ** (30 + e)).astype(np.float32)
    Cm = synth.normal(5, 5, 0, np.arange(B * N)).reshape(B, 1, N).astype(np.float32) / np.float32(np.sqrt(N))
    assert oracle.decay(float(dt[0, 0]), float(A[0])) == 1.0
    ost = oracle.make_state(fmt, rows, N)
    gst = par.new_gpu_state(m2desc(fmt, B, H, P))
    say(f"ties fmt={fmt}")
    yg = run_step(gst, x, dt, A, Bm, Cm, D, ssq.SSQ_READ_POST_QUANT)
    yo, hpre, vq = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, diag=True)
    # the test reaches exact ties: h*inv + z has fraction exactly 1/2 in most entries
    t = vq.astype(np.float64) + (ost.zero[:, None].astype(np.float64) if asym else 0.0)
    ties = int(np.sum(t - np.floor(t) == 0.5))
    assert ties > rows * N // 2, ties
    assert np.all(ost.code[np.abs(t - np.floor(t) - 0.5) == 0] % 2 == 0)
    g = par.read_gpu_state(gst, fmt)
    assert np.array_equal(g["code"], ost.code), int((g["code"] != ost.code).sum())
    assert np.array_equal(g["scale"].view(np.uint32), ost.scale.view(np.uint32))
    assert np.array_equal(g["zero"], ost.zero)
    assert par.block_rel(yg, yo, axis=2) <= 1e-5
    say(f"  {ties} exact ties, all on the even code on both sides")


# ---------------------------------------------------------------------------
def test_edge_shapes_and_zero_input():
    """Smallest head (P = 16), one group per head, one token, and x = 0 from a zero state
    (every row degenerate: it must stay exactly zero)."""
    for fmt in QFORMATS:
        B, H, G, P = 1, 3, 3, 16
        rows = B * H * P
        say(f"edge fmt={fmt}")
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(61, 0, B, H, G, P, 128)
        x[:] = 0
        gst = par.new_gpu_state(m2desc(fmt, B, H, P, G))
        y = run_step(gst, x, dt, A, Bm, Cm, D, ssq.SSQ_READ_POST_QUANT)
        g = par.read_gpu_state(gst, fmt)
        assert np.all(g["code"] == 0) and np.all(g["scale"] == 0) and np.all(y == 0)
        ost = oracle.make_state(fmt, rows, 128, init_rows(61, 0, rows))
        par.write_gpu_state(gst, ost)
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(61, 0, B, H, G, P, 128, t=1)
        yg = run_step(gst, x, dt, A, Bm, Cm, D, ssq.SSQ_READ_POST_QUANT)
        yo, _, vq = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, diag=True)
        par.check_codes(par.read_gpu_state(gst, fmt), ost.code, ost.scale, ost.zero, vq, fmt, fmt)
        assert par.block_rel(yg, yo, axis=2) <= 1e-5


@pytest.mark.parametrize("fmt", ["fp32", "int8_asym", "int4_asym", "int8_sym"])
def test_non_finite_inputs_stay_in_their_rows(fmt):
    """NaN and infinity in x (two rows) and an infinite dt (one head of one sequence): the call
    completes, and every row those values do not reach matches the oracle run on clean inputs."""
    B, H, G, P = 2, 4, 1, 16
    rows = B * H * P
    say(f"non-finite fmt={fmt}")
    init = init_rows(44, 0, rows)
    ost = oracle.make_state(fmt, rows, 128, init)
    gst = par.new_gpu_state(m2desc(fmt, B, H, P, G))
    par.write_gpu_state(gst, ost)
    x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(44, 0, B, H, G, P, 128)
    yo, _, vq = oracle.mamba2_step(ost, x, dt, A, Bm, Cm, D, diag=True)
    xb, dtb = x.copy(), dt.copy()
    xb[0, 1, 3] = np.nan
    xb[1, 2, 5] = np.inf
    dtb[1, 3] = np.inf
    yg = run_step(gst, xb, dtb, A, Bm, Cm, D, ssq.SSQ_READ_POST_QUANT)
    torch.cuda.synchronize()
    bad = np.zeros((B, H, P), bool)
    bad[0, 1, 3] = bad[1, 2, 5] = True
    bad[1, 3, :] = True
    ok = ~bad.reshape(-1)
    g = par.read_gpu_state(gst, fmt)
    if fmt == "fp32":
        assert np.array_equal(g["h"][ok], ost.h[ok])
    else:
        par.check_codes({k: v[ok] for k, v in g.items()}, ost.code[ok], ost.scale[ok], ost.zero[ok], vq[ok], fmt,
                        "finite rows")
    assert par.block_rel(yg.reshape(-1)[ok], yo.reshape(-1)[ok]) <= 1e-5


def test_repeat_runs_are_bit_identical():
    B, H, P, fmt = 4, 8, 64, "int4_asym"
    rows = B * H * P
    init = init_rows(71, 0, rows)
    x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(71, 0, B, H, 1, P, 128)
    outs = []
    for _ in range(2):
        gst = par.new_gpu_state(m2desc(fmt, B, H, P), init)
        y = run_step(gst, x, dt, A, Bm, Cm, D, ssq.SSQ_READ_POST_QUANT)
        torch.cuda.synchronize()
        outs.append((gst.storage.cpu().numpy().copy(), y))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1].view(np.uint32),
                                                                      outs[1][1].view(np.uint32))


def test_errors_leave_the_state_unchanged():
    B, H, P, fmt = 2, 2, 16, "int8_asym"
    gst = par.new_gpu_state(m2desc(fmt, B, H, P), init_rows(81, 0, B * H * P, special=False))
    before = gst.storage.cpu().numpy().copy()
    q = torch.zeros(B * H * 128, device="cuda")
    with pytest.raises(ssq.SsqError) as e:
        ssq.ssq_delta_step(gst, q, q, q, torch.zeros(B * H, device="cuda"), torch.zeros(B * H, device="cuda"), q)
    assert e.value.status == ssq.SSQ_ERR_KIND_MISMATCH
    x = torch.zeros(B * H * P, device="cuda")
    with pytest.raises(ValueError):  # short buffer caught by the binding
        ssq.ssq_decode_step(gst, x[:-1], x[:B * H], x[:H], q[:B * 128], q[:B * 128], x[:H], x)
    import ctypes
    bad = ssq.lib.ssq_scan(gst.handle, 0, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                           ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                           ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                           ctypes.c_void_p(x.data_ptr()), 0, None)
    assert bad == ssq.SSQ_ERR_INVALID_ARG
    assert np.array_equal(gst.storage.cpu().numpy(), before)


def test_library_owned_storage():
    d = m2desc("int4_asym", 2, 2, 16)
    st = ssq.ssq_alloc_state(d)
    _, ptr, lay = ssq.ssq_state_info(st)
    assert ptr and lay.total_bytes == ssq.ssq_state_bytes(d)
    x = torch.zeros(2 * 2 * 16, device="cuda")
    ssq.ssq_decode_step(st, x, torch.ones(4, device="cuda"), -torch.ones(2, device="cuda"),
                        torch.zeros(256, device="cuda"), torch.zeros(256, device="cuda"), torch.zeros(2, device="cuda"),
                        x)
    out = torch.empty(2 * 2 * 16 * 128, device="cuda")
    ssq.ssq_dequant(st, out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    st.free()
