"""GPU parity of the delta-rule path (ssq_delta_step) against the CPU oracle, through the C ABI."""
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def ddesc(fmt, B, H):
    return ssq.make_desc(ssq.SSQ_DELTA, fmt, B, H, 128, 128)


def run_delta(gst, q, k, v, al, be, readout):
    o = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_delta_step(gst, par.dev(q), par.dev(k), par.dev(v), par.dev(al), par.dev(be), o, readout)
    return o.cpu().numpy()


def u_tie_rows(ost_before, k, B, H):
    """Key rows whose update read a column sum u_j = k^T S that lies near an fp32 rounding midpoint
    (there the double-precision sums of the two sides may round u differently).  Returns a
    boolean per matrix: True if some column of that matrix is near a midpoint."""
    if ost_before.fmt == "fp32":
        S = ost_before.h.astype(np.float64)
    else:
        S = ost_before.scale.astype(np.float64)[:, None] * (ost_before.code - ost_before.zero[:, None])
    S = S.reshape(B * H, 128, 128)
    u = np.einsum("mi,mij->mj", k.reshape(B * H, 128).astype(np.float64), S)
    uf = u.astype(np.float32)
    nxt = np.nextafter(uf, np.where(u > uf, np.inf, -np.inf).astype(np.float32))
    mid = (uf.astype(np.float64) + nxt.astype(np.float64)) / 2
    near = np.abs(u - mid) <= np.abs(u) * 2.0 ** -40
    return near.any(axis=1)


@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_delta_step_teacher_forced(fmt, readout):
    B, H, T = 2, 3, 4
    rows = B * H * 128
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    init = synth.init_state(91, 0, rows, 128)
    init[5] = 0.0          # a degenerate key row
    init[200] = 2.5        # a constant key row
    ost = oracle.make_state(fmt, rows, 128, init)
    gst = par.new_gpu_state(ddesc(fmt, B, H))
    for t in range(T):
        say(f"delta teacher-forced fmt={fmt} readout={readout} t={t}")
        q, k, v, al, be = synth.delta_inputs(91, 0, B, H, 128, 128, t=t)
        par.write_gpu_state(gst, ost)
        before = ost.copy()
        og = run_delta(gst, q, k, v, al, be, ro)
        oo, _, vq = oracle.delta_step(ost, q, k, v, al, be, B, H, readout=readout, diag=True)
        g = par.read_gpu_state(gst, fmt)
        if fmt == "fp32":
            tie = u_tie_rows(before, k, B, H)
            same = np.array_equal(g["h"], ost.h)
            if not same:
                bad = np.unique(np.nonzero((g["h"] != ost.h).any(axis=1))[0] // 128)
                assert np.all(tie[bad]), t
        else:
            par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, f"t={t}")
        assert par.block_rel(og, oo, axis=2) <= 1e-5, t


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym"])
@pytest.mark.parametrize("mag", [2.0 ** -118, 2.0 ** 100])
def test_delta_step_far_from_unit_scale(mag, fmt, kda):
    """States, v and part of k far from unit size: the reconstructed entries sit near 2^-118
    or 2^100 (down to the subnormal range for the smallest), the products k_i*Sh_ij of u near
    2^-180 or 2^100, and some keys are tiny; the double accumulation of u, the update and the
    refit must still match the oracle under the contract."""
    B, H = 2, 2
    rows = B * H * 128
    init = (synth.init_state(98, 0, rows, 128).astype(np.float64) * mag).astype(np.float32)
    ost = oracle.make_state(fmt, rows, 128, init)
    gst = par.new_gpu_state(ddesc(fmt, B, H))
    q, k, v, al, be = synth.delta_inputs(98, 0, B, H, 128, 128)
    v = (v.astype(np.float64) * mag).astype(np.float32)
    k = k.copy()
    k.reshape(B * H, 128)[:, ::5] *= np.float32(2.0 ** -60)
    say(f"delta far from unit scale mag=2^{int(np.log2(mag))} fmt={fmt} kda={kda}")
    par.write_gpu_state(gst, ost)
    if kda:
        al = synth.kda_alpha(98, 0, B, H, 128)
        og = run_kda(gst, q, k, v, al, be, ssq.SSQ_READ_POST_QUANT)
        oo, _, vq = oracle.kda_step(ost, q, k, v, al, be, B, H, readout="post", diag=True)
    else:
        og = run_delta(gst, q, k, v, al, be, ssq.SSQ_READ_POST_QUANT)
        oo, _, vq = oracle.delta_step(ost, q, k, v, al, be, B, H, readout="post", diag=True)
    g = par.read_gpu_state(gst, fmt)
    assert np.all(np.isfinite(ost.scale)) and np.all(ost.scale > 0)
    par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, "far from unit scale")
    assert par.block_rel(og, oo, axis=2) <= 1e-5


def test_delta_identity_and_decay_on_gpu():
    """alpha = beta = 1 with unit k writes v at key k (fp32 state); beta = 0 is a pure decay
    that keeps the codes of full-range rows."""
    B, H = 2, 2
    rows = B * H * 128
    q, k, v, al, be = synth.delta_inputs(92, 0, B, H, 128, 128)
    al[:] = 1
    be[:] = 1
    gst = par.new_gpu_state(ddesc("fp32", B, H), synth.init_state(92, 0, rows, 128))
    o = run_delta(gst, k, k, v, al, be, ssq.SSQ_READ_POST_QUANT)
    assert par.block_rel(o, v) <= 1e-5
    init = synth.init_state(93, 0, rows, 128)
    g8 = par.new_gpu_state(ddesc("int8_asym", B, H), init)
    c0 = par.read_gpu_state(g8, "int8_asym")
    full = c0["code"].max(axis=1) == 255
    q, k, v, al, be = synth.delta_inputs(93, 0, B, H, 128, 128)
    be[:] = 0
    run_delta(g8, q, k, v, al, be, ssq.SSQ_READ_POST_QUANT)
    c1 = par.read_gpu_state(g8, "int8_asym")
    assert np.array_equal(c1["code"][full], c0["code"][full]) and np.array_equal(c1["zero"][full], c0["zero"][full])


def test_delta_layer_full_size_sampled():
    """Delta-rule layer at the footprint the pages profile: batch 256 x 32 heads x 128 x 128, int8
    asymmetric state from a seeded random state, one step; 48 sampled matrices checked."""
    B, H, fmt = 256, 32, "int8_asym"
    rows = B * H * 128
    say("delta full layer: generating init")
    init = synth.init_state(3, 0, rows, 128, threads=8)
    gst = par.new_gpu_state(ddesc(fmt, B, H), init)
    mats = np.unique(np.linspace(0, B * H - 1, 48).astype(np.int64))
    srows = (mats[:, None] * 128 + np.arange(128)).reshape(-1)
    ost = oracle.make_state(fmt, len(srows), 128, init[srows])
    del init
    g0 = par.read_gpu_state(gst, fmt)
    assert np.array_equal(g0["code"][srows], ost.code)
    q, k, v, al, be = synth.delta_inputs(3, 0, B, H, 128, 128)
    say("delta full layer: step")
    og = run_delta(gst, q, k, v, al, be, ssq.SSQ_READ_POST_QUANT).reshape(B * H, 128)
    sel = lambda a: a.reshape(B * H, *a.shape[2:])[mats][None]  # noqa: E731
    oo, _, vq = oracle.delta_step(ost, sel(q), sel(k), sel(v), al.reshape(-1)[mats][None],
                                  be.reshape(-1)[mats][None], 1, len(mats), diag=True)
    g = par.read_gpu_state(gst, fmt)
    sub = {"code": g["code"][srows], "scale": g["scale"][srows], "zero": g["zero"][srows]}
    par.check_codes(sub, ost.code, ost.scale, ost.zero, vq, fmt, "full layer")
    assert par.block_rel(og[mats], oo[0], axis=1) <= 1e-5


# ---------------------------------------------------------------------------
# KDA-style step: a decay per key channel (ssq_kda_step)
# ---------------------------------------------------------------------------
def run_kda(gst, q, k, v, al, be, readout):
    o = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_kda_step(gst, par.dev(q), par.dev(k), par.dev(v), par.dev(al), par.dev(be), o, readout)
    return o.cpu().numpy()


@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_kda_step_teacher_forced(fmt, readout):
    B, H, T = 2, 3, 3
    rows = B * H * 128
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    init = synth.init_state(95, 0, rows, 128)
    init[7] = 0.0
    init[300] = -1.5
    ost = oracle.make_state(fmt, rows, 128, init)
    gst = par.new_gpu_state(ddesc(fmt, B, H))
    for t in range(T):
        say(f"kda teacher-forced fmt={fmt} readout={readout} t={t}")
        q, k, v, _, be = synth.delta_inputs(95, 0, B, H, 128, 128, t=t)
        al = synth.kda_alpha(95, 0, B, H, 128, t=t)
        par.write_gpu_state(gst, ost)
        before = ost.copy()
        og = run_kda(gst, q, k, v, al, be, ro)
        oo, _, vq = oracle.kda_step(ost, q, k, v, al, be, B, H, readout=readout, diag=True)
        g = par.read_gpu_state(gst, fmt)
        if fmt == "fp32":
            tie = u_tie_rows(before, k * al, B, H)  # u = (k*alpha)^T S
            if not np.array_equal(g["h"], ost.h):
                bad = np.unique(np.nonzero((g["h"] != ost.h).any(axis=1))[0] // 128)
                assert np.all(tie[bad]), t
        else:
            par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, f"t={t}")
        assert par.block_rel(og, oo, axis=2) <= 1e-5, t


def test_kda_layer_full_size_sampled_with_stochastic_rounding():
    """KDA-style layer at the profiled footprint (batch 256 x 32 heads x 128 x 128, int8
    asymmetric), one round-to-nearest step then one stochastic step; 32 sampled matrices."""
    B, H, fmt = 256, 32, "int8_asym"
    rows = B * H * 128
    say("kda full layer: generating init")
    init = synth.init_state(6, 0, rows, 128, threads=8)
    gst = par.new_gpu_state(ddesc(fmt, B, H), init)
    mats = np.unique(np.linspace(0, B * H - 1, 32).astype(np.int64))
    srows = (mats[:, None] * 128 + np.arange(128)).reshape(-1)
    # the sampled matrices' rows, indexed as their own small state, with their state row ids
    ost = oracle.make_state(fmt, len(srows), 128, init[srows])
    del init
    sel = lambda a: a.reshape(B * H, *a.shape[2:])[mats][None]  # noqa: E731
    for t, sr in enumerate([None, (77, 12)]):
        say(f"kda full layer: step {t}")
        if sr is not None:
            ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, *sr)
        q, k, v, _, be = synth.delta_inputs(6, 0, B, H, 128, 128, t=t)
        al = synth.kda_alpha(6, 0, B, H, 128, t=t)
        og = run_kda(gst, q, k, v, al, be, ssq.SSQ_READ_POST_QUANT).reshape(B * H, 128)
        if sr is None:
            oo, _, vq = oracle.kda_step(ost, sel(q), sel(k), sel(v), sel(al), be.reshape(-1)[mats][None],
                                        1, len(mats), diag=True)
        else:
            # the oracle draws per state row: run each sampled matrix as matrix m of the full layer
            oo = np.empty((1, len(mats), 128), np.float32)
            for i, m in enumerate(mats):
                one = oracle.make_state(fmt, 128, 128)
                one.code, one.scale, one.zero = (ost.code[i * 128:(i + 1) * 128].copy(),
                                                 ost.scale[i * 128:(i + 1) * 128].copy(),
                                                 ost.zero[i * 128:(i + 1) * 128].copy())
                # a full-layer state row index enters only through the uniforms' counter
                U = np.stack([oracle.sr_row_uniforms(sr[0], sr[1], rows, m * 128 + r, 128) for r in range(128)])
                _, Spre, _ = oracle.kda_step(one.copy(), sel(q)[:, i:i + 1], sel(k)[:, i:i + 1],
                                             sel(v)[:, i:i + 1], sel(al)[:, i:i + 1],
                                             be.reshape(-1)[[m]][None], 1, 1, diag=True)
                for r in range(128):
                    c, s_, z_ = oracle.quantize_row_sr(Spre[r], fmt, U[r])
                    one.code[r], one.scale[r], one.zero[r] = c, s_, z_
                deq = one.dequant().astype(np.float64)
                oo[0, i] = (deq * sel(q)[0, i].astype(np.float64)[:, None]).sum(axis=0)
                ost.code[i * 128:(i + 1) * 128] = one.code
                ost.scale[i * 128:(i + 1) * 128] = one.scale
                ost.zero[i * 128:(i + 1) * 128] = one.zero
        g = par.read_gpu_state(gst, fmt)
        sub = {"code": g["code"][srows], "scale": g["scale"][srows], "zero": g["zero"][srows]}
        if sr is None:
            par.check_codes(sub, ost.code, ost.scale, ost.zero, vq, fmt, "kda full layer")
            # continue from the GPU's state so that the stochastic step starts from the same codes
            ost.code, ost.scale, ost.zero = sub["code"].copy(), sub["scale"].copy(), sub["zero"].copy()
        else:
            assert np.array_equal(sub["code"], ost.code)
            assert np.array_equal(sub["scale"], ost.scale) and np.array_equal(sub["zero"], ost.zero)
        assert par.block_rel(og[mats], oo[0], axis=1) <= 1e-5


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_sym", "fp32"])
def test_non_finite_inputs_stay_in_their_matrix(fmt):
    """A NaN in v of one matrix and an infinite beta of another: the call completes, and every
    other matrix matches the oracle run on clean inputs."""
    B, H = 2, 3
    rows = B * H * 128
    say(f"delta non-finite fmt={fmt}")
    init = synth.init_state(92, 0, rows, 128)
    ost = oracle.make_state(fmt, rows, 128, init)
    gst = par.new_gpu_state(ddesc(fmt, B, H))
    par.write_gpu_state(gst, ost)
    q, k, v, al, be = synth.delta_inputs(92, 0, B, H, 128, 128)
    oo, _, vq = oracle.delta_step(ost, q, k, v, al, be, B, H, diag=True)
    vb, beb = v.copy(), be.copy()
    vb[0, 1, 7] = np.nan
    beb[1, 2] = np.inf
    og = run_delta(gst, q, k, vb, al, beb, ssq.SSQ_READ_POST_QUANT)
    torch.cuda.synchronize()
    okm = np.ones((B, H), bool)
    okm[0, 1] = okm[1, 2] = False
    okr = np.repeat(okm.reshape(-1), 128)
    g = par.read_gpu_state(gst, fmt)
    if fmt == "fp32":
        assert par.block_rel(g["h"][okr], ost.h[okr]) <= 1e-5
    else:
        par.check_codes({kk: vv[okr] for kk, vv in g.items()}, ost.code[okr], ost.scale[okr], ost.zero[okr],
                        vq[okr], fmt, "finite matrices")
    assert par.block_rel(og[okm], oo[okm], axis=-1) <= 1e-5
