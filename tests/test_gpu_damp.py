"""GPU parity of the two-tier delta state (SSQ_DAMP: half rows 0..15, uint8 rows 16..127,
rows rotated by H_128/16) against the CPU oracle, through the C ABI."""
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

NHI = 16


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def ddesc(B, H):
    return ssq.make_desc(ssq.SSQ_DELTA, "damp", B, H, 128, 128)


def run(gst, q, k, v, al, be, readout=None):
    o = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ro = ssq.SSQ_READ_POST_QUANT if readout is None else readout
    ssq.ssq_delta_step(gst, par.dev(q), par.dev(k), par.dev(v), par.dev(al), par.dev(be), o, ro)
    return o.cpu().numpy()


def check(g, ost, where, exact=False, pre=None):
    """uint8 codes per the contract (at most 1e-4 differ, by one), scales and zero points equal
    outside such rows; half rows at most 1e-4 differ, each by one half ulp."""
    dc = g["code"] != ost.code
    assert dc.mean() <= (0 if exact else 1e-4), where
    assert np.all(np.abs(g["code"] - ost.code)[dc] == 1), where
    same = ~dc.any(axis=1)
    assert np.array_equal(g["scale"][same], ost.scale[same]) and np.array_equal(g["zero"][same], ost.zero[same]), where
    dh = g["hi"] != ost.hi
    if dh.any():
        idx = np.argwhere(dh)[:8]
        info = [(tuple(int(v) for v in ix), float(g["hi"][tuple(ix)]), float(ost.hi[tuple(ix)]),
                 None if pre is None else float(pre[ix[0], ix[1], ix[2]])) for ix in idx]
        say(f"  {where}: {int(dh.sum())} half values differ: {info}")
    assert dh.mean() <= (0 if exact else 1e-4), where
    if dh.any():
        a, b = g["hi"][dh].astype(np.float16), ost.hi[dh].astype(np.float16)
        assert np.all(np.abs(a.view(np.int16).astype(int) - b.view(np.int16).astype(int)) == 1), where


def hadamard_s():
    Hm = np.array([[1.0]])
    while Hm.shape[0] < 128:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm / 16.0


def test_init_and_dequant():
    B, H = 2, 3
    S0 = synth.init_state(81, 0, B * H * 128, 128)
    say("damp init")
    gst = par.new_gpu_state(ddesc(B, H), S0)
    ost = oracle.damp_from_fp32(S0.reshape(B, H, 128, 128), B, H)
    check(par.read_gpu_damp(gst), ost, "init", exact=True)
    out = torch.empty(B * H * 128 * 128, dtype=torch.float32, device="cuda")
    ssq.ssq_dequant(gst, out)
    deq = out.cpu().numpy().reshape(B * H, 128, 128).astype(np.float64)
    ref = 2.0 * ost.rotated().astype(np.float64) @ hadamard_s()
    assert par.block_rel(deq, ref, axis=(1, 2)) <= 1e-6
    # the reconstruction of the start is close to the fp32 state it was built from
    assert par.block_rel(deq, S0.reshape(B * H, 128, 128), axis=2) <= 5e-2


@pytest.mark.parametrize("readout", ["post", "pre"])
def test_step_teacher_forced(readout):
    B, H, T = 2, 3, 3
    ro = ssq.SSQ_READ_PRE_QUANT if readout == "pre" else ssq.SSQ_READ_POST_QUANT
    S0 = synth.init_state(82, 0, B * H * 128, 128)
    S0[3] = 0.0  # a zero half row
    S0[140] = 1.25  # a constant uint8 row (of matrix 1)
    ost = oracle.damp_from_fp32(S0.reshape(B, H, 128, 128), B, H)
    gst = par.new_gpu_state(ddesc(B, H))
    for t in range(T):
        say(f"damp teacher-forced readout={readout} t={t}")
        q, k, v, al, be = synth.delta_inputs(82, 0, B, H, 128, 128, t=t)
        par.write_gpu_damp(gst, ost)
        og = run(gst, q, k, v, al, be, ro)
        oo, Spre = oracle.damp_step(ost, q, k, v, al, be, B, H, readout=readout, diag=True)
        check(par.read_gpu_damp(gst), ost, f"t={t}", pre=Spre)
        assert par.block_rel(og, oo, axis=2) <= 1e-5, t


def test_step_stochastic():
    B, H = 2, 2
    S0 = synth.init_state(83, 0, B * H * 128, 128)
    ost = oracle.damp_from_fp32(S0.reshape(B, H, 128, 128), B, H)
    gst = par.new_gpu_state(ddesc(B, H), S0)
    ssq.ssq_set_rounding(gst, ssq.SSQ_ROUND_STOCHASTIC, 21, 4)
    q, k, v, al, be = synth.delta_inputs(83, 0, B, H, 128, 128)
    og = run(gst, q, k, v, al, be)
    oo = oracle.damp_step(ost, q, k, v, al, be, B, H, sr=(21, 4))
    check(par.read_gpu_damp(gst), ost, "stochastic", exact=True)
    assert par.block_rel(og, oo, axis=2) <= 1e-5
    with pytest.raises(ssq.SsqError):
        ssq.ssq_kda_step(gst, par.dev(q), par.dev(k), par.dev(v), par.dev(np.ones((B, H, 128), np.float32)),
                         par.dev(be), torch.empty(v.shape, dtype=torch.float32, device="cuda"))


def test_full_layer_sampled():
    """The two-tier layer at the profiled footprint: batch 256 x 32 heads x 128 x 128, one step
    from a seeded random state; 32 sampled matrices checked."""
    B, H = 256, 32
    mats = np.unique(np.linspace(0, B * H - 1, 32).astype(np.int64))
    say("damp full layer: init")
    S0 = synth.init_state(7, 0, B * H * 128, 128, threads=8)
    gst = par.new_gpu_state(ddesc(B, H), S0)
    ost = oracle.damp_from_fp32(S0.reshape(B * H, 128, 128)[mats][None], 1, len(mats))
    del S0
    q, k, v, al, be = synth.delta_inputs(7, 0, B, H, 128, 128)
    say("damp full layer: step")
    og = run(gst, q, k, v, al, be).reshape(B * H, 128)
    sel = lambda a: a.reshape(B * H, *a.shape[2:])[mats][None]  # noqa: E731
    oo = oracle.damp_step(ost, sel(q), sel(k), sel(v), al.reshape(-1)[mats][None], be.reshape(-1)[mats][None],
                          1, len(mats))
    g = par.read_gpu_damp(gst)
    lo = (mats[:, None] * 112 + np.arange(112)).reshape(-1)
    sub = {"code": g["code"][lo], "scale": g["scale"][lo], "zero": g["zero"][lo], "hi": g["hi"][mats]}
    check(sub, ost, "full layer")
    assert par.block_rel(og[mats], oo[0], axis=1) <= 1e-5
