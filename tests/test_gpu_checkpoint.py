"""GPU: a state's storage bytes plus its rounding settings are a complete checkpoint.  T tokens
on one state give bit for bit what T/2 tokens, a copy of the storage to the host, a new
handle over fresh caller-owned storage holding those bytes, and T/2 more tokens give (the
outputs of the second half and the final bytes).  The fixed-size per-request state is
what a server keeps per request ("Recurrent state is fixed per request, not free"), so
saving it must need nothing the layout does not describe.  Through the C ABI."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mamba_decode_amd as ssq
    from tests import parity as par

B, H, P, T = 2, 4, 64, 6


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def new_state(desc, init, storage=None):
    if storage is None:
        storage = torch.empty(ssq.ssq_state_bytes(desc), dtype=torch.uint8, device="cuda")
    st = ssq.ssq_alloc_state(desc, storage=storage, init=None if init is None else par.dev(init))
    return st, storage


def mamba2_tokens(st, seed, t0, t1, scan):
    """Tokens t0 .. t1-1 as decode steps, or as one scan; the outputs, token-major."""
    steps = [synth.mamba2_step_inputs(seed, 0, B, H, 1, P, 128, t=t) for t in range(t0, t1)]
    if not scan:
        ys = []
        for x, dt, Bm, Cm, A, D in steps:
            y = torch.empty(B * H * P, device="cuda")
            ssq.ssq_decode_step(st, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
            ys.append(y)
        return torch.cat(ys).cpu().numpy()
    n = t1 - t0
    # [B][T][...] sequence layout from the per-token inputs
    x = np.stack([s[0].reshape(B, H * P) for s in steps], axis=1)
    dt = np.stack([s[1].reshape(B, H) for s in steps], axis=1)
    Bm = np.stack([s[2].reshape(B, 128) for s in steps], axis=1)
    Cm = np.stack([s[3].reshape(B, 128) for s in steps], axis=1)
    A, D = steps[0][4], steps[0][5]
    y = torch.empty(B * n * H * P, device="cuda")
    ssq.ssq_scan(st, n, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
    return np.ascontiguousarray(y.cpu().numpy().reshape(B, n, H * P).transpose(1, 0, 2)).ravel()  # token-major


def delta_tokens(st, seed, t0, t1):
    os_ = []
    for t in range(t0, t1):
        q, k, v, al, be = synth.delta_inputs(seed, 0, B, H, 128, 128, t=t)
        o = torch.empty(B * H * 128, device="cuda")
        ssq.ssq_delta_step(st, par.dev(q), par.dev(k), par.dev(v), par.dev(al), par.dev(be), o)
        os_.append(o)
    return torch.cat(os_).cpu().numpy()


CASES = [("m2", "int4_asym", False, False), ("m2", "int8_sym", False, False), ("m2", "fp32", False, False),
         ("m2", "int4_asym", True, False), ("m2", "int8_asym", True, True), ("m2", "int8_sym", False, True),
         ("delta", "int8_asym", False, False), ("delta", "int8_asym", True, False), ("delta", "damp", True, False)]


@pytest.mark.parametrize("kind,fmt,stochastic,scan", CASES)
def test_checkpoint_and_resume_is_bit_identical(kind, fmt, stochastic, scan):
    say(f"checkpoint: {kind} {fmt} stochastic={stochastic} scan={scan}")
    seed = 120 + CASES.index((kind, fmt, stochastic, scan))
    if kind == "m2":
        desc = ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P)
        init = synth.init_state(seed, 0, B * H * P, 128)
        run = lambda st, t0, t1: mamba2_tokens(st, seed, t0, t1, scan)  # noqa: E731
    else:
        desc = ssq.make_desc(ssq.SSQ_DELTA, fmt, B, H, 128, 128)
        init = synth.init_state(seed, 0, B * H * 128, 128)
        run = lambda st, t0, t1: delta_tokens(st, seed, t0, t1)  # noqa: E731

    def rounding(st):
        if stochastic:
            ssq.ssq_set_rounding(st, ssq.SSQ_ROUND_STOCHASTIC, seed=0x5EED0000 + seed, step=3)

    # uninterrupted
    sa, store_a = new_state(desc, init)
    rounding(sa)
    out_a = run(sa, 0, T)
    torch.cuda.synchronize()
    bytes_a = store_a.cpu().numpy().copy()

    # first half, then the checkpoint: the storage bytes and the rounding settings
    sb, store_b = new_state(desc, init)
    rounding(sb)
    out_b1 = run(sb, 0, T // 2)
    torch.cuda.synchronize()
    saved = store_b.cpu().numpy().copy()
    mode, sd, nxt = ssq.ssq_get_rounding(sb)
    assert nxt == (3 + T // 2 if stochastic else 0)
    sb.free()
    store_b.fill_(0xA5)  # the old storage is gone
    del store_b

    # restore into fresh caller-owned storage under a new handle
    sc, store_c = new_state(desc, None)
    torch.cuda.synchronize()
    store_c.copy_(torch.from_numpy(saved).cuda())
    ssq.ssq_set_rounding(sc, mode, sd, nxt)
    out_c2 = run(sc, T // 2, T)
    torch.cuda.synchronize()

    half = out_a.size // 2
    assert np.array_equal(out_b1.view(np.uint32), out_a[:half].view(np.uint32))
    assert np.array_equal(out_c2.view(np.uint32), out_a[half:].view(np.uint32))
    assert np.array_equal(store_c.cpu().numpy(), bytes_a)
    assert ssq.ssq_get_rounding(sc)[2] == ssq.ssq_get_rounding(sa)[2]
    sa.free()
    sc.free()
