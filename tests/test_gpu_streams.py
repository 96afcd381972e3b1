"""GPU: calls on different states, enqueued on different streams, run concurrently and each
gives the oracle's result: the library keeps no state between calls beyond the state
handles themselves.  Through the C ABI."""
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_three_states_on_three_streams():
    B, H, P, T = 2, 4, 64, 3
    rows = B * H * P
    fmts = ["int4_asym", "int8_sym"]
    osts, gsts, ins = [], [], []
    for n, fmt in enumerate(fmts):
        init = synth.init_state(81 + n, 0, rows, 128)
        osts.append(oracle.make_state(fmt, rows, 128, init))
        gsts.append(par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P), init))
        ins.append([synth.mamba2_step_inputs(81 + n, 0, B, H, 1, P, 128, t=t) for t in range(T)])
    dinit = synth.init_state(90, 0, B * H * 128, 128)
    dost = oracle.make_state("int8_asym", B * H * 128, 128, dinit)
    dgst = par.new_gpu_state(ssq.make_desc(ssq.SSQ_DELTA, "int8_asym", B, H, 128, 128), dinit)
    dins = [synth.delta_inputs(90, 0, B, H, 128, 128, t=t) for t in range(T)]

    dev_ins = [[tuple(par.dev(a) for a in step) for step in per] for per in ins]
    dev_dins = [tuple(par.dev(a) for a in step) for step in dins]
    ys = [[torch.empty(rows, device="cuda") for _ in range(T)] for _ in fmts]
    os_ = [torch.empty(B * H * 128, device="cuda") for _ in range(T)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    say("three states on three streams: enqueue")
    for t in range(T):  # interleaved enqueueing: the streams' calls overlap on the GPU
        for n in range(2):
            with torch.cuda.stream(streams[n]):
                x, dt, Bm, Cm, A, D = dev_ins[n][t]
                ssq.ssq_decode_step(gsts[n], x, dt, A, Bm, Cm, D, ys[n][t])
        with torch.cuda.stream(streams[2]):
            q, k, v, al, be = dev_dins[t]
            ssq.ssq_delta_step(dgst, q, k, v, al, be, os_[t])
    torch.cuda.synchronize()
    for n, fmt in enumerate(fmts):
        for t in range(T):
            x, dt, Bm, Cm, A, D = ins[n][t]
            yo = oracle.mamba2_step(osts[n], x, dt, A, Bm, Cm, D)
            assert par.block_rel(ys[n][t].cpu().numpy().reshape(yo.shape), yo, axis=2) <= 1e-5, (fmt, t)
        g = par.read_gpu_state(gsts[n], fmt)
        assert np.array_equal(g["code"], osts[n].code), fmt
        assert np.array_equal(g["scale"].view(np.uint32), osts[n].scale.view(np.uint32)), fmt
    for t in range(T):
        q, k, v, al, be = dins[t]
        oo = oracle.delta_step(dost, q, k, v, al, be, B, H)
        assert par.block_rel(os_[t].cpu().numpy().reshape(oo.shape), oo, axis=2) <= 1e-5, t
    g = par.read_gpu_state(dgst, "int8_asym")
    assert np.array_equal(g["code"], dost.code)
