"""GPU: the calls captured in a HIP graph (as the bench replays them) give, on every replay, the
eager result bit for bit.  Each replay starts from the same state, restored by an eager copy
outside the graph, with the program's own synchronizations between replays."""
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


def _check_replays(st, start, eager_state, eager_out, out, graph, where):
    for rep in range(3):
        st.storage.copy_(start)          # eager work between replays
        torch.cuda.synchronize()
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.storage, eager_state), f"{where}: state differs on replay {rep}"
        assert torch.equal(out, eager_out), f"{where}: output differs on replay {rep}"


def _capture(fn):
    fn()  # warm the launch path outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("fmt", ["int4_asym", "int8_sym", "int8_asym", "fp32"])
def test_decode_step_in_a_graph(fmt):
    B, H, P = 4, 8, 64
    rows = B * H * P
    say(f"graph decode {fmt}")
    st = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P), synth.init_state(71, 0, rows, 128))
    x, dt, Bm, Cm, A, D = (par.dev(a) for a in synth.mamba2_step_inputs(71, 0, B, H, 1, P, 128))
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    start = st.storage.clone()
    ssq.ssq_decode_step(st, x, dt, A, Bm, Cm, D, y)
    torch.cuda.synchronize()
    eager_state, eager_y = st.storage.clone(), y.clone()
    st.storage.copy_(start)
    g = _capture(lambda: ssq.ssq_decode_step(st, x, dt, A, Bm, Cm, D, y))
    _check_replays(st, start, eager_state, eager_y, y, g, f"decode {fmt}")


@pytest.mark.parametrize("fmt", ["int8_asym", "damp"])
def test_delta_step_in_a_graph(fmt):
    B, H = 2, 4
    rows = B * H * 128
    say(f"graph delta {fmt}")
    st = par.new_gpu_state(ssq.make_desc(ssq.SSQ_DELTA, fmt, B, H, 128, 128), synth.init_state(72, 0, rows, 128))
    q, k, v, al, be = (par.dev(a) for a in synth.delta_inputs(72, 0, B, H, 128, 128))
    o = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    start = st.storage.clone()
    ssq.ssq_delta_step(st, q, k, v, al, be, o)
    torch.cuda.synchronize()
    eager_state, eager_o = st.storage.clone(), o.clone()
    st.storage.copy_(start)
    g = _capture(lambda: ssq.ssq_delta_step(st, q, k, v, al, be, o))
    _check_replays(st, start, eager_state, eager_o, o, g, f"delta {fmt}")


def test_scan_in_a_graph():
    B, H, P, T = 2, 4, 32, 16
    rows = B * H * P
    say("graph scan")
    st = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, "int8_asym", B, H, P), synth.init_state(73, 0, rows, 128))
    x, dt, Bm, Cm, A, D = (par.dev(a) for a in synth.mamba2_scan_inputs(73, 0, B, T, H, 1, P, 128))
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    start = st.storage.clone()
    ssq.ssq_scan(st, T, x, dt, A, Bm, Cm, D, y)
    torch.cuda.synchronize()
    eager_state, eager_y = st.storage.clone(), y.clone()
    st.storage.copy_(start)
    g = _capture(lambda: ssq.ssq_scan(st, T, x, dt, A, Bm, Cm, D, y))
    _check_replays(st, start, eager_state, eager_y, y, g, "scan")


def test_prefill_in_a_graph():
    B, H, P, T, chunk = 2, 4, 64, 40, 16
    rows = B * H * P
    say("graph prefill")
    st = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, "int8_asym", B, H, P), synth.init_state(74, 0, rows, 128))
    x, dt, Bm, Cm, A, D = (par.dev(a) for a in synth.mamba2_scan_inputs(74, 0, B, T, H, 1, P, 128))
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    start = st.storage.clone()
    ssq.ssq_prefill(st, T, chunk, x, dt, A, Bm, Cm, D, y)
    torch.cuda.synchronize()
    eager_state, eager_y = st.storage.clone(), y.clone()
    st.storage.copy_(start)
    g = _capture(lambda: ssq.ssq_prefill(st, T, chunk, x, dt, A, Bm, Cm, D, y))
    _check_replays(st, start, eager_state, eager_y, y, g, "prefill")


def test_stochastic_decode_in_a_graph_draws_the_next_token_per_replay():
    """The token counter of stochastic rounding lives in the state's storage and every call
    advances it on the device, so successive replays of one captured decode step draw the
    uniforms of successive tokens: each replay equals the oracle's step at its own token."""
    B, H, P, fmt = 4, 8, 64, "int4_asym"
    rows = B * H * P
    seed, step0 = 777, 5
    say("graph stochastic decode")
    init = synth.init_state(75, 0, rows, 128)
    st = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P), init)
    ost = oracle.make_state(fmt, rows, 128, init)
    xn, dtn, Bn, Cn, An, Dn = synth.mamba2_step_inputs(75, 0, B, H, 1, P, 128)
    x, dt, Bm, Cm, A, D = (par.dev(a) for a in (xn, dtn, Bn, Cn, An, Dn))
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_set_rounding(st, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    g = _capture(lambda: ssq.ssq_decode_step(st, x, dt, A, Bm, Cm, D, y))  # the warm call runs token step0
    oracle.mamba2_step(ost, xn, dtn, An, Bn, Cn, Dn, sr=(seed, step0))
    assert ssq.ssq_get_rounding(st)[2] == step0 + 1
    prev = None
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        yo = oracle.mamba2_step(ost, xn, dtn, An, Bn, Cn, Dn, sr=(seed, step0 + 1 + rep))
        gs = par.read_gpu_state(st, fmt)
        assert np.array_equal(gs["code"], ost.code), f"replay {rep}: codes differ from the oracle's token"
        assert np.array_equal(gs["scale"].view(np.uint32), ost.scale.view(np.uint32)), rep
        assert np.array_equal(gs["zero"], ost.zero), rep
        assert par.block_rel(y.cpu().numpy(), yo, axis=2) <= 1e-5, rep
        assert ssq.ssq_get_rounding(st)[2] == step0 + 2 + rep
        # the same inputs at a new token: the rounding draws differ from the last replay's
        cur = gs["code"].copy()
        if prev is not None:
            assert not np.array_equal(cur, prev)
        prev = cur


def test_stochastic_scan_in_a_graph_advances_by_T_per_replay():
    B, H, P, T, fmt = 2, 4, 32, 6, "int8_asym"
    rows = B * H * P
    seed, step0 = 4321, 9
    say("graph stochastic scan")
    init = synth.init_state(76, 0, rows, 128)
    st = par.new_gpu_state(ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P), init)
    ost = oracle.make_state(fmt, rows, 128, init)
    arrs = synth.mamba2_scan_inputs(76, 0, B, T, H, 1, P, 128)
    x, dt, Bm, Cm, A, D = (par.dev(a) for a in arrs)
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_set_rounding(st, ssq.SSQ_ROUND_STOCHASTIC, seed, step0)
    g = _capture(lambda: ssq.ssq_scan(st, T, x, dt, A, Bm, Cm, D, y))
    oracle.mamba2_scan(ost, *arrs[:2], arrs[4], arrs[2], arrs[3], arrs[5], sr=(seed, step0))
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        yo = oracle.mamba2_scan(ost, *arrs[:2], arrs[4], arrs[2], arrs[3], arrs[5], sr=(seed, step0 + T * (rep + 1)))
        gs = par.read_gpu_state(st, fmt)
        assert np.array_equal(gs["code"], ost.code), rep
        assert np.array_equal(gs["scale"].view(np.uint32), ost.scale.view(np.uint32)), rep
        assert par.block_rel(y.cpu().numpy(), yo, axis=(1, 3)) <= 1e-5, rep
        assert ssq.ssq_get_rounding(st)[2] == step0 + T * (rep + 2)
