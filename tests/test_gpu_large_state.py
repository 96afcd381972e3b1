"""States larger than 4 GiB: the rows past byte 2^32 of the codes.

* Mamba-2 int8 symmetric, 4,100 sequences x 128 heads x 64 rows (33.6 M rows, 4.30 GB of
  codes): two decode steps from a zero state, so that the second step reads the codes the
  first one stored.
* Delta rule int8 asymmetric, 8,200 sequences x 32 heads of 128 x 128 (4.30 GB of codes): two
  steps from a zero state.
* Mamba-2 int8 asymmetric scan of 2 tokens on the same Mamba-2 shape.

The rows of the last two sequences (every one of them past byte 2^32) and of the first two
are compared with the oracle under the contract: rows and matrices are independent, so the
oracle steps just those sequences with their own inputs.  Outputs read from a state that
started at zero can cancel within a head, so they are also held element by element to the
error bound of an fp32 sum of their 128 terms.  Only the compared rows are read
back from the GPU.
"""
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

K = oracle.workers()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def read_rows(gst, fmt, sl):
    """Codes, scales and zero points of the rows in slice ``sl`` only."""
    torch.cuda.synchronize()
    codes, scale, zero = gst.regions()
    out = {"code": par.unpack_codes(codes[sl].cpu().numpy(), fmt), "scale": scale[sl].cpu().numpy()}
    out["zero"] = zero[sl].cpu().numpy() if zero is not None else np.zeros_like(out["scale"])
    return out


def write_rows(gst, ost, sl):
    """Teacher forcing on the rows in slice ``sl`` only."""
    codes, scale, zero = gst.regions()
    codes[sl].copy_(torch.from_numpy(par.pack_codes(ost.code, ost.fmt)))
    scale[sl].copy_(torch.from_numpy(ost.scale))
    if zero is not None:
        zero[sl].copy_(torch.from_numpy(ost.zero))
    torch.cuda.synchronize()


def _parts(nseq, rows_per_seq):
    """(sequence slice, row slice) of the first two and the last two sequences."""
    return [(slice(0, 2), slice(0, 2 * rows_per_seq)),
            (slice(nseq - 2, nseq), slice((nseq - 2) * rows_per_seq, nseq * rows_per_seq))]


def test_mamba2_decode_state_beyond_4_gib():
    fmt, B, H, P = "int8_sym", 4100, 128, 64
    desc = ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, 1)
    L = ssq.ssq_state_layout(desc)
    assert L.row_bytes * B * H * P > (1 << 32)
    say(f"Mamba-2 {fmt} state of {B * H * P} rows, {ssq.ssq_state_bytes(desc) / 1e9:.2f} GB")
    gst = par.new_gpu_state(desc)
    parts = _parts(B, H * P)
    osts = [oracle.make_state(fmt, 2 * H * P, 128) for _ in parts]
    for t in range(2):
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(11, 0, B, H, 1, P, 128, t=t)
        y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
        ssq.ssq_decode_step(gst, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
        torch.cuda.synchronize()
        for (bs, rs), ost in zip(parts, osts):
            yo, _, vq = oracle.mamba2_step(ost, x[bs], dt[bs], A, Bm[bs], Cm[bs], D, diag=True)
            g = read_rows(gst, fmt, rs)
            flips = par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, f"step {t} rows {rs}")
            err = par.block_rel(y[bs].cpu().numpy(), yo, axis=2)
            say(f"  step {t}, rows {rs.start}..{rs.stop - 1}: {flips} boundary flips, y error {err:.2e}")
            assert err <= 1e-3
            if flips:
                write_rows(gst, ost, rs)
        del x, y
    gst.free()
    del gst
    torch.cuda.empty_cache()


def test_delta_state_beyond_4_gib():
    fmt, B, H = "int8_asym", 8200, 32
    desc = ssq.make_desc(ssq.SSQ_DELTA, fmt, B, H, 128, 128)
    L = ssq.ssq_state_layout(desc)
    assert L.row_bytes * B * H * 128 > (1 << 32)
    say(f"delta {fmt} state of {B * H} matrices, {ssq.ssq_state_bytes(desc) / 1e9:.2f} GB")
    gst = par.new_gpu_state(desc)
    parts = _parts(B, H * 128)
    osts = [oracle.make_state(fmt, 2 * H * 128, 128) for _ in parts]
    for t in range(2):
        q, k, v, al, be = synth.delta_inputs(12, 0, B, H, 128, 128, t=t)
        o = torch.empty(v.shape, dtype=torch.float32, device="cuda")
        ssq.ssq_delta_step(gst, par.dev(q), par.dev(k), par.dev(v), par.dev(al), par.dev(be), o)
        torch.cuda.synchronize()
        for (bs, rs), ost in zip(parts, osts):
            oo, _, vq = oracle.delta_step(ost, q[bs], k[bs], v[bs], al[bs], be[bs], 2, H, diag=True)
            g = read_rows(gst, fmt, rs)
            flips = par.check_codes(g, ost.code, ost.scale, ost.zero, vq, fmt, f"step {t} rows {rs}")
            og = o[bs].cpu().numpy()
            err = par.block_rel(og, oo, axis=2)
            # o_j = sum_i q_i r_ij over the new stored matrix: a rank-one or rank-two matrix (a zero
            # start) makes a head's sum cancel when q.k is small, so besides the contract's 1e-3 for
            # quantized outputs every element is held to the error bound of an fp32 sum of its 128
            # terms
            deq = ost.dequant().reshape(2, H, 128, 128)
            rcols = deq.transpose(0, 1, 3, 2).reshape(-1, 128)
            qrows = np.repeat(q[bs].reshape(2 * H, 1, 128), 128, axis=1).reshape(-1, 128)
            ratio = par.y_within_sum_bound(og, oo, qrows, rcols, np.zeros(og.size, np.float32))
            say(f"  step {t}, rows {rs.start}..{rs.stop - 1}: {flips} boundary flips, o error {err:.2e}, "
                f"largest error / fp32-sum bound {ratio:.3f}")
            assert err <= 1e-3 and ratio <= 1.0
            if flips:
                write_rows(gst, ost, rs)
        del q, k, v, o
    gst.free()
    del gst
    torch.cuda.empty_cache()


def test_mamba2_scan_state_beyond_4_gib():
    fmt, B, H, P, T = "int8_asym", 4100, 128, 64, 2
    desc = ssq.make_desc(ssq.SSQ_MAMBA2, fmt, B, H, P, 128, 1)
    assert ssq.ssq_state_layout(desc).row_bytes * B * H * P > (1 << 32)
    say(f"Mamba-2 {fmt} scan of {T} tokens on {B * H * P} rows")
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(13, 0, B, T, H, 1, P, 128, threads=K)
    gst = par.new_gpu_state(desc)
    y = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    ssq.ssq_scan(gst, T, par.dev(x), par.dev(dt), par.dev(A), par.dev(Bm), par.dev(Cm), par.dev(D), y)
    torch.cuda.synchronize()
    for bs, rs in _parts(B, H * P):
        ost = oracle.make_state(fmt, 2 * H * P, 128)
        yo = oracle.mamba2_scan(ost, x[bs], dt[bs], A, Bm[bs], Cm[bs], D)
        g = read_rows(gst, fmt, rs)
        diff = int((g["code"] != ost.code).sum())
        deq = oracle.dequantize_rows(g["code"], g["scale"], g["zero"])
        es = par.block_rel(deq, ost.dequant(), axis=1)
        ey = par.block_rel(y[bs].cpu().numpy(), yo, axis=(1, 3))
        say(f"  rows {rs.start}..{rs.stop - 1}: {diff} codes differ, y error {ey:.2e}, state {es:.2e}")
        assert ey <= 1e-3 and es <= 1e-3
        assert diff <= 1e-4 * g["code"].size
    gst.free()
    del gst, y
    torch.cuda.empty_cache()
