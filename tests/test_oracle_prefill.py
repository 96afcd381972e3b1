"""Pins of the oracle's chunked prefill (CPU only).

"Mamba state quantization for inference" (section "Mamba state quantization needs
phase-aware benchmarks") describes DAMP's prefill: the recurrence runs in FP32 inside
each chunk and the chunk-final state is written into the packed cache, which decode
then reads and rewrites.  Reading taken: the stored state is dequantized once; every
token applies the fp32 update; at each chunk end (and after the last token) the row is
refit and rounded, y follows the readout flag, and the next chunk starts from the
dequantized codes.

Pins: with an fp32 state the prefill is the fp32 scan; one chunk over the whole prompt
is the fp32 scan from the dequantized start followed by one quantization; a prompt
cut into chunks equals the chunks run one after another; chunk-end stochastic
rounding draws the uniforms of its token.
"""
import numpy as np
import pytest

import oracle
import synth

QUANT = ["int8_sym", "int8_asym", "int4_sym", "int4_asym"]


def _inputs(seed, T, B=2, H=3, G=1, P=4, N=128):
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(seed, 0, B, T, H, G, P, N)
    init = synth.init_state(seed, 0, B * H * P, N)
    return (x, dt, Bm, Cm, A, D), init


def test_fp32_prefill_is_the_fp32_scan():
    (x, dt, Bm, Cm, A, D), init = _inputs(41, 12)
    s1 = oracle.make_state("fp32", init.shape[0], 128, init)
    s2 = oracle.make_state("fp32", init.shape[0], 128, init)
    y1 = oracle.mamba2_prefill(s1, x, dt, A, Bm, Cm, D, chunk=5)
    y2 = oracle.mamba2_scan(s2, x, dt, A, Bm, Cm, D)
    assert np.array_equal(y1, y2) and np.array_equal(s1.h, s2.h)


@pytest.mark.parametrize("readout", ["post", "pre"])
@pytest.mark.parametrize("fmt", QUANT)
def test_one_chunk_is_an_fp32_scan_then_one_quantization(fmt, readout):
    T = 10
    (x, dt, Bm, Cm, A, D), init = _inputs(42, T, H=4, G=2)  # two heads per B/C group
    rows = init.shape[0]
    st = oracle.make_state(fmt, rows, 128, init)
    f32 = oracle.make_state("fp32", rows, 128, st.dequant())
    y = oracle.mamba2_prefill(st, x, dt, A, Bm, Cm, D, chunk=T, readout=readout)
    yf = oracle.mamba2_scan(f32, x, dt, A, Bm, Cm, D)
    code, s, z = oracle.quantize_rows(f32.h, fmt)
    assert np.array_equal(st.code, code) and np.array_equal(st.scale, s) and np.array_equal(st.zero, z)
    assert np.array_equal(y[:, :T - 1], yf[:, :T - 1])       # inside the chunk: the fp32 readout
    if readout == "pre":
        assert np.array_equal(y[:, T - 1], yf[:, T - 1])
    else:                                                   # the last token reads the new codes
        B, _, H, P = x.shape
        r = oracle.dequantize_rows(code, s, z).astype(np.float64).reshape(B, H, P, 128)
        Cg = np.repeat(Cm[:, T - 1].astype(np.float64), H // Cm.shape[2], axis=1)  # [B][H][N]
        ref = np.einsum("bhpn,bhn->bhp", r, Cg) \
            + (D.astype(np.float64)[None, :, None] * x[:, T - 1].astype(np.float64))
        assert np.max(np.abs(y[:, T - 1] - ref) / np.maximum(np.abs(ref), 1e-3)) < 1e-5


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_sym"])
def test_chunks_compose(fmt):
    T, c = 12, 4
    (x, dt, Bm, Cm, A, D), init = _inputs(43, T)
    rows = init.shape[0]
    whole = oracle.make_state(fmt, rows, 128, init)
    y = oracle.mamba2_prefill(whole, x, dt, A, Bm, Cm, D, chunk=c)
    part = oracle.make_state(fmt, rows, 128, init)
    ys = []
    for k in range(0, T, c):
        sl = slice(k, k + c)
        ys.append(oracle.mamba2_prefill(part, x[:, sl], dt[:, sl], A, Bm[:, sl], Cm[:, sl], D, chunk=c))
    assert np.array_equal(y, np.concatenate(ys, axis=1))
    assert np.array_equal(whole.code, part.code) and np.array_equal(whole.scale, part.scale)
    # a chunk longer than the prompt quantizes once, after the last token
    a = oracle.make_state(fmt, rows, 128, init)
    b = oracle.make_state(fmt, rows, 128, init)
    assert np.array_equal(oracle.mamba2_prefill(a, x, dt, A, Bm, Cm, D, chunk=T),
                          oracle.mamba2_prefill(b, x, dt, A, Bm, Cm, D, chunk=10 * T))
    assert np.array_equal(a.code, b.code)


def test_chunk_end_stochastic_rounding_uses_its_token():
    T, c, seed, step0 = 6, 3, 17, 100
    (x, dt, Bm, Cm, A, D), init = _inputs(44, T)
    rows = init.shape[0]
    st = oracle.make_state("int8_asym", rows, 128, init)
    oracle.mamba2_prefill(st, x, dt, A, Bm, Cm, D, chunk=c, sr=(seed, step0))
    # the same prompt as two chunks, each ending with the uniforms of token step0 + 2 and step0 + 5
    ref = oracle.make_state("int8_asym", rows, 128, init)
    f32 = oracle.make_state("fp32", rows, 128, ref.dequant())
    for k in range(0, T, c):
        sl = slice(k, k + c)
        oracle.mamba2_scan(f32, x[:, sl], dt[:, sl], A, Bm[:, sl], Cm[:, sl], D)
        for r in range(rows):
            cc, ss, zz = oracle.quantize_row_sr(f32.h[r], "int8_asym",
                                               oracle.sr_row_uniforms(seed, step0 + k + c - 1, rows, r, 128))
            ref.code[r], ref.scale[r], ref.zero[r] = cc, ss, zz
        f32.h[:] = ref.dequant()
    assert np.array_equal(st.code, ref.code) and np.array_equal(st.scale, ref.scale)
