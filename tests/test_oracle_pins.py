"""Pins of the CPU oracle to what the pages and the mathematics fix (CPU only).

Every test here checks the oracle against something other than itself: the
unrolled closed form of the recurrence, the masked-matrix (state space
duality) form, the decay-only special case, the grid's own invariants, brute
force over every code, hand-derived rows, the error recurrence of the
quantized state and the algebra of the delta rule.

Sources: "ssm-state-quantization" README (Setup: decay lambda = exp(dt*A), the
per-row quantizer, both grids, the readout from the quantized state; Findings
1: round to nearest at 8 and 4 bits); "Mamba state quantization for
inference" (the delta-rule state; "Quantization error returns on the next
token": S_t = A_t S_(t-1) + W_t and Delta_t = A_t Delta_(t-1) + R_t); the
SSDi8 summary (Related work: the equivalence of SSMs and linear attention).
"""
import math

import numpy as np
import pytest

import oracle
import synth

U = 2.0 ** -24  # fp32 unit roundoff
F64 = np.float64


def block_rel(got, ref, axis=-1):
    """max |got - ref| / max(|ref|, RMS of ref over the block)."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    rms = np.sqrt(np.mean(ref * ref, axis=axis, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))


# --------------------------------------------------------------------------
# P1: fp32 control = the unrolled closed form of h_t = lambda_t h_(t-1) + dt_t x_t B_t
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,T", [(4, 1), (4, 5), (8, 8)])
def test_fp32_scan_matches_unrolled_closed_form(N, T):
    Bsz, H, G, P = 2, 3, 1, 2
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(11, 0, Bsz, T, H, G, P, N)
    h0 = synth.init_state(11, 0, Bsz * H * P, N)
    st = oracle.make_state("fp32", Bsz * H * P, N, h0)
    y = oracle.mamba2_scan(st, x, dt, A, Bm, Cm, D)

    lam = np.exp(dt.astype(F64) * A.astype(F64))  # [B][T][H]
    h0 = h0.astype(F64).reshape(Bsz, H, P, N)
    yref = np.zeros((Bsz, T, H, P))
    hT = np.zeros((Bsz, H, P, N))
    for b in range(Bsz):
        for hh in range(H):
            for p in range(P):
                for t in range(T):
                    # h_t = (prod_{s<=t} lam_s) h0 + sum_{t'<=t} (prod_{t'<s<=t} lam_s) dt_t' x_t' B_t'
                    ht = np.prod(lam[b, : t + 1, hh]) * h0[b, hh, p]
                    for tp in range(t + 1):
                        ht = ht + (np.prod(lam[b, tp + 1: t + 1, hh]) * F64(dt[b, tp, hh])
                                   * F64(x[b, tp, hh, p]) * Bm[b, tp, 0].astype(F64))
                    yref[b, t, hh, p] = np.dot(Cm[b, t, 0].astype(F64), ht) + F64(D[hh]) * x[b, t, hh, p]
                    if t == T - 1:
                        hT[b, hh, p] = ht
    assert block_rel(st.h.reshape(Bsz, H, P, N), hT) < 2e-6
    assert block_rel(y, yref, axis=(1, 3)) < 2e-6


# --------------------------------------------------------------------------
# P2: fp32 scan = masked-matrix (duality) form y = (L o C B^T)(dt x) + D x
# --------------------------------------------------------------------------
def test_fp32_scan_matches_masked_matrix_form():
    Bsz, T, H, G, P, N = 2, 256, 3, 1, 4, 16
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(5, 2, Bsz, T, H, G, P, N)
    st = oracle.make_state("fp32", Bsz * H * P, N)
    y = oracle.mamba2_scan(st, x, dt, A, Bm, Cm, D)
    yref = np.zeros((Bsz, T, H, P))
    for b in range(Bsz):
        CB = Cm[b, :, 0].astype(F64) @ Bm[b, :, 0].astype(F64).T  # [T][T]: C_t . B_s
        for hh in range(H):
            loglam = dt[b, :, hh].astype(F64) * F64(A[hh])  # log lambda_t
            cs = np.cumsum(loglam)
            L = np.exp(cs[:, None] - cs[None, :])  # prod_{s<r<=t} lambda_r
            L = np.tril(L)
            u = dt[b, :, hh].astype(F64)[:, None] * x[b, :, hh, :].astype(F64)  # [T][P]
            yref[b, :, hh, :] = (L * CB) @ u + F64(D[hh]) * x[b, :, hh, :]
    assert block_rel(y, yref, axis=(1, 3)) < 1e-5


# --------------------------------------------------------------------------
# P3: x = 0 leaves only the decay
# --------------------------------------------------------------------------
def test_fp32_zero_input_is_pure_decay():
    Bsz, T, H, G, P, N = 2, 30, 6, 1, 3, 32
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(3, 0, Bsz, T, H, G, P, N)
    x[:] = 0
    h0 = synth.init_state(3, 0, Bsz * H * P, N)
    st = oracle.make_state("fp32", Bsz * H * P, N, h0)
    y = oracle.mamba2_scan(st, x, dt, A, Bm, Cm, D)
    prod = np.prod(np.exp(dt.astype(F64) * A.astype(F64)), axis=1)  # [B][H]
    ref = h0.astype(F64).reshape(Bsz, H, P, N) * prod[:, :, None, None]
    got = st.h.reshape(Bsz, H, P, N).astype(F64)
    nz = ref != 0
    assert np.all(np.abs(got[nz] / ref[nz] - 1) <= 4 * T * U)


@pytest.mark.parametrize("fmt", ["int8_sym", "int8_asym", "int4_sym", "int4_asym"])
def test_quantized_zero_input_keeps_codes(fmt):
    """With x = 0 the new row is the old grid scaled by lambda: the nearest codes and the zero
    point are unchanged and the scale follows lambda*s (rows whose codes span the whole grid)."""
    bits, asym = oracle.FORMATS[fmt]
    Bsz, T, H, G, P, N = 2, 24, 6, 1, 8, 128
    rows = Bsz * H * P
    st = oracle.make_state(fmt, rows, N, synth.init_state(7, 1, rows, N))
    top = (1 << bits) - 1 if asym else (1 << (bits - 1)) - 1
    full = (st.code.max(axis=1) == top) if asym else np.ones(rows, bool)
    assert full.mean() > 0.9
    code0, z0 = st.code.copy(), st.zero.copy()
    alive = np.ones(rows, bool)
    for t in range(T):
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(7, 1, Bsz, H, G, P, N, t=t)
        x[:] = 0
        s_prev = st.scale.copy()
        oracle.mamba2_step(st, x, dt, A, Bm, Cm, D)
        lam = np.exp(dt.astype(F64) * A.astype(F64))  # [B][H]
        lam_rows = np.repeat(lam.reshape(-1), P)
        alive &= st.scale > 1e-30  # stop following rows that decayed toward underflow
        chk = full & alive
        assert np.array_equal(st.code[chk], code0[chk]), t
        assert np.array_equal(st.zero[chk], z0[chk]), t
        ratio = st.scale[chk].astype(F64) / (lam_rows[chk] * s_prev[chk].astype(F64))
        assert np.all(np.abs(ratio - 1) <= 8 * U), t
    assert alive.mean() > 0.5


# --------------------------------------------------------------------------
# P4 / P5: the grids' invariants and brute force over every code
# --------------------------------------------------------------------------
def _test_rows(n=128):
    rows = [synth.init_state(9, 3, 64, n).astype(F64)]
    rng = synth.normal(9, 99, 0, np.arange(8 * n)).reshape(8, n)
    rows.append(10.0 + 1e-2 * rng)          # offset rows: large negative zero point
    rows.append(-3.0 + 1e-3 * rng)
    rows.append(1e-20 * rng)                # tiny but normal
    rows.append(np.abs(rng) * 1e5)          # all positive, wide
    return np.concatenate(rows).astype(np.float32)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_asymmetric_grid_invariants(bits):
    h = _test_rows()
    code, s, z, v = oracle.quantize_rows(h, None, bits=bits, asym=1, with_v=True)
    qa = (1 << bits) - 1
    assert code.min() >= 0 and code.max() <= qa
    assert np.all(z == np.round(z))
    rows = np.arange(h.shape[0])
    amin, amax = h.argmin(axis=1), h.argmax(axis=1)
    assert np.all(code[rows, amin] == 0)
    top = code[rows, amax]
    vz_top = v[rows, amax].astype(F64) + z.astype(F64)
    # the largest entry takes the top code unless its grid value fell below top - 1/2
    assert np.all((top == qa) | ((top == qa - 1) & (vz_top <= qa - 0.5 + 1e-3)))
    assert (top == qa).mean() > 0.9
    deq = oracle.dequantize_rows(code, s, z).astype(F64)
    err = np.abs(deq - h.astype(F64))
    bound = (s.astype(F64)[:, None] / 2) * (1 + 2.0 ** -18) + 4 * U * np.abs(h).max(axis=1, keepdims=True)
    assert np.all(err <= bound)
    # min and max are reproduced to within half a step
    assert np.all(np.abs(deq[rows, amin] - h[rows, amin]) <= bound[:, 0])
    assert np.all(np.abs(deq[rows, amax] - h[rows, amax]) <= bound[:, 0])


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_symmetric_grid_invariants(bits):
    h = _test_rows()
    code, s, z = oracle.quantize_rows(h, None, bits=bits, asym=0)
    qs = (1 << (bits - 1)) - 1
    assert np.all(z == 0) and code.min() >= -qs and code.max() <= qs
    rows = np.arange(h.shape[0])
    am = np.abs(h).argmax(axis=1)
    assert np.all(np.abs(code[rows, am]) == qs)
    assert np.all(np.sign(code[rows, am]) == np.sign(h[rows, am]))
    deq = oracle.dequantize_rows(code, s, z).astype(F64)
    bound = (s.astype(F64)[:, None] / 2) * (1 + 2.0 ** -18) + 4 * U * np.abs(h).max(axis=1, keepdims=True)
    assert np.all(np.abs(deq - h) <= bound)


@pytest.mark.parametrize("asym", [0, 1])
@pytest.mark.parametrize("bits", [2, 4, 6, 8])
def test_codes_are_nearest_by_brute_force(bits, asym):
    h = _test_rows(n=32)
    code, s, z = oracle.quantize_rows(h, None, bits=bits, asym=asym)
    if asym:
        ks = np.arange(0, 1 << bits, dtype=F64)
    else:
        qs = (1 << (bits - 1)) - 1
        ks = np.arange(-qs, qs + 1, dtype=F64)
    s64, z64, h64 = s.astype(F64), z.astype(F64), h.astype(F64)
    grid = s64[:, None, None] * (ks[None, None, :] - z64[:, None, None])  # [rows][1][K]
    err_all = np.abs(grid - h64[:, :, None])
    best = err_all.min(axis=2)
    chosen = np.abs(s64[:, None] * (code - z64[:, None]) - h64)
    assert np.all(chosen <= best + (2.0 ** -18) * s64[:, None] + 4 * U * np.abs(h64))


def test_hand_derived_rows():
    def q(row, bits, asym):
        c, s, z = oracle.quantize_rows(np.array([row], np.float32), None, bits=bits, asym=asym)
        return c[0].tolist(), float(s[0]), float(z[0])

    # step (max-min)/(2^b-1) = 1, zero point 1: codes are h + 1
    assert q([-1, 0, 1, 2], 2, 1) == ([0, 1, 2, 3], 1.0, 1.0)
    # integer zero point: z = -rne(0.5) = 0, so the grid is {0,1,2,3}; ties go to the even code,
    # the top entry is clamped to 3
    c, s, z = q([0.5, 1.5, 2.5, 3.5], 2, 1)
    assert c == [0, 2, 2, 3] and s == 1.0 and z == 0.0
    # exact binary step 1/8 with a large negative zero point
    c, s, z = q([10.0, 10.0 + 255 / 8, 10.0 + 100.25 / 8, 10.0 + 0.0625], 8, 1)
    assert (s, z) == (0.125, -80.0) and c == [0, 255, 100, 0]
    # symmetric: step amax/127 = 2^-4, ties to even
    c, s, z = q([127 / 16, -63.5 / 16, 0.25 / 16, -127 / 16], 8, 0)
    assert c == [127, -64, 0, -127] and s == 1 / 16 and z == 0.0
    # degenerate rows: a constant row is kept exactly, a zero row stays zero
    assert q([3, 3, 3, 3], 4, 1) == ([0, 0, 0, 0], 3.0, -1.0)
    assert q([-2, -2], 8, 1) == ([0, 0], 2.0, 1.0)
    assert q([0, 0, 0], 8, 1)[0:2] == ([0, 0, 0], 0.0)
    assert q([0, 0, 0], 8, 0) == ([0, 0, 0], 0.0, 0.0)
    deq = oracle.dequantize_rows(np.array([[0, 0]], np.int32), np.array([2.0], np.float32),
                                 np.array([1.0], np.float32))
    assert deq.tolist() == [[-2.0, -2.0]]


@pytest.mark.parametrize("fmt", ["int8_sym", "int8_asym", "int4_sym", "int4_asym"])
def test_requantizing_a_grid_row_is_idempotent(fmt):
    bits, asym = oracle.FORMATS[fmt]
    h = synth.init_state(2, 0, 256, 128)
    code, s, z = oracle.quantize_rows(h, fmt)
    top = (1 << bits) - 1 if asym else (1 << (bits - 1)) - 1
    full = (code.max(axis=1) == top) if asym else np.ones(len(s), bool)
    code2, s2, z2 = oracle.quantize_rows(oracle.dequantize_rows(code, s, z), fmt)
    assert np.array_equal(code2[full], code[full])
    assert np.array_equal(z2[full], z[full])
    assert np.all(np.abs(s2[full].astype(F64) / s[full] - 1) <= 4 * U)


# --------------------------------------------------------------------------
# readout: from the quantized state (default) or before rounding
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym", "int8_sym"])
def test_readout_reads_the_state_it_names(fmt):
    Bsz, H, G, P, N = 2, 3, 1, 4, 128
    rows = Bsz * H * P
    init = synth.init_state(4, 0, rows, N)
    x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(4, 0, Bsz, H, G, P, N)
    st = oracle.make_state(fmt, rows, N, init)
    y_post, hpre, _ = oracle.mamba2_step(st, x, dt, A, Bm, Cm, D, readout="post", diag=True)
    deq = st.dequant().reshape(Bsz, H, P, N).astype(F64)
    C = Cm[:, 0].astype(F64)
    ref_post = np.einsum("bn,bhpn->bhp", C, deq) + (D[None, :, None] * x).astype(F64)
    assert block_rel(y_post, ref_post, axis=2) < 1e-6
    st2 = oracle.make_state(fmt, rows, N, init)
    y_pre = oracle.mamba2_step(st2, x, dt, A, Bm, Cm, D, readout="pre")
    ref_pre = np.einsum("bn,bhpn->bhp", C, hpre.reshape(Bsz, H, P, N).astype(F64)) + \
        (D[None, :, None] * x).astype(F64)
    assert block_rel(y_pre, ref_pre, axis=2) < 1e-6
    # the two readouts share the state update
    assert np.array_equal(st.code, st2.code) and np.array_equal(st.scale, st2.scale)


# --------------------------------------------------------------------------
# P6: Delta_t = A_t Delta_(t-1) + R_t
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym", "int8_sym"])
def test_error_recurrence(fmt):
    Bsz, T, H, G, P, N = 1, 40, 6, 1, 4, 64
    rows = Bsz * H * P
    init = synth.init_state(6, 0, rows, N)
    sq = oracle.make_state(fmt, rows, N, init)
    sf = oracle.make_state("fp32", rows, N, sq.dequant())  # same starting value
    d_prev = (sq.dequant().astype(F64) - sf.h.astype(F64))
    assert np.all(d_prev == 0)
    for t in range(T):
        x, dt, Bm, Cm, A, D = synth.mamba2_step_inputs(6, 0, Bsz, H, G, P, N, t=t)
        hq_prev, hf_prev = sq.dequant().astype(F64), sf.h.astype(F64)
        _, htil, _ = oracle.mamba2_step(sq, x, dt, A, Bm, Cm, D, diag=True)
        oracle.mamba2_step(sf, x, dt, A, Bm, Cm, D)
        lam = np.float32(np.exp(np.float32(dt * A).astype(F64)))  # the fp32 decay [B][H]
        lam_r = np.repeat(lam.reshape(-1), P).astype(F64)[:, None]
        W = (dt[:, :, None].astype(F64) * x.astype(F64)).reshape(rows, 1) * \
            np.repeat(Bm[:, 0].astype(F64), H * P, axis=0)
        hq, hf, ht = sq.dequant().astype(F64), sf.h.astype(F64), htil.astype(F64)
        delta = hq - hf
        R = hq - ht
        lhs = np.abs(delta - lam_r * d_prev - R)
        # Both sides apply the same fp32 update to the state they hold (the quantized side to
        # its reconstructed row), h' = fma(lambda, h, fl(fl(dt*x)*B)): the product lambda*h is
        # exact inside the fma, so each side is off the exact recurrence only by the two
        # roundings of the write term and the one of the result,
        # |h' - lambda*h - W| <= (2u + u^2)|W| + u|h'|.  lhs is the difference of the two.
        bound = U * (1 + 2.0 ** -20) * (4 * (1 + 2.0 ** -20) * np.abs(W) + np.abs(ht) + np.abs(hf)) + 1e-37
        assert np.all(lhs <= bound), t
        d_prev = delta
    # the injected residual is the rounding: at most half a step per entry
    assert np.all(np.abs(R) <= sq.scale.astype(F64)[:, None] * 0.5 * (1 + 2.0 ** -18) + 4 * U * np.abs(ht))


# --------------------------------------------------------------------------
# P7: the delta rule
# --------------------------------------------------------------------------
def delta_rounding_bound(Sh, k, v, beta, alpha=None, a_vec=None, v_err=None):
    """Entrywise bound on |S' - S*| for one fp32 delta-rule step of one matrix.

    S* = A S + beta k v^T is the exact step from the fp32 matrix Sh [dk][dv] (the state the
    step starts from: the reconstructed rows of a quantized state), with A = alpha (I - beta k k^T)
    (one decay) or (I - beta k k^T) Diag(a_vec) (a decay per key row).  S' is what an fp32
    evaluation returns when u = k^T S (or k^T Diag(a) S) is summed in double and rounded once,
    w = beta (v - alpha u) (or beta (v - u)) is taken one rounding per operation, and each entry
    is fma(a_i, S_ij, fl(k_i w_j)): the product a_i S_ij sits inside the fma, so apart from the
    propagated error of w only the roundings of k_i w_j and of the result remain.  v_err bounds
    an error already in v (a rotated v rounded once).  First order in u, with slack."""
    u32 = U * (1 + 2.0 ** -18)
    Sh = np.asarray(Sh, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    a = np.full(k.shape, F64(alpha)) if a_vec is None else np.asarray(a_vec, F64)
    kap = k * (a if a_vec is not None else 1.0)
    ustar = kap @ Sh
    e_u = u32 * np.abs(ustar) + 2.0 ** -45 * (np.abs(kap) @ np.abs(Sh))
    if a_vec is None:
        vm = v - F64(alpha) * ustar
        e_vm = F64(alpha) * e_u + u32 * np.abs(F64(alpha) * ustar) + u32 * np.abs(vm)
    else:
        vm = v - ustar
        e_vm = e_u + u32 * np.abs(vm)
    if v_err is not None:
        e_vm = e_vm + v_err
    w = F64(beta) * vm
    e_w = F64(beta) * e_vm + u32 * np.abs(w)
    Sstar = a[:, None] * Sh + np.outer(k, w)
    bound = np.abs(k)[:, None] * e_w[None, :] + u32 * np.abs(np.outer(k, w)) + u32 * np.abs(Sstar)
    return Sstar, bound * (1 + 2.0 ** -16) + 1e-37


@pytest.mark.parametrize("dk,dv", [(4, 4), (8, 8), (8, 4)])
def test_delta_fp32_matches_dense_form(dk, dv):
    Bsz, H, T = 2, 2, 3
    S0 = synth.init_state(8, 0, Bsz * H * dk, dv)
    st = oracle.make_state("fp32", Bsz * H * dk, dv, S0)
    S = S0.astype(F64).reshape(Bsz, H, dk, dv)
    for t in range(T):
        q, k, v, al, be = synth.delta_inputs(8, 0, Bsz, H, dk, dv, t=t)
        o = oracle.delta_step(st, q, k, v, al, be, Bsz, H)
        for b in range(Bsz):
            for hh in range(H):
                kk = k[b, hh].astype(F64)
                Aop = F64(al[b, hh]) * (np.eye(dk) - F64(be[b, hh]) * np.outer(kk, kk))
                S[b, hh] = Aop @ S[b, hh] + F64(be[b, hh]) * np.outer(kk, v[b, hh].astype(F64))
                oref = S[b, hh].T @ q[b, hh].astype(F64)
                assert block_rel(o[b, hh], oref) < 1e-5
        assert block_rel(st.h.reshape(Bsz, H, dk, dv), S, axis=(2, 3)) < 1e-5


def test_delta_writes_v_at_unit_key():
    """alpha = beta = 1 and |k| = 1: the step overwrites the value stored at key k with v."""
    Bsz, H, dk, dv = 2, 3, 16, 8
    st = oracle.make_state("fp32", Bsz * H * dk, dv, synth.init_state(1, 0, Bsz * H * dk, dv))
    q, k, v, al, be = synth.delta_inputs(1, 0, Bsz, H, dk, dv)
    al[:] = 1
    be[:] = 1
    oracle.delta_step(st, k, k, v, al, be, Bsz, H)  # read with q = k
    S = st.h.reshape(Bsz, H, dk, dv).astype(F64)
    readback = np.einsum("bhij,bhi->bhj", S, k.astype(F64))
    assert block_rel(readback, v.astype(F64)) < 1e-5


@pytest.mark.parametrize("fmt", ["int8_asym", "int8_sym", "int4_asym"])
def test_delta_zero_beta_is_pure_decay(fmt):
    bits, asym = oracle.FORMATS[fmt]
    Bsz, H, dk, dv = 2, 2, 32, 128
    rows = Bsz * H * dk
    st = oracle.make_state(fmt, rows, dv, synth.init_state(12, 0, rows, dv))
    top = (1 << bits) - 1 if asym else (1 << (bits - 1)) - 1
    full = (st.code.max(axis=1) == top) if asym else np.ones(rows, bool)
    code0, z0, s0 = st.code.copy(), st.zero.copy(), st.scale.copy()
    q, k, v, al, be = synth.delta_inputs(12, 0, Bsz, H, dk, dv)
    be[:] = 0
    oracle.delta_step(st, q, k, v, al, be, Bsz, H)
    assert np.array_equal(st.code[full], code0[full]) and np.array_equal(st.zero[full], z0[full])
    al_r = np.repeat(al.reshape(-1), dk).astype(F64)
    assert np.all(np.abs(st.scale[full] / (al_r[full] * s0[full]) - 1) <= 8 * U)


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym"])
def test_delta_quantized_state_within_half_step(fmt):
    Bsz, H, dk, dv = 2, 2, 16, 128
    rows = Bsz * H * dk
    st = oracle.make_state(fmt, rows, dv, synth.init_state(13, 0, rows, dv))
    S_start = st.dequant().astype(F64).reshape(Bsz, H, dk, dv)
    q, k, v, al, be = synth.delta_inputs(13, 0, Bsz, H, dk, dv)
    o, Spre, _ = oracle.delta_step(st, q, k, v, al, be, Bsz, H, diag=True)
    # the pre-rounding matrix is the dense delta rule applied to the dequantized start, up to
    # the rounding of one fp32 step
    Spre4 = Spre.reshape(Bsz, H, dk, dv).astype(F64)
    for b in range(Bsz):
        for hh in range(H):
            kk = k[b, hh].astype(F64)
            ref = F64(al[b, hh]) * (np.eye(dk) - F64(be[b, hh]) * np.outer(kk, kk)) @ S_start[b, hh] \
                + F64(be[b, hh]) * np.outer(kk, v[b, hh].astype(F64))
            Sstar, bound = delta_rounding_bound(S_start[b, hh], k[b, hh], v[b, hh], be[b, hh], alpha=al[b, hh])
            assert np.allclose(Sstar, ref, rtol=1e-12, atol=1e-12)
            assert np.all(np.abs(Spre4[b, hh] - ref) <= bound)
    deq = st.dequant().astype(F64)
    err = np.abs(deq - Spre.astype(F64))
    assert np.all(err <= st.scale.astype(F64)[:, None] * 0.5 * (1 + 2.0 ** -18) + 4 * U * np.abs(Spre))
    # readout from the quantized matrix
    oref = np.einsum("bhij,bhi->bhj", deq.reshape(Bsz, H, dk, dv), q.astype(F64))
    assert block_rel(o, oref) < 1e-6


@pytest.mark.parametrize("fmt", ["int8_asym", "int4_asym", "int8_sym"])
def test_delta_error_recurrence(fmt):
    """Delta_t = A_t Delta_(t-1) + R_t for the delta rule, A_t = alpha (I - beta k k^T): the
    quantized and the fp32 state, started from the same values and fed the same inputs,
    differ after each step by the decayed difference plus the injected rounding residual,
    within the rounding of one fp32 step on each side."""
    Bsz, H, dk, dv, T = 1, 3, 32, 128, 12
    rows = Bsz * H * dk
    sq = oracle.make_state(fmt, rows, dv, synth.init_state(14, 0, rows, dv))
    sf = oracle.make_state("fp32", rows, dv, sq.dequant())
    d_prev = np.zeros((Bsz * H, dk, dv))
    for t in range(T):
        q, k, v, al, be = synth.delta_inputs(14, 0, Bsz, H, dk, dv, t=t)
        hq_prev = sq.dequant().astype(F64).reshape(Bsz * H, dk, dv)
        hf_prev = sf.h.astype(F64).reshape(Bsz * H, dk, dv)
        _, ht, _ = oracle.delta_step(sq, q, k, v, al, be, Bsz, H, diag=True)
        oracle.delta_step(sf, q, k, v, al, be, Bsz, H)
        hq = sq.dequant().astype(F64).reshape(Bsz * H, dk, dv)
        hf = sf.h.astype(F64).reshape(Bsz * H, dk, dv)
        ht = ht.astype(F64).reshape(Bsz * H, dk, dv)
        for m in range(Bsz * H):
            b, hh = divmod(m, H)
            kk = k[b, hh].astype(F64)
            Aop = F64(al[b, hh]) * (np.eye(dk) - F64(be[b, hh]) * np.outer(kk, kk))
            delta, R = hq[m] - hf[m], hq[m] - ht[m]
            lhs = np.abs(delta - Aop @ d_prev[m] - R)
            _, bq = delta_rounding_bound(hq_prev[m], k[b, hh], v[b, hh], be[b, hh], alpha=al[b, hh])
            _, bf = delta_rounding_bound(hf_prev[m], k[b, hh], v[b, hh], be[b, hh], alpha=al[b, hh])
            # the two exact steps differ by exactly A (hq_prev - hf_prev); A is applied in double
            slack = 2.0 ** -40 * (np.abs(Aop) @ np.abs(d_prev[m]))
            assert np.all(lhs <= bq + bf + slack), (t, m)
            d_prev[m] = delta
    # the injected residual is the rounding: at most half a step per entry
    assert np.all(np.abs(R) <= sq.scale.astype(F64)[-dk:, None] * 0.5 * (1 + 2.0 ** -18) + 4 * U * np.abs(ht[-1]))


# --------------------------------------------------------------------------
# decay: lambda is exp(dt*A) rounded once
# --------------------------------------------------------------------------
def test_decay_is_correctly_rounded_exp():
    dt = synth.uniform(1, 50, 0, np.arange(2000)).astype(np.float32) * 3
    A = -(1 + 15 * synth.uniform(1, 51, 0, np.arange(2000))).astype(np.float32)
    for a, b in zip(dt[:400], A[:400]):
        lam = oracle.decay(float(a), float(b))
        e = F64(np.float32(a) * np.float32(b))  # the fp32 product, then exact exp
        ref = math.exp(e)
        # the nearest float: no other float is closer to exp(e)
        lf = np.float32(lam)
        assert abs(F64(lf) - ref) <= abs(F64(np.nextafter(lf, np.float32(np.inf))) - ref)
        assert abs(F64(lf) - ref) <= abs(F64(np.nextafter(lf, np.float32(0))) - ref)


# --------------------------------------------------------------------------
# oracle entry points agree on indexing (rows scan vs full scan)
# --------------------------------------------------------------------------
def test_rows_scan_indexes_like_full_scan():
    Bsz, T, H, G, P, N = 2, 6, 4, 2, 3, 16
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(21, 4, Bsz, T, H, G, P, N)
    nrows = Bsz * H * P
    init = synth.init_state(21, 4, nrows, N)
    st = oracle.make_state("int8_asym", nrows, N, init)
    y = oracle.mamba2_scan(st, x, dt, A, Bm, Cm, D)
    rows = np.array([0, 5, 11, 17, 23])
    xr, dtr, Br, Cr, Ar, Dr = synth.mamba2_rows_scan_inputs(21, 4, Bsz, T, H, G, P, N, rows)
    sr = oracle.make_state("int8_asym", len(rows), N, init[rows])
    yr = oracle.mamba2_rows_scan(sr, xr, dtr, Ar, Br, Cr, Dr)
    b, hh, p = rows // (H * P), (rows // P) % H, rows % P
    assert np.array_equal(yr, y[b, :, hh, p])
    assert np.array_equal(sr.code, st.code[rows]) and np.array_equal(sr.scale, st.scale[rows])
