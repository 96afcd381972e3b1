"""CPU oracle for the quantized recurrent-state update (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  The product path (``mamba_decode_amd``) never
does, and this package never imports the product path.

The arithmetic lives in ``ssq_oracle.c`` (plain single-threaded C, built with
``-O2 -ffp-contract=off``); this module builds it with gcc when needed and
marshals numpy arrays into it.  States are kept unpacked: one int32 code per
entry plus one fp32 scale and zero point per row, or a plain fp32 state for the
unquantized control.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]

# format name -> (bits, asymmetric); bits == 0 is the fp32 control
FORMATS = {
    "fp32": (0, 0),
    "int8_sym": (8, 0),
    "int8_asym": (8, 1),
    "int4_sym": (4, 0),
    "int4_asym": (4, 1),
}


def build(force: bool = False) -> str:
    """Compile ``ssq_oracle.c`` into ``liboracle.so`` next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def bind(path: str):
    """Load an oracle shared library from ``path`` and declare its C signatures."""
    L = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    i32p = ctypes.POINTER(ctypes.c_int32)
    ci, cl = ctypes.c_int, ctypes.c_int64
    L.orc_decay.argtypes = [ctypes.c_float, ctypes.c_float]
    L.orc_decay.restype = ctypes.c_float
    L.orc_quantize_row.argtypes = [f32p, ci, ci, ci, i32p, f32p, f32p, f32p]
    L.orc_quantize_row.restype = None
    L.orc_quantize_rows.argtypes = [cl, ci, ci, ci, f32p, i32p, f32p, f32p, f32p]
    L.orc_quantize_rows.restype = None
    L.orc_dequantize_rows.argtypes = [cl, ci, i32p, f32p, f32p, f32p]
    L.orc_dequantize_rows.restype = None
    L.orc_mamba2_step.argtypes = [ci, ci, ci, ci, ci, ci, ci, i32p, f32p, f32p, f32p,
                                  f32p, f32p, f32p, f32p, f32p, f32p, f32p, ci, f32p, f32p]
    L.orc_mamba2_step.restype = ci
    L.orc_mamba2_scan.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, i32p, f32p, f32p, f32p,
                                  f32p, f32p, f32p, f32p, f32p, f32p, f32p, ci]
    L.orc_mamba2_scan.restype = ci
    L.orc_mamba2_rows_scan.argtypes = [cl, ci, ci, ci, ci, i32p, f32p, f32p, f32p, f32p,
                                       f32p, f32p, f32p, f32p, f32p, f32p, ci]
    L.orc_mamba2_rows_scan.restype = ci
    L.orc_delta_step.argtypes = [ci, ci, ci, ci, ci, ci, i32p, f32p, f32p, f32p, f32p, f32p,
                                 f32p, f32p, f32p, f32p, ci, f32p, f32p]
    L.orc_delta_step.restype = ci
    u64 = ctypes.c_uint64
    i64p = ctypes.POINTER(ctypes.c_int64)
    L.orc_splitmix64.argtypes = [u64, u64]
    L.orc_splitmix64.restype = u64
    L.orc_sr_uniform.argtypes = [u64, u64, cl, cl, ci, ci]
    L.orc_sr_uniform.restype = ctypes.c_float
    L.orc_sr_row_uniforms.argtypes = [u64, u64, cl, cl, ci, f32p]
    L.orc_sr_row_uniforms.restype = None
    L.orc_quantize_row_sr.argtypes = [f32p, ci, ci, ci, i32p, f32p, f32p, f32p, f32p]
    L.orc_quantize_row_sr.restype = None
    L.orc_mamba2_step_sr.argtypes = L.orc_mamba2_step.argtypes + [ci, u64, u64]
    L.orc_mamba2_step_sr.restype = ci
    L.orc_mamba2_step_sr_part.argtypes = L.orc_mamba2_step_sr.argtypes + [cl, cl]
    L.orc_mamba2_step_sr_part.restype = ci
    L.orc_mamba2_scan_sr.argtypes = L.orc_mamba2_scan.argtypes + [ci, u64, u64]
    L.orc_mamba2_scan_sr.restype = ci
    L.orc_mamba2_rows_scan_sr.argtypes = L.orc_mamba2_rows_scan.argtypes + [ci, u64, u64, cl, i64p]
    L.orc_mamba2_rows_scan_sr.restype = ci
    L.orc_delta_step_sr.argtypes = L.orc_delta_step.argtypes + [ci, u64, u64]
    L.orc_delta_step_sr.restype = ci
    L.orc_kda_step_sr.argtypes = L.orc_delta_step_sr.argtypes
    L.orc_kda_step_sr.restype = ci
    L.orc_mamba2_prefill_sr.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ci, i32p, f32p, f32p, f32p,
                                        f32p, f32p, f32p, f32p, f32p, f32p, f32p, ci, ci, u64, u64]
    L.orc_mamba2_prefill_sr.restype = ci
    L.orc_round_half.argtypes = [ctypes.c_float]
    L.orc_round_half.restype = ctypes.c_float
    L.orc_damp_step_sr.argtypes = [ci, ci, ci, ci, ci, f32p, i32p, f32p, f32p, f32p, f32p, f32p, f32p,
                                   f32p, f32p, ci, f32p, ci, u64, u64]
    L.orc_damp_step_sr.restype = ci
    L.orc_damp_from_fp32.argtypes = [ci, ci, ci, ci, ci, f32p, f32p, i32p, f32p, f32p]
    L.orc_damp_from_fp32.restype = ci
    return L


def lib():
    """The oracle library: the build next to the source, or the build of the same source
    named by the environment variable SSQ_ORACLE_LIB (the tests' sanitized build)."""
    global _lib
    if _lib is None:
        _lib = bind(os.environ.get("SSQ_ORACLE_LIB") or build())
    return _lib


def _f(a):
    if a is None:
        return None
    assert a.dtype == np.float32 and a.flags.c_contiguous, (a.dtype, a.flags)
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _i(a):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _c32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


@dataclass
class State:
    """One layer's state for every row: ``code`` [rows][n] int32, ``scale``/``zero`` [rows]
    (quantized), or ``h`` [rows][n] fp32 (``fmt == 'fp32'``)."""
    fmt: str
    rows: int
    n: int
    code: np.ndarray | None = None
    scale: np.ndarray | None = None
    zero: np.ndarray | None = None
    h: np.ndarray | None = None
    shape: tuple = field(default=())

    @property
    def bits(self):
        return FORMATS[self.fmt][0]

    @property
    def asym(self):
        return FORMATS[self.fmt][1]

    def copy(self) -> "State":
        c = lambda a: None if a is None else a.copy()  # noqa: E731
        return State(self.fmt, self.rows, self.n, c(self.code), c(self.scale), c(self.zero),
                     c(self.h), self.shape)

    def dequant(self) -> np.ndarray:
        """The fp32 value the state stands for, [rows][n]."""
        if self.fmt == "fp32":
            return self.h.copy()
        out = np.empty((self.rows, self.n), np.float32)
        lib().orc_dequantize_rows(self.rows, self.n, _i(self.code), _f(self.scale),
                                  _f(self.zero), _f(out))
        return out


def quantize_rows(h: np.ndarray, fmt: str, bits: int | None = None, asym: int | None = None,
                  with_v: bool = False):
    """Refit and round every row of ``h`` [rows][n]; returns (code, scale, zero[, v])."""
    h = _c32(h)
    rows, n = h.shape
    if bits is None:
        bits, asym = FORMATS[fmt]
    code = np.empty((rows, n), np.int32)
    s = np.empty(rows, np.float32)
    z = np.empty(rows, np.float32)
    v = np.empty((rows, n), np.float32) if with_v else None
    lib().orc_quantize_rows(rows, n, bits, asym, _f(h), _i(code), _f(s), _f(z), _f(v))
    return (code, s, z, v) if with_v else (code, s, z)


def dequantize_rows(code, s, z) -> np.ndarray:
    code = np.ascontiguousarray(code, np.int32)
    rows, n = code.shape
    out = np.empty((rows, n), np.float32)
    lib().orc_dequantize_rows(rows, n, _i(code), _f(_c32(s)), _f(_c32(z)), _f(out))
    return out


def make_state(fmt: str, rows: int, n: int, init: np.ndarray | None = None) -> State:
    """A state of ``rows`` rows of ``n`` entries: zero, or ``init`` [rows][n] quantized."""
    if fmt == "fp32":
        h = np.zeros((rows, n), np.float32) if init is None else _c32(init).reshape(rows, n).copy()
        return State(fmt, rows, n, h=h)
    if init is None:
        return State(fmt, rows, n, code=np.zeros((rows, n), np.int32),
                     scale=np.zeros(rows, np.float32), zero=np.zeros(rows, np.float32))
    code, s, z = quantize_rows(_c32(init).reshape(rows, n), fmt)
    return State(fmt, rows, n, code=code, scale=s, zero=z)


def decay(dt: float, A: float) -> float:
    return lib().orc_decay(ctypes.c_float(dt), ctypes.c_float(A))


def splitmix64(seed: int, i: int) -> int:
    """Output number ``i`` (>= 1) of SplitMix64 started at ``seed``."""
    return int(lib().orc_splitmix64(seed, i))


def sr_uniform(seed: int, step: int, rows: int, r: int, n_len: int, n: int) -> float:
    """The uniform entry ``n`` of state row ``r`` draws at token ``step``."""
    return float(lib().orc_sr_uniform(seed, step, rows, r, n_len, n))


def sr_row_uniforms(seed: int, step: int, rows: int, r: int, n_len: int) -> np.ndarray:
    """The ``n_len`` uniforms of state row ``r`` at token ``step``."""
    U = np.empty(n_len, np.float32)
    lib().orc_sr_row_uniforms(seed, step, rows, r, n_len, _f(U))
    return U


def quantize_row_sr(h: np.ndarray, fmt: str, U: np.ndarray | None):
    """One row refit and rounded; stochastically with uniforms ``U`` (same length, each a
    multiple of 2^-16 in [0, 1)), or to nearest when ``U`` is None.  Returns (code, scale,
    zero)."""
    h = _c32(h)
    if U is not None:
        K = _c32(U).astype(np.float64) * 65536.0
        if not (np.all(K == np.floor(K)) and np.all(K >= 0) and np.all(K < 65536)):
            raise ValueError("stochastic rounding takes uniforms that are multiples of 2^-16 in [0, 1)")
    n = h.shape[0]
    bits, asym = FORMATS[fmt]
    code = np.empty(n, np.int32)
    s = np.empty(1, np.float32)
    z = np.empty(1, np.float32)
    lib().orc_quantize_row_sr(_f(h), n, bits, asym, _i(code), _f(s), _f(z), None,
                              None if U is None else _f(_c32(U)))
    return code, float(s[0]), float(z[0])


def _sr_args(sr):
    """``sr``: None (round to nearest) or (seed, step) of stochastic rounding."""
    if sr is None:
        return 0, 0, 0
    seed, step = sr
    return 1, seed, step


def _ro(readout: str) -> int:
    if readout not in ("post", "pre"):
        raise ValueError("readout must be 'post' or 'pre'")
    return 1 if readout == "pre" else 0


def mamba2_step(st: State, x, dt, A, Bm, Cm, D, readout: str = "post", diag: bool = False,
                sr=None):
    """One decode token of one layer.  ``x`` [B][H][P], ``dt`` [B][H], ``A``/``D`` [H],
    ``Bm``/``Cm`` [B][G][N]; updates ``st`` in place and returns ``y`` [B][H][P]
    (plus the pre-rounding row and the rounded fp32 values when ``diag``).  ``sr``:
    (seed, step) for stochastic rounding."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    Bsz, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    assert st.rows == Bsz * H * P and st.n == N
    y = np.empty((Bsz, H, P), np.float32)
    hpre = np.empty((st.rows, N), np.float32) if diag else None
    vq = np.empty((st.rows, N), np.float32) if diag and st.fmt != "fp32" else None
    rc = lib().orc_mamba2_step_sr(Bsz, H, G, P, N, st.bits, st.asym, _i(st.code), _f(st.scale),
                                  _f(st.zero), _f(st.h), _f(x), _f(dt), _f(A), _f(Bm), _f(Cm),
                                  _f(D), _f(y), _ro(readout), _f(hpre), _f(vq), *_sr_args(sr))
    assert rc == 0
    return (y, hpre, vq) if diag else y


def mamba2_scan(st: State, x, dt, A, Bm, Cm, D, readout: str = "post", sr=None):
    """``T`` tokens, the state rounded after each.  ``x`` [B][T][H][P], ``dt`` [B][T][H],
    ``Bm``/``Cm`` [B][T][G][N]; returns ``y`` [B][T][H][P].  ``sr``: (seed, first step)."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    Bsz, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert st.rows == Bsz * H * P and st.n == N
    y = np.empty((Bsz, T, H, P), np.float32)
    rc = lib().orc_mamba2_scan_sr(Bsz, T, H, G, P, N, st.bits, st.asym, _i(st.code),
                                  _f(st.scale), _f(st.zero), _f(st.h), _f(x), _f(dt), _f(A), _f(Bm),
                                  _f(Cm), _f(D), _f(y), _ro(readout), *_sr_args(sr))
    assert rc == 0
    return y


def mamba2_rows_scan(st: State, x, dt, A, Bm, Cm, D, readout: str = "post", sr=None,
                     rows: int = 0, row_id=None):
    """``T`` tokens for independent rows with per-row inputs: ``x``/``dt`` [R][T], ``A``/``D`` [R],
    ``Bm``/``Cm`` [R][T][N]; returns ``y`` [R][T].  With ``sr`` = (seed, first step), row i draws
    the uniforms of state row ``row_id[i]`` of a state of ``rows`` rows."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    R, T = x.shape
    N = Bm.shape[2]
    assert st.rows == R and st.n == N
    y = np.empty((R, T), np.float32)
    ids = None
    if sr is not None:
        ids = np.ascontiguousarray(row_id, np.int64)
        assert ids.shape == (R,) and rows > 0
    rc = lib().orc_mamba2_rows_scan_sr(R, T, N, st.bits, st.asym, _i(st.code), _f(st.scale),
                                       _f(st.zero), _f(st.h), _f(x), _f(dt), _f(A), _f(Bm), _f(Cm),
                                       _f(D), _f(y), _ro(readout), *_sr_args(sr), rows,
                                       None if ids is None else
                                       ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    assert rc == 0
    return y


def delta_step(st: State, q, k, v, alpha, beta, Bsz: int, H: int, readout: str = "post",
               diag: bool = False, sr=None):
    """One delta-rule step for ``Bsz*H`` matrices of ``dk`` rows by ``dv``: ``q``/``k`` [B][H][dk],
    ``v`` [B][H][dv], ``alpha``/``beta`` [B][H]; returns ``o`` [B][H][dv]."""
    q, k, v, alpha, beta = map(_c32, (q, k, v, alpha, beta))
    dk, dv = k.shape[-1], v.shape[-1]
    assert st.rows == Bsz * H * dk and st.n == dv
    o = np.empty((Bsz, H, dv), np.float32)
    Spre = np.empty((st.rows, dv), np.float32) if diag else None
    vq = np.empty((st.rows, dv), np.float32) if diag and st.fmt != "fp32" else None
    rc = lib().orc_delta_step_sr(Bsz, H, dk, dv, st.bits, st.asym, _i(st.code), _f(st.scale),
                                 _f(st.zero), _f(st.h), _f(q), _f(k), _f(v), _f(alpha), _f(beta),
                                 _f(o), _ro(readout), _f(Spre), _f(vq), *_sr_args(sr))
    assert rc == 0
    return (o, Spre, vq) if diag else o


def kda_step(st: State, q, k, v, alpha, beta, Bsz: int, H: int, readout: str = "post",
             diag: bool = False, sr=None):
    """One KDA-style step (a decay per key channel): ``alpha`` [B][H][dk], the rest as
    ``delta_step``; returns ``o`` [B][H][dv]."""
    q, k, v, alpha, beta = map(_c32, (q, k, v, alpha, beta))
    dk, dv = k.shape[-1], v.shape[-1]
    assert st.rows == Bsz * H * dk and st.n == dv and alpha.size == Bsz * H * dk
    o = np.empty((Bsz, H, dv), np.float32)
    Spre = np.empty((st.rows, dv), np.float32) if diag else None
    vq = np.empty((st.rows, dv), np.float32) if diag and st.fmt != "fp32" else None
    rc = lib().orc_kda_step_sr(Bsz, H, dk, dv, st.bits, st.asym, _i(st.code), _f(st.scale),
                               _f(st.zero), _f(st.h), _f(q), _f(k), _f(v), _f(alpha), _f(beta),
                               _f(o), _ro(readout), _f(Spre), _f(vq), *_sr_args(sr))
    assert rc == 0
    return (o, Spre, vq) if diag else o


def mamba2_prefill(st: State, x, dt, A, Bm, Cm, D, chunk: int, readout: str = "post", sr=None):
    """``T`` prompt tokens with the state quantized only at chunk ends (and after the last
    token); shapes as ``mamba2_scan``; returns ``y`` [B][T][H][P]."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    Bsz, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert st.rows == Bsz * H * P and st.n == N
    y = np.empty((Bsz, T, H, P), np.float32)
    rc = lib().orc_mamba2_prefill_sr(Bsz, T, chunk, H, G, P, N, st.bits, st.asym, _i(st.code),
                                     _f(st.scale), _f(st.zero), _f(st.h), _f(x), _f(dt), _f(A), _f(Bm),
                                     _f(Cm), _f(D), _f(y), _ro(readout), *_sr_args(sr))
    assert rc == 0
    return y


# --------------------------------------------------------------------------
# DAMP-style two-tier delta state: rows rotated by Hs = H_128/16, the first
# NHI key channels of each matrix in half precision, the rest int8 asymmetric
# --------------------------------------------------------------------------
DAMP_NHI = 16


@dataclass
class DampState:
    """``hi`` [mats][nhi][dv] half values (as float32), ``code`` [mats*(dk-nhi)][dv] int32,
    ``scale``/``zero`` [mats*(dk-nhi)]; all rows in rotated coordinates."""
    mats: int
    dk: int
    dv: int
    nhi: int
    hi: np.ndarray
    code: np.ndarray
    scale: np.ndarray
    zero: np.ndarray

    def copy(self) -> "DampState":
        return DampState(self.mats, self.dk, self.dv, self.nhi, self.hi.copy(), self.code.copy(),
                         self.scale.copy(), self.zero.copy())

    def rotated(self) -> np.ndarray:
        """The stored rows' values [mats][dk][dv] (rotated coordinates)."""
        lo = dequantize_rows(self.code, self.scale, self.zero).reshape(self.mats, self.dk - self.nhi, self.dv)
        return np.concatenate([self.hi.reshape(self.mats, self.nhi, self.dv), lo], axis=1)


def round_half(x: float) -> float:
    return float(lib().orc_round_half(ctypes.c_float(x)))


def damp_from_fp32(S: np.ndarray, Bsz: int, H: int, nhi: int = DAMP_NHI) -> DampState:
    """The two-tier state of an fp32 state ``S`` [Bsz][H][dk][dv] (original coordinates)."""
    S = _c32(S)
    dk, dv = S.shape[-2], S.shape[-1]
    mats = Bsz * H
    hi = np.empty((mats, nhi, dv), np.float32)
    code = np.empty((mats * (dk - nhi), dv), np.int32)
    s = np.empty(mats * (dk - nhi), np.float32)
    z = np.empty(mats * (dk - nhi), np.float32)
    rc = lib().orc_damp_from_fp32(Bsz, H, dk, dv, nhi, _f(S), _f(hi), _i(code), _f(s), _f(z))
    assert rc == 0
    return DampState(mats, dk, dv, nhi, hi, code, s, z)


def damp_step(st: DampState, q, k, v, alpha, beta, Bsz: int, H: int, readout: str = "post",
              diag: bool = False, sr=None):
    """One step of the two-tier delta state; returns ``o`` [B][H][dv] (and the rotated
    pre-rounding matrices [mats][dk][dv] with ``diag``)."""
    q, k, v, alpha, beta = map(_c32, (q, k, v, alpha, beta))
    assert st.mats == Bsz * H
    o = np.empty((Bsz, H, st.dv), np.float32)
    Spre = np.empty((st.mats, st.dk, st.dv), np.float32) if diag else None
    rc = lib().orc_damp_step_sr(Bsz, H, st.dk, st.dv, st.nhi, _f(st.hi), _i(st.code), _f(st.scale),
                                _f(st.zero), _f(q), _f(k), _f(v), _f(alpha), _f(beta), _f(o),
                                _ro(readout), _f(Spre), *_sr_args(sr))
    assert rc == 0
    return (o, Spre) if diag else o


# --------------------------------------------------------------------------
# K host workers on disjoint slices.  Each worker runs the single-threaded oracle on
# its own sequences (or rows) through the same C entry points as above; ctypes
# releases the interpreter lock during each call, so the workers run in parallel.
# The results are those of the single calls: the slices share nothing.
# --------------------------------------------------------------------------
def workers() -> int:
    """Host workers for the parallel drivers: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _slices(n: int, k: int):
    k = max(1, min(k, n))
    return [(i * n // k, (i + 1) * n // k) for i in range(k)]


def _run_par(fn, parts, k: int):
    from concurrent.futures import ThreadPoolExecutor
    if k <= 1 or len(parts) <= 1:
        for p in parts:
            fn(*p)
        return
    with ThreadPoolExecutor(k) as ex:
        for f in [ex.submit(fn, *p) for p in parts]:
            f.result()


def _rows(a, r0, r1):
    return None if a is None else a[r0:r1]


def mamba2_step_par(st: State, x, dt, A, Bm, Cm, D, readout: str = "post", diag: bool = False,
                    k: int | None = None, sr=None):
    """``mamba2_step`` with the sequences split over ``k`` host workers (``sr``: (seed, step)
    for stochastic rounding, each row drawing the uniforms of its place in the whole state)."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    Bsz, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    assert st.rows == Bsz * H * P and st.n == N
    k = k or workers()
    y = np.empty((Bsz, H, P), np.float32)
    hpre = np.empty((st.rows, N), np.float32) if diag else None
    vq = np.empty((st.rows, N), np.float32) if diag and st.fmt != "fp32" else None

    def run(b0, b1):
        r0, r1 = b0 * H * P, b1 * H * P
        rc = lib().orc_mamba2_step_sr_part(b1 - b0, H, G, P, N, st.bits, st.asym, _i(_rows(st.code, r0, r1)),
                                           _f(_rows(st.scale, r0, r1)), _f(_rows(st.zero, r0, r1)),
                                           _f(_rows(st.h, r0, r1)), _f(x[b0:b1]), _f(dt[b0:b1]), _f(A),
                                           _f(Bm[b0:b1]), _f(Cm[b0:b1]), _f(D), _f(y[b0:b1]), _ro(readout),
                                           _f(_rows(hpre, r0, r1)), _f(_rows(vq, r0, r1)), *_sr_args(sr), b0,
                                           st.rows)
        assert rc == 0

    _run_par(run, _slices(Bsz, k), k)
    return (y, hpre, vq) if diag else y


def mamba2_scan_par(st: State, x, dt, A, Bm, Cm, D, readout: str = "post", k: int | None = None):
    """``mamba2_scan`` (round to nearest) with the sequences split over ``k`` host workers."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    Bsz, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert st.rows == Bsz * H * P and st.n == N
    k = k or workers()
    y = np.empty((Bsz, T, H, P), np.float32)

    def run(b0, b1):
        r0, r1 = b0 * H * P, b1 * H * P
        rc = lib().orc_mamba2_scan_sr(b1 - b0, T, H, G, P, N, st.bits, st.asym, _i(_rows(st.code, r0, r1)),
                                      _f(_rows(st.scale, r0, r1)), _f(_rows(st.zero, r0, r1)),
                                      _f(_rows(st.h, r0, r1)), _f(x[b0:b1]), _f(dt[b0:b1]), _f(A),
                                      _f(Bm[b0:b1]), _f(Cm[b0:b1]), _f(D), _f(y[b0:b1]), _ro(readout), 0, 0, 0)
        assert rc == 0

    _run_par(run, _slices(Bsz, k), k)
    return y


def mamba2_rows_scan_par(st: State, x, dt, A, Bm, Cm, D, readout: str = "post", k: int | None = None):
    """``mamba2_rows_scan`` (round to nearest) with the rows split over ``k`` host workers."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    R, T = x.shape
    N = Bm.shape[2]
    assert st.rows == R and st.n == N
    k = k or workers()
    y = np.empty((R, T), np.float32)

    def run(r0, r1):
        rc = lib().orc_mamba2_rows_scan_sr(r1 - r0, T, N, st.bits, st.asym, _i(_rows(st.code, r0, r1)),
                                           _f(_rows(st.scale, r0, r1)), _f(_rows(st.zero, r0, r1)),
                                           _f(_rows(st.h, r0, r1)), _f(x[r0:r1]), _f(dt[r0:r1]), _f(A[r0:r1]),
                                           _f(Bm[r0:r1]), _f(Cm[r0:r1]), _f(D[r0:r1]), _f(y[r0:r1]),
                                           _ro(readout), 0, 0, 0, 0, None)
        assert rc == 0

    _run_par(run, _slices(R, k), k)
    return y


def delta_step_par(st: State, q, k_vec, v, alpha, beta, Bsz: int, H: int, readout: str = "post",
                   diag: bool = False, k: int | None = None):
    """``delta_step`` (round to nearest) with the sequences split over ``k`` host workers."""
    q, k_vec, v, alpha, beta = map(_c32, (q, k_vec, v, alpha, beta))
    dk, dv = k_vec.shape[-1], v.shape[-1]
    assert st.rows == Bsz * H * dk and st.n == dv
    k = k or workers()
    o = np.empty((Bsz, H, dv), np.float32)
    Spre = np.empty((st.rows, dv), np.float32) if diag else None
    vq = np.empty((st.rows, dv), np.float32) if diag and st.fmt != "fp32" else None

    def run(b0, b1):
        r0, r1 = b0 * H * dk, b1 * H * dk
        rc = lib().orc_delta_step_sr(b1 - b0, H, dk, dv, st.bits, st.asym, _i(_rows(st.code, r0, r1)),
                                     _f(_rows(st.scale, r0, r1)), _f(_rows(st.zero, r0, r1)),
                                     _f(_rows(st.h, r0, r1)), _f(q[b0:b1]), _f(k_vec[b0:b1]), _f(v[b0:b1]),
                                     _f(alpha[b0:b1]), _f(beta[b0:b1]), _f(o[b0:b1]), _ro(readout),
                                     _f(_rows(Spre, r0, r1)), _f(_rows(vq, r0, r1)), 0, 0, 0)
        assert rc == 0

    _run_par(run, _slices(Bsz, k), k)
    return (o, Spre, vq) if diag else o


def kda_step_par(st: State, q, k_vec, v, alpha, beta, Bsz: int, H: int, readout: str = "post",
                 k: int | None = None):
    """``kda_step`` (round to nearest) with the sequences split over ``k`` host workers."""
    q, k_vec, v, alpha, beta = map(_c32, (q, k_vec, v, alpha, beta))
    dk, dv = k_vec.shape[-1], v.shape[-1]
    assert st.rows == Bsz * H * dk and st.n == dv and alpha.size == Bsz * H * dk
    k = k or workers()
    o = np.empty((Bsz, H, dv), np.float32)

    def run(b0, b1):
        r0, r1 = b0 * H * dk, b1 * H * dk
        rc = lib().orc_kda_step_sr(b1 - b0, H, dk, dv, st.bits, st.asym, _i(_rows(st.code, r0, r1)),
                                   _f(_rows(st.scale, r0, r1)), _f(_rows(st.zero, r0, r1)),
                                   _f(_rows(st.h, r0, r1)), _f(q[b0:b1]), _f(k_vec[b0:b1]), _f(v[b0:b1]),
                                   _f(alpha[b0:b1]), _f(beta[b0:b1]), _f(o[b0:b1]), _ro(readout), None, None,
                                   0, 0, 0)
        assert rc == 0

    _run_par(run, _slices(Bsz, k), k)
    return o


def damp_step_par(st: "DampState", q, k_vec, v, alpha, beta, Bsz: int, H: int, readout: str = "post",
                  k: int | None = None):
    """``damp_step`` (round to nearest) with the sequences split over ``k`` host workers."""
    q, k_vec, v, alpha, beta = map(_c32, (q, k_vec, v, alpha, beta))
    assert st.mats == Bsz * H
    k = k or workers()
    o = np.empty((Bsz, H, st.dv), np.float32)
    nlo = st.dk - st.nhi

    def run(b0, b1):
        m0, m1 = b0 * H, b1 * H
        rc = lib().orc_damp_step_sr(b1 - b0, H, st.dk, st.dv, st.nhi, _f(st.hi[m0:m1]),
                                    _i(st.code[m0 * nlo:m1 * nlo]), _f(st.scale[m0 * nlo:m1 * nlo]),
                                    _f(st.zero[m0 * nlo:m1 * nlo]), _f(q[b0:b1]), _f(k_vec[b0:b1]), _f(v[b0:b1]),
                                    _f(alpha[b0:b1]), _f(beta[b0:b1]), _f(o[b0:b1]), _ro(readout), None, 0, 0, 0)
        assert rc == 0

    _run_par(run, _slices(Bsz, k), k)
    return o


def mamba2_prefill_par(st: State, x, dt, A, Bm, Cm, D, chunk: int, readout: str = "post",
                       k: int | None = None):
    """``mamba2_prefill`` (round to nearest) with the sequences split over ``k`` host workers."""
    x, dt, A, Bm, Cm, D = map(_c32, (x, dt, A, Bm, Cm, D))
    Bsz, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert st.rows == Bsz * H * P and st.n == N
    k = k or workers()
    y = np.empty((Bsz, T, H, P), np.float32)

    def run(b0, b1):
        r0, r1 = b0 * H * P, b1 * H * P
        rc = lib().orc_mamba2_prefill_sr(b1 - b0, T, chunk, H, G, P, N, st.bits, st.asym,
                                         _i(_rows(st.code, r0, r1)), _f(_rows(st.scale, r0, r1)),
                                         _f(_rows(st.zero, r0, r1)), _f(_rows(st.h, r0, r1)), _f(x[b0:b1]),
                                         _f(dt[b0:b1]), _f(A), _f(Bm[b0:b1]), _f(Cm[b0:b1]), _f(D), _f(y[b0:b1]),
                                         _ro(readout), 0, 0, 0)
        assert rc == 0

    _run_par(run, _slices(Bsz, k), k)
    return y


def damp_from_fp32_par(S: np.ndarray, Bsz: int, H: int, nhi: int = DAMP_NHI, k: int | None = None) -> DampState:
    """``damp_from_fp32`` with the sequences split over ``k`` host workers."""
    S = _c32(S)
    dk, dv = S.shape[-2], S.shape[-1]
    mats = Bsz * H
    nlo = dk - nhi
    hi = np.empty((mats, nhi, dv), np.float32)
    code = np.empty((mats * nlo, dv), np.int32)
    s = np.empty(mats * nlo, np.float32)
    z = np.empty(mats * nlo, np.float32)
    k = k or workers()
    S4 = S.reshape(Bsz, H, dk, dv)

    def run(b0, b1):
        m0, m1 = b0 * H, b1 * H
        rc = lib().orc_damp_from_fp32(b1 - b0, H, dk, dv, nhi, _f(S4[b0:b1]), _f(hi[m0:m1]),
                                      _i(code[m0 * nlo:m1 * nlo]), _f(s[m0 * nlo:m1 * nlo]), _f(z[m0 * nlo:m1 * nlo]))
        assert rc == 0

    _run_par(run, _slices(Bsz, k), k)
    return DampState(mats, dk, dv, nhi, hi, code, s, z)
