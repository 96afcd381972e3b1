"""Seeded synthetic inputs for the quantized recurrent-state update.

This module only draws numbers.  It holds none of the method's arithmetic and
is imported, unchanged, by the tests, the bench and the smoke check, which hand
the same arrays to the CPU oracle and to the GPU library.

Every value is a pure function of (seed, stream, layer, flat index): a
SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) applied to a Weyl counter gives 64 random
bits, the top 53 of them a uniform in (0, 1), and the Box-Muller transform
(Box and Muller, 1958) two uniforms a standard normal, all in float64 and
rounded once to float32.  Because the generator is counter based, any subset
of a tensor (say the rows a test samples) regenerates bit-identically without
drawing the rest.

Distributions (the Mamba-2 and delta-rule workloads of the quantized-state
pages and of the benchmark configurations built on them):

* ``A_h = -exp(U(0, ln 16))`` per head and layer.
* ``dt = softplus(N(0,1) + b_h)`` per (token, sequence, head), with ``b_h``
  chosen so that the decay ``lambda = exp(dt*A)`` of head ``h`` has its median
  in decay band ``h mod 3``: lambda <= 0.9, 0.9 < lambda <= 0.99 and
  lambda > 0.99 (the three bands of the ssm-state-quantization README,
  Setup).  The band medians of ``-ln lambda`` are 0.325, 0.0325 and 0.00325,
  one decade apart with the middle one at the geometric centre of its band.
* ``x ~ N(0,1)``; ``B, C ~ N(0,1)/sqrt(N)``; ``D ~ N(0,1)`` per head.
* Initial states: ``N(0,1)`` rows, each row independently an outlier with
  probability 0.05 and then scaled by 20.
* Delta rule: ``k, q`` are ``N(0,1)`` vectors normalised to unit L2 norm,
  ``v ~ N(0,1)``, ``alpha = sigmoid(N(3,1))``, ``beta = sigmoid(N(0,1))``; the
  KDA-style step draws ``alpha`` per key channel from the same distribution.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "STREAMS", "uniform", "normal", "band_of_head", "BAND_MEDIAN_NEG_LOG_LAMBDA",
    "mamba2_head_params", "mamba2_step_inputs", "mamba2_scan_inputs", "mamba2_rows_scan_inputs",
    "init_state", "init_state_rows", "delta_inputs", "kda_alpha",
]

_GOLD = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

# one independent stream per tensor
STREAMS = {
    "A": 1, "dt": 2, "x": 3, "B": 4, "C": 5, "D": 6, "init": 7, "outlier": 8,
    "k": 9, "q": 10, "v": 11, "alpha": 12, "beta": 13, "alpha_k": 14,
}

# median of -ln(lambda) for decay bands 0 (lambda <= 0.9), 1 (0.9..0.99], 2 (> 0.99)
BAND_MEDIAN_NEG_LOG_LAMBDA = (0.325, 0.0325, 0.00325)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int, layer: int) -> np.uint64:
    # python ints wrap explicitly, so no numpy scalar overflow warnings
    def mix(v: int) -> int:
        v &= _MASK64
        v = ((v ^ (v >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        v = ((v ^ (v >> 27)) * 0x94D049BB133111EB) & _MASK64
        return v ^ (v >> 31)
    k = mix(seed + 0x9E3779B97F4A7C15)
    k = mix(k ^ (stream * 0xD1B54A32D192ED03))
    k = mix(k ^ (layer * 0xABC98388FB8FAC03))
    return np.uint64(k)


def _bits(seed: int, stream: int, layer: int, idx: np.ndarray) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(_key(seed, stream, layer) + (idx + np.uint64(1)) * _GOLD)


def uniform(seed: int, stream: int, layer: int, idx) -> np.ndarray:
    """Uniform in (0, 1), float64, one per counter in ``idx``."""
    b = _bits(seed, stream, layer, idx) >> np.uint64(11)
    return (b.astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed: int, stream: int, layer: int, idx) -> np.ndarray:
    """Standard normal, float64, one per counter in ``idx`` (Box-Muller, cosine branch)."""
    idx = np.asarray(idx, dtype=np.uint64)
    u1 = uniform(seed, stream, layer, idx * np.uint64(2))
    u2 = uniform(seed, stream, layer, idx * np.uint64(2) + np.uint64(1))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.where(x > 30.0, x, np.log1p(np.exp(np.minimum(x, 30.0))))


def band_of_head(h) -> np.ndarray:
    return np.asarray(h) % 3


def mamba2_head_params(seed: int, layer: int, H: int):
    """Per-head ``A`` (float32, < 0), ``D`` (float32) and the softplus bias ``b_h`` (float64)."""
    h = np.arange(H, dtype=np.uint64)
    A = _f32(-np.exp(uniform(seed, STREAMS["A"], layer, h) * math.log(16.0)))
    D = _f32(normal(seed, STREAMS["D"], layer, h))
    m = np.asarray(BAND_MEDIAN_NEG_LOG_LAMBDA)[band_of_head(np.arange(H))]
    bias = np.log(np.expm1(m / np.abs(A.astype(np.float64))))
    return A, D, bias


def _scan_block(seed, layer, Bsz, t0, t1, H, G, P, N, bias):
    """dt, x, Bm, Cm of tokens t0 .. t1-1 ([Bsz][t1-t0][...]), indexed as in a full scan."""
    b, t, h = np.meshgrid(np.arange(Bsz), np.arange(t0, t1), np.arange(H), indexing="ij")
    dt_idx = ((t.astype(np.uint64) * Bsz + b) * H + h).astype(np.uint64)
    dt = _f32(_softplus(normal(seed, STREAMS["dt"], layer, dt_idx) + bias[h]))
    x_idx = (dt_idx[..., None] * np.uint64(P) + np.arange(P, dtype=np.uint64))
    x = _f32(normal(seed, STREAMS["x"], layer, x_idx))
    b2, t2, g2 = np.meshgrid(np.arange(Bsz), np.arange(t0, t1), np.arange(G), indexing="ij")
    bc_idx = (((t2.astype(np.uint64) * Bsz + b2) * G + g2)[..., None] * np.uint64(N)
              + np.arange(N, dtype=np.uint64))
    sc = 1.0 / math.sqrt(N)
    Bm = _f32(normal(seed, STREAMS["B"], layer, bc_idx) * sc)
    Cm = _f32(normal(seed, STREAMS["C"], layer, bc_idx) * sc)
    return x, dt, Bm, Cm


def mamba2_scan_inputs(seed: int, layer: int, Bsz: int, T: int, H: int, G: int, P: int, N: int,
                       threads: int = 1):
    """Inputs of a ``T``-token scan of one layer.

    Returns ``(x, dt, Bm, Cm, A, D)`` with ``x`` [Bsz][T][H][P], ``dt`` [Bsz][T][H] (already through
    softplus, > 0), ``Bm``/``Cm`` [Bsz][T][G][N], ``A``/``D`` [H], all float32 C-contiguous.
    ``threads`` > 1 draws blocks of tokens concurrently (same values: the generator is counter
    based).
    """
    A, D, bias = mamba2_head_params(seed, layer, H)
    if threads <= 1 or Bsz * T * H * P < (1 << 22):
        x, dt, Bm, Cm = _scan_block(seed, layer, Bsz, 0, T, H, G, P, N, bias)
        return x, dt, Bm, Cm, A, D
    from concurrent.futures import ThreadPoolExecutor
    x = np.empty((Bsz, T, H, P), np.float32)
    dt = np.empty((Bsz, T, H), np.float32)
    Bm = np.empty((Bsz, T, G, N), np.float32)
    Cm = np.empty((Bsz, T, G, N), np.float32)
    # blocks of about 2^20 values of x, so that the float64 temporaries stay small
    step = max(1, min(T, (1 << 20) // max(1, Bsz * H * P)))

    def fill(t0):
        t1 = min(T, t0 + step)
        x[:, t0:t1], dt[:, t0:t1], Bm[:, t0:t1], Cm[:, t0:t1] = _scan_block(seed, layer, Bsz, t0, t1, H, G, P, N,
                                                                            bias)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(0, T, step)))
    return x, dt, Bm, Cm, A, D


def mamba2_step_inputs(seed: int, layer: int, Bsz: int, H: int, G: int, P: int, N: int, t: int = 0):
    """Inputs of decode token ``t`` of one layer: ``x`` [Bsz][H][P], ``dt`` [Bsz][H],
    ``Bm``/``Cm`` [Bsz][G][N], ``A``/``D`` [H]; identical to slice ``t`` of a scan's inputs."""
    A, D, bias = mamba2_head_params(seed, layer, H)
    b, h = np.meshgrid(np.arange(Bsz), np.arange(H), indexing="ij")
    dt_idx = ((np.uint64(t) * np.uint64(Bsz) + b.astype(np.uint64)) * np.uint64(H)
              + h.astype(np.uint64))
    dt = _f32(_softplus(normal(seed, STREAMS["dt"], layer, dt_idx) + bias[h]))
    x = _f32(normal(seed, STREAMS["x"], layer,
                    dt_idx[..., None] * np.uint64(P) + np.arange(P, dtype=np.uint64)))
    b2, g2 = np.meshgrid(np.arange(Bsz), np.arange(G), indexing="ij")
    bc_idx = (((np.uint64(t) * np.uint64(Bsz) + b2.astype(np.uint64)) * np.uint64(G)
               + g2.astype(np.uint64))[..., None] * np.uint64(N) + np.arange(N, dtype=np.uint64))
    sc = 1.0 / math.sqrt(N)
    Bm = _f32(normal(seed, STREAMS["B"], layer, bc_idx) * sc)
    Cm = _f32(normal(seed, STREAMS["C"], layer, bc_idx) * sc)
    return x, dt, Bm, Cm, A, D


def mamba2_rows_scan_inputs(seed: int, layer: int, Bsz: int, T: int, H: int, G: int, P: int,
                            N: int, rows: np.ndarray):
    """The scan inputs that the state rows ``rows`` (flat (b*H + h)*P + p indices) read, regenerated
    without drawing the rest: ``x`` [R][T], ``dt`` [R][T], ``Bm``/``Cm`` [R][T][N], ``A``/``D`` [R]."""
    rows = np.asarray(rows, dtype=np.int64)
    A, D, bias = mamba2_head_params(seed, layer, H)
    b = rows // (H * P)
    h = (rows // P) % H
    p = rows % P
    g = h // (H // G)
    t = np.arange(T)
    dt_idx = ((t[None, :].astype(np.uint64) * np.uint64(Bsz) + b[:, None].astype(np.uint64))
              * np.uint64(H) + h[:, None].astype(np.uint64))
    dt = _f32(_softplus(normal(seed, STREAMS["dt"], layer, dt_idx) + bias[h][:, None]))
    x = _f32(normal(seed, STREAMS["x"], layer, dt_idx * np.uint64(P) + p[:, None].astype(np.uint64)))
    bc_idx = (((t[None, :].astype(np.uint64) * np.uint64(Bsz) + b[:, None].astype(np.uint64))
               * np.uint64(G) + g[:, None].astype(np.uint64))[..., None] * np.uint64(N)
              + np.arange(N, dtype=np.uint64))
    sc = 1.0 / math.sqrt(N)
    Bm = _f32(normal(seed, STREAMS["B"], layer, bc_idx) * sc)
    Cm = _f32(normal(seed, STREAMS["C"], layer, bc_idx) * sc)
    return x, dt, Bm, Cm, A[h], D[h]


def init_state_rows(seed: int, layer: int, rows: np.ndarray, N: int,
                    outlier_p: float = 0.05, outlier_scale: float = 20.0) -> np.ndarray:
    """Initial fp32 state of the given flat rows: N(0,1) entries, a row an outlier (x20) with
    probability 0.05.  Returns [len(rows)][N] float32."""
    rows = np.asarray(rows, dtype=np.uint64)
    idx = rows[:, None] * np.uint64(N) + np.arange(N, dtype=np.uint64)
    v = normal(seed, STREAMS["init"], layer, idx)
    out = uniform(seed, STREAMS["outlier"], layer, rows) < outlier_p
    v = np.where(out[:, None], v * outlier_scale, v)
    return _f32(v)


def init_state(seed: int, layer: int, nrows: int, N: int, threads: int = 1, **kw) -> np.ndarray:
    """Initial fp32 state of rows 0..nrows-1: [nrows][N] float32 (see ``init_state_rows``).
    ``threads`` > 1 draws row chunks concurrently (same values: the generator is counter based)."""
    if threads <= 1 or nrows < 4096:
        return init_state_rows(seed, layer, np.arange(nrows, dtype=np.uint64), N, **kw)
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty((nrows, N), np.float32)
    step = max(1024, (nrows + 4 * threads - 1) // (4 * threads))

    def work(r0):
        r1 = min(nrows, r0 + step)
        out[r0:r1] = init_state_rows(seed, layer, np.arange(r0, r1, dtype=np.uint64), N, **kw)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(0, nrows, step)))
    return out


def delta_inputs(seed: int, layer: int, Bsz: int, H: int, dk: int, dv: int, t: int = 0):
    """Inputs of one delta-rule step: ``q``, ``k`` [Bsz][H][dk] (unit L2 norm), ``v`` [Bsz][H][dv],
    ``alpha`` = sigmoid(N(3,1)) and ``beta`` = sigmoid(N(0,1)) [Bsz][H]; float32."""
    bh = (np.uint64(t) * np.uint64(Bsz * H) + np.arange(Bsz * H, dtype=np.uint64)).reshape(Bsz, H)

    def unit(stream):
        r = normal(seed, stream, layer, bh[..., None] * np.uint64(dk) + np.arange(dk, dtype=np.uint64))
        return _f32(r / np.sqrt(np.sum(r * r, axis=-1, keepdims=True)))

    k = unit(STREAMS["k"])
    q = unit(STREAMS["q"])
    v = _f32(normal(seed, STREAMS["v"], layer,
                    bh[..., None] * np.uint64(dv) + np.arange(dv, dtype=np.uint64)))
    alpha = _f32(1.0 / (1.0 + np.exp(-(3.0 + normal(seed, STREAMS["alpha"], layer, bh)))))
    beta = _f32(1.0 / (1.0 + np.exp(-normal(seed, STREAMS["beta"], layer, bh))))
    return q, k, v, alpha, beta


def kda_alpha(seed: int, layer: int, Bsz: int, H: int, dk: int, t: int = 0):
    """A decay per key channel for the KDA-style step: ``sigmoid(N(3,1))`` per (sequence, head,
    key channel), [Bsz][H][dk] float32 (the scalar gate's distribution, drawn per channel)."""
    idx = (np.uint64(t) * np.uint64(Bsz * H * dk) + np.arange(Bsz * H * dk, dtype=np.uint64))
    return _f32(1.0 / (1.0 + np.exp(-(3.0 + normal(seed, STREAMS["alpha_k"], layer, idx))))).reshape(Bsz, H, dk)
