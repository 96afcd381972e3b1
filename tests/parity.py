"""Parity helpers shared by the GPU tests and the smoke check.

* code (un)packing for the public state layout of ``include/ssq.h``
  (int4: entry 2j in the low nibble of byte j, symmetric codes in two's complement);
* moving a state between the oracle and the GPU: a GPU state can be set from
  the oracle's (teacher forcing) and read back; nothing read back from the GPU
  is ever fed to the oracle;
* the accuracy contract: integer codes bit-exact, except at most 1e-4 of the
  codes differing by one where the oracle's rounded fp32 value lies within one
  ulp of the boundary between the two codes; scales and zero points bit-exact
  outside rows holding such a code; float outputs compared relative to
  max(|ref|, RMS of the reference over its block).
"""
from __future__ import annotations

import numpy as np
import torch

import mamba_decode_amd as ssq
import oracle

F64 = np.float64
FMT_ID = ssq.FORMAT_NAMES


def unpack_codes(raw: np.ndarray, fmt: str) -> np.ndarray:
    raw = np.asarray(raw, np.uint8)
    if fmt == "int8_asym":
        return raw.astype(np.int32)
    if fmt == "int8_sym":
        return raw.view(np.int8).astype(np.int32)
    lo = (raw & 0x0F).astype(np.int32)
    hi = (raw >> 4).astype(np.int32)
    out = np.empty((raw.shape[0], raw.shape[1] * 2), np.int32)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    if fmt == "int4_sym":
        out = ((out ^ 8) - 8).astype(np.int32)
    return out


def pack_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    codes = np.asarray(codes, np.int64)
    if fmt in ("int8_asym", "int8_sym"):
        return (codes & 0xFF).astype(np.uint8)
    c = (codes & 0x0F).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def new_gpu_state(desc, init: np.ndarray | None = None):
    """A GPU state in torch-held storage (so that the test can read its bytes)."""
    storage = torch.empty(ssq.ssq_state_bytes(desc), dtype=torch.uint8, device="cuda")
    init_t = None if init is None else torch.from_numpy(np.ascontiguousarray(init, np.float32)).cuda()
    st = ssq.ssq_alloc_state(desc, storage=storage, init=init_t)
    torch.cuda.synchronize()
    return st


def write_gpu_state(gst, ost: oracle.State):
    """Overwrite a GPU state with the oracle's state (teacher forcing)."""
    codes, scale, zero = gst.regions()
    if ost.fmt == "fp32":
        codes.copy_(torch.from_numpy(ost.h))
    else:
        codes.copy_(torch.from_numpy(pack_codes(ost.code, ost.fmt)))
        scale.copy_(torch.from_numpy(ost.scale))
        if zero is not None:
            zero.copy_(torch.from_numpy(ost.zero))
    torch.cuda.synchronize()


def read_gpu_state(gst, fmt: str) -> dict:
    torch.cuda.synchronize()
    codes, scale, zero = gst.regions()
    if fmt == "fp32":
        return {"h": codes.cpu().numpy().copy()}
    out = {"code": unpack_codes(codes.cpu().numpy(), fmt), "scale": scale.cpu().numpy().copy()}
    out["zero"] = zero.cpu().numpy().copy() if zero is not None else np.zeros_like(out["scale"])
    return out


def block_rel(got, ref, axis=-1) -> float:
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    rms = np.sqrt(np.mean(ref * ref, axis=axis, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den)) if got.size else 0.0


def check_codes(gpu: dict, orc_code, orc_scale, orc_zero, orc_v, fmt: str, where: str = ""):
    """Assert the contract for one step's codes; returns the number of (allowed) flipped codes.

    orc_v is the oracle's fp32 value that was rounded (None when the step cannot be checked
    for near-ties, in which case every code must match)."""
    gc = gpu["code"]
    mism = gc != orc_code
    n = int(mism.sum())
    if n:
        assert orc_v is not None, f"{where}: {n} codes differ"
        r, c = np.nonzero(mism)
        assert np.all(np.abs(gc[r, c] - orc_code[r, c]) == 1), f"{where}: a code differs by more than one"
        assert n <= max(1, 1e-4 * gc.size), f"{where}: {n} of {gc.size} codes differ"
        v = orc_v[r, c].astype(np.float32)
        zz = orc_zero[r].astype(F64) if fmt.endswith("asym") else 0.0
        t = v.astype(F64) + zz
        boundary = (gc[r, c].astype(F64) + orc_code[r, c]) / 2.0
        ulp = np.spacing(np.abs(v)).astype(F64)
        assert np.all(np.abs(t - boundary) <= ulp), f"{where}: a flipped code is not at a rounding boundary"
    ok_rows = ~mism.any(axis=1)
    assert np.array_equal(gpu["scale"][ok_rows].view(np.uint32), orc_scale[ok_rows].view(np.uint32)), \
        f"{where}: scales differ"
    if fmt.endswith("asym"):
        assert np.array_equal(gpu["zero"][ok_rows], orc_zero[ok_rows]), f"{where}: zero points differ"
    return n


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


# ---------------------------------------------------------------------------
# two-tier delta state
# ---------------------------------------------------------------------------
def write_gpu_damp(gst, ost: "oracle.DampState"):
    codes, scale, zero = gst.regions()
    codes.copy_(torch.from_numpy(pack_codes(ost.code, "int8_asym")))
    scale.copy_(torch.from_numpy(ost.scale))
    zero.copy_(torch.from_numpy(ost.zero))
    gst.hi_region().copy_(torch.from_numpy(ost.hi.astype(np.float16)))
    torch.cuda.synchronize()


def read_gpu_damp(gst) -> dict:
    torch.cuda.synchronize()
    codes, scale, zero = gst.regions()
    return {"code": unpack_codes(codes.cpu().numpy(), "int8_asym"), "scale": scale.cpu().numpy().copy(),
            "zero": zero.cpu().numpy().copy(), "hi": gst.hi_region().cpu().numpy().astype(np.float32)}


def y_within_sum_bound(yg, yo, Crows, rrows, dx, terms: int = 128):
    """y read as an fp32 sum: |y_gpu - y_exact| <= 2*terms*u*sum_n |C_n r_n| + 2u|y_exact| + u|D x|
    for every row, where r is the row the readout names (the dequantized new row, or the row
    before rounding) and y_exact the oracle's (the sum in double, rounded once).  This bounds any
    fp32 summation order of the terms; the head-relative tolerance alone cannot hold to 1e-5 when
    a whole head's sum cancels (a zero start state makes every row of a head a multiple of B).
    Crows [R][N] (the C each row reads), rrows [R][N], yg/yo/dx [R].  Returns the largest ratio
    of the error to its bound."""
    u = 2.0 ** -24
    yg = np.asarray(yg, F64).reshape(-1)
    yo = np.asarray(yo, F64).reshape(-1)
    dx = np.asarray(dx, F64).reshape(-1)
    mag = np.einsum("rn,rn->r", np.abs(np.asarray(Crows, np.float32)), np.abs(np.asarray(rrows, np.float32)),
                    dtype=F64)
    bound = 2 * terms * u * mag + 2 * u * np.abs(yo) + u * np.abs(dx) + 1e-37
    err = np.abs(yg - yo)
    return float(np.max(err / bound))
