"""Python binding of ``libssq.so``: the quantized recurrent-state update on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels
behind the C ABI of ``include/ssq.h``; PyTorch supplies device memory (tensor
data pointers) and the stream (``torch.cuda.current_stream()``).  The binding
checks that tensors have the dtype, device, contiguity and size that the
state's description implies, so that the kernels never see a short buffer.

Importing this package fails loudly if the library has not been built
(``python -m mamba_decode_amd.build``): there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported first: the library binds to the HIP runtime torch has loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSQ_LIBRARY names another build of the same sources (the host tests' sanitized build)
LIB_PATH = os.environ.get("SSQ_LIBRARY") or os.path.join(_HERE, "libssq.so")

# ssq_status
SSQ_OK, SSQ_ERR_INVALID_ARG, SSQ_ERR_UNSUPPORTED, SSQ_ERR_KIND_MISMATCH, SSQ_ERR_ALLOC, SSQ_ERR_DEVICE = range(6)
# ssq_format
SSQ_FP32, SSQ_INT8_SYM, SSQ_INT8_ASYM, SSQ_INT4_SYM, SSQ_INT4_ASYM, SSQ_DAMP = range(6)
SSQ_DAMP_NHI = 16
# ssq_kind
SSQ_MAMBA2, SSQ_DELTA = 0, 1
# ssq_readout
SSQ_READ_POST_QUANT, SSQ_READ_PRE_QUANT = 0, 1
# ssq_rounding
SSQ_ROUND_NEAREST, SSQ_ROUND_STOCHASTIC = 0, 1

FORMAT_NAMES = {"fp32": SSQ_FP32, "int8_sym": SSQ_INT8_SYM, "int8_asym": SSQ_INT8_ASYM,
                "int4_sym": SSQ_INT4_SYM, "int4_asym": SSQ_INT4_ASYM, "damp": SSQ_DAMP}
FORMAT_BITS = {SSQ_FP32: 32, SSQ_INT8_SYM: 8, SSQ_INT8_ASYM: 8, SSQ_INT4_SYM: 4, SSQ_INT4_ASYM: 4, SSQ_DAMP: 8}


class SsqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


class ssq_desc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("format", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("ngroups", ctypes.c_int32),
                ("rows_per_head", ctypes.c_int32), ("row_len", ctypes.c_int32)]


class ssq_layout(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_size_t), ("row_bytes", ctypes.c_size_t),
                ("codes_offset", ctypes.c_size_t), ("scale_offset", ctypes.c_size_t),
                ("zero_offset", ctypes.c_size_t), ("total_bytes", ctypes.c_size_t),
                ("hi_offset", ctypes.c_size_t), ("counter_offset", ctypes.c_size_t)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m mamba_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, f32p = ctypes.c_void_p, ctypes.c_void_p
    st = ctypes.c_int
    dp = ctypes.POINTER(ssq_desc)
    L.ssq_state_bytes.argtypes = [dp]
    L.ssq_state_bytes.restype = ctypes.c_size_t
    L.ssq_state_layout.argtypes = [dp, ctypes.POINTER(ssq_layout)]
    L.ssq_state_layout.restype = st
    L.ssq_alloc_state.argtypes = [dp, vp, f32p, vp, ctypes.POINTER(ctypes.c_void_p)]
    L.ssq_alloc_state.restype = st
    L.ssq_free_state.argtypes = [vp]
    L.ssq_free_state.restype = st
    L.ssq_state_info.argtypes = [vp, dp, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ssq_layout)]
    L.ssq_state_info.restype = st
    L.ssq_decode_step.argtypes = [vp, f32p, f32p, f32p, f32p, f32p, f32p, f32p, ctypes.c_int32, vp]
    L.ssq_decode_step.restype = st
    L.ssq_scan.argtypes = [vp, ctypes.c_int32, f32p, f32p, f32p, f32p, f32p, f32p, f32p, ctypes.c_int32, vp]
    L.ssq_scan.restype = st
    L.ssq_delta_step.argtypes = [vp, f32p, f32p, f32p, f32p, f32p, f32p, ctypes.c_int32, vp]
    L.ssq_delta_step.restype = st
    L.ssq_dequant.argtypes = [vp, f32p, vp]
    L.ssq_dequant.restype = st
    L.ssq_stream_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    L.ssq_stream_copy.restype = st
    L.ssq_status_string.argtypes = [ctypes.c_int32]
    L.ssq_status_string.restype = ctypes.c_char_p
    L.ssq_last_error.argtypes = []
    L.ssq_last_error.restype = ctypes.c_char_p
    L.ssq_prefill.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, f32p, f32p, f32p, f32p, f32p, f32p, f32p,
                              ctypes.c_int32, vp]
    L.ssq_prefill.restype = st
    L.ssq_kda_step.argtypes = [vp, f32p, f32p, f32p, f32p, f32p, f32p, ctypes.c_int32, vp]
    L.ssq_kda_step.restype = st
    u64 = ctypes.c_uint64
    L.ssq_set_rounding.argtypes = [vp, ctypes.c_int32, u64, u64, vp]
    L.ssq_set_rounding.restype = st
    L.ssq_get_rounding.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(u64), ctypes.POINTER(u64), vp]
    L.ssq_get_rounding.restype = st
    return L


lib = _load()


def ssq_status_string(status: int) -> str:
    return lib.ssq_status_string(status).decode()


def ssq_last_error() -> str:
    return lib.ssq_last_error().decode()


def _check(status: int, where: str):
    if status != SSQ_OK:
        raise SsqError(status, where, ssq_last_error() or ssq_status_string(status))


def make_desc(kind: int, fmt, batch: int, nheads: int, rows_per_head: int, row_len: int = 128,
              ngroups: int = 1) -> ssq_desc:
    if isinstance(fmt, str):
        fmt = FORMAT_NAMES[fmt]
    return ssq_desc(kind, fmt, batch, nheads, ngroups, rows_per_head, row_len)


def ssq_state_bytes(desc: ssq_desc) -> int:
    return int(lib.ssq_state_bytes(ctypes.byref(desc)))


def ssq_state_layout(desc: ssq_desc) -> ssq_layout:
    lay = ssq_layout()
    _check(lib.ssq_state_layout(ctypes.byref(desc), ctypes.byref(lay)), "ssq_state_layout")
    return lay


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, name: str, numel, dtype=torch.float32) -> ctypes.c_void_p:
    """Device pointer of a tensor; ``numel`` None skips the size check (the call is rejected by
    the library anyway, e.g. for a state of the other kind)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


class State:
    """A state handle plus the torch tensor that holds its storage (if torch allocated it)."""

    def __init__(self, handle: ctypes.c_void_p, desc: ssq_desc, layout: ssq_layout, storage):
        self.handle = handle
        self.desc = desc
        self.layout = layout
        self.storage = storage  # torch uint8 tensor, or None when the library owns the memory

    @property
    def rows(self) -> int:
        return int(self.layout.rows)

    def regions(self):
        """(codes, scale, zero) views of a torch-held storage: codes [rows][row_bytes] uint8
        (fp32 format: [rows][row_len] float32), scale/zero [rows] float32 or None."""
        if self.storage is None:
            raise ValueError("the library owns this state's memory; pass a torch storage to view it")
        L, s = self.layout, self.storage
        n = self.rows
        if self.desc.format == SSQ_DAMP:  # the uint8 rows only; hi_region() holds the half rows
            n = n // self.desc.rows_per_head * (self.desc.rows_per_head - SSQ_DAMP_NHI)
        if self.desc.format == SSQ_FP32:
            codes = s[: n * L.row_bytes].view(torch.float32).view(n, self.desc.row_len)
            return codes, None, None
        codes = s[: n * L.row_bytes].view(n, L.row_bytes)
        scale = s[L.scale_offset: L.scale_offset + 4 * n].view(torch.float32)
        zero = s[L.zero_offset: L.zero_offset + 4 * n].view(torch.float32) if L.zero_offset else None
        return codes, scale, zero

    def hi_region(self):
        """Two-tier state: the half rows [mats][16][row_len] as float16 (a view of the storage)."""
        L, s, d = self.layout, self.storage, self.desc
        mats = self.rows // d.rows_per_head
        nb = mats * SSQ_DAMP_NHI * d.row_len * 2
        return s[L.hi_offset: L.hi_offset + nb].view(torch.float16).view(mats, SSQ_DAMP_NHI, d.row_len)

    def free(self):
        if self.handle is not None:
            _check(lib.ssq_free_state(self.handle), "ssq_free_state")
            self.handle = None

    def __del__(self):
        try:
            if self.handle is not None and lib is not None:
                lib.ssq_free_state(self.handle)
                self.handle = None
        except Exception:
            pass


def ssq_alloc_state(desc: ssq_desc, storage: torch.Tensor | None = None, init: torch.Tensor | None = None,
                    stream=None) -> State:
    """Create a state (zero, or ``init`` quantized).  ``storage``: a uint8 CUDA tensor of at least
    ``ssq_state_bytes(desc)`` bytes that outlives the state, or None for library-owned memory."""
    layout = ssq_state_layout(desc)
    sp = None
    if storage is not None:
        if not storage.is_cuda or storage.dtype != torch.uint8 or not storage.is_contiguous():
            raise ValueError("storage must be a contiguous uint8 CUDA tensor")
        if storage.numel() < layout.total_bytes:
            raise ValueError(f"storage has {storage.numel()} bytes, needs {layout.total_bytes}")
        sp = ctypes.c_void_p(storage.data_ptr())
    ip = None
    if init is not None:
        ip = _dev(init, "init", int(layout.rows) * desc.row_len)
    h = ctypes.c_void_p()
    _check(lib.ssq_alloc_state(ctypes.byref(desc), sp, ip, _stream(stream), ctypes.byref(h)), "ssq_alloc_state")
    return State(h, desc, layout, storage)


def ssq_free_state(state: State):
    state.free()


def ssq_state_info(state: State):
    """(desc, storage device pointer, layout) of a state."""
    d, lay, ptr = ssq_desc(), ssq_layout(), ctypes.c_void_p()
    _check(lib.ssq_state_info(state.handle, ctypes.byref(d), ctypes.byref(ptr), ctypes.byref(lay)),
           "ssq_state_info")
    return d, ptr.value, lay


def ssq_set_rounding(state: State, mode: int, seed: int = 0, step: int = 0, stream=None):
    """Round the state's codes to nearest or stochastically (seed; the next token is written to the
    state's counter on ``stream``)."""
    _check(lib.ssq_set_rounding(state.handle, mode, seed, step, _stream(stream)), "ssq_set_rounding")


def ssq_get_rounding(state: State, stream=None):
    """(mode, seed, next token) of a state; the token is read from the device on ``stream``."""
    m, sd, sp = ctypes.c_int32(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib.ssq_get_rounding(state.handle, ctypes.byref(m), ctypes.byref(sd), ctypes.byref(sp), _stream(stream)),
           "ssq_get_rounding")
    return m.value, sd.value, sp.value


def _sizes(state: State, kind: int, *sizes):
    return sizes if state.desc.kind == kind else (None,) * len(sizes)


def ssq_decode_step(state: State, x, dt, A, B, C, D, y, readout: int = SSQ_READ_POST_QUANT, stream=None):
    d = state.desc
    rows, bh, bc, nh = _sizes(state, SSQ_MAMBA2, d.batch * d.nheads * d.rows_per_head, d.batch * d.nheads,
                              d.batch * d.ngroups * d.row_len, d.nheads)
    _check(lib.ssq_decode_step(state.handle, _dev(x, "x", rows), _dev(dt, "dt", bh), _dev(A, "A", nh),
                               _dev(B, "B", bc), _dev(C, "C", bc), _dev(D, "D", nh), _dev(y, "y", rows),
                               readout, _stream(stream)), "ssq_decode_step")


def ssq_scan(state: State, T: int, x, dt, A, B, C, D, y, readout: int = SSQ_READ_POST_QUANT, stream=None):
    d = state.desc
    Tn = max(int(T), 0)
    xs, dts, bcs, nh = _sizes(state, SSQ_MAMBA2, d.batch * d.nheads * d.rows_per_head * Tn,
                              d.batch * Tn * d.nheads, d.batch * Tn * d.ngroups * d.row_len, d.nheads)
    _check(lib.ssq_scan(state.handle, T, _dev(x, "x", xs), _dev(dt, "dt", dts), _dev(A, "A", nh),
                        _dev(B, "B", bcs), _dev(C, "C", bcs), _dev(D, "D", nh), _dev(y, "y", xs),
                        readout, _stream(stream)), "ssq_scan")


def ssq_prefill(state: State, T: int, chunk: int, x, dt, A, B, C, D, y, readout: int = SSQ_READ_POST_QUANT,
                stream=None):
    d = state.desc
    Tn = max(int(T), 0)
    xs, dts, bcs, nh = _sizes(state, SSQ_MAMBA2, d.batch * d.nheads * d.rows_per_head * Tn,
                              d.batch * Tn * d.nheads, d.batch * Tn * d.ngroups * d.row_len, d.nheads)
    _check(lib.ssq_prefill(state.handle, T, chunk, _dev(x, "x", xs), _dev(dt, "dt", dts), _dev(A, "A", nh),
                           _dev(B, "B", bcs), _dev(C, "C", bcs), _dev(D, "D", nh), _dev(y, "y", xs),
                           readout, _stream(stream)), "ssq_prefill")


def ssq_delta_step(state: State, q, k, v, alpha, beta, o, readout: int = SSQ_READ_POST_QUANT, stream=None):
    d = state.desc
    bh = d.batch * d.nheads
    nk, nv, nb = _sizes(state, SSQ_DELTA, bh * d.rows_per_head, bh * d.row_len, bh)
    _check(lib.ssq_delta_step(state.handle, _dev(q, "q", nk), _dev(k, "k", nk), _dev(v, "v", nv),
                              _dev(alpha, "alpha", nb), _dev(beta, "beta", nb), _dev(o, "o", nv), readout,
                              _stream(stream)), "ssq_delta_step")


def ssq_kda_step(state: State, q, k, v, alpha, beta, o, readout: int = SSQ_READ_POST_QUANT, stream=None):
    d = state.desc
    bh = d.batch * d.nheads
    nk, nv, nb = _sizes(state, SSQ_DELTA, bh * d.rows_per_head, bh * d.row_len, bh)
    _check(lib.ssq_kda_step(state.handle, _dev(q, "q", nk), _dev(k, "k", nk), _dev(v, "v", nv),
                            _dev(alpha, "alpha", nk), _dev(beta, "beta", nb), _dev(o, "o", nv), readout,
                            _stream(stream)), "ssq_kda_step")


def ssq_dequant(state: State, out, stream=None):
    _check(lib.ssq_dequant(state.handle, _dev(out, "out", state.rows * state.desc.row_len), _stream(stream)),
           "ssq_dequant")


def ssq_stream_copy(dst, src, nbytes: int | None = None, stream=None):
    """Copy ``nbytes`` (default: all of ``src``) from one CUDA tensor to another with the
    library's streaming copy kernel."""
    for name, t in (("dst", dst), ("src", src)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size() or n > dst.numel() * dst.element_size():
        raise ValueError("nbytes exceeds a tensor")
    _check(lib.ssq_stream_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n, _stream(stream)),
           "ssq_stream_copy")
