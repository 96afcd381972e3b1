"""The C ABI on the host: exported symbols, state sizing and layout, argument
validation and error reporting.  No kernel is launched (no GPU needed)."""
import ctypes
import json
import os
import re

import pytest

import mamba_decode_amd as ssq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(ssq.lib, n), n  # ctypes resolves the exported symbol


def test_binding_covers_every_declared_function():
    for n in declared_functions():
        assert callable(getattr(ssq, n, None)), n


def desc(kind=ssq.SSQ_MAMBA2, fmt="int8_asym", batch=2, nheads=4, P=64, N=128, ngroups=1):
    return ssq.make_desc(kind, fmt, batch, nheads, P, N, ngroups)


@pytest.mark.parametrize("fmt,row_bytes", [("fp32", 512), ("int8_sym", 128), ("int8_asym", 128),
                                           ("int4_sym", 64), ("int4_asym", 64)])
def test_layout(fmt, row_bytes):
    d = desc(fmt=fmt, batch=3, nheads=5, P=48)
    lay = ssq.ssq_state_layout(d)
    rows = 3 * 5 * 48
    assert lay.rows == rows and lay.row_bytes == row_bytes and lay.codes_offset == 0
    for off in (lay.codes_offset, lay.scale_offset, lay.zero_offset, lay.counter_offset, lay.total_bytes):
        assert off % 256 == 0
    if fmt == "fp32":
        assert lay.scale_offset == 0 and lay.zero_offset == 0 and lay.counter_offset == 0
        assert lay.total_bytes >= rows * 512
    else:
        assert lay.scale_offset >= rows * row_bytes
        if fmt.endswith("asym"):
            assert lay.zero_offset >= lay.scale_offset + 4 * rows
            assert lay.counter_offset >= lay.zero_offset + 4 * rows
        else:
            assert lay.zero_offset == 0 and lay.counter_offset >= lay.scale_offset + 4 * rows
        # the stochastic-rounding token counter (8 bytes)
        assert lay.total_bytes >= lay.counter_offset + 8
    assert ssq.ssq_state_bytes(d) == lay.total_bytes
    payload = rows * row_bytes + (0 if fmt == "fp32" else 4 * rows * (2 if "asym" in fmt else 1) + 8)
    assert lay.total_bytes - payload < 4 * 256


def test_state_sizes_match_the_pages():
    """15 GB of fp32 state for 30 delta-rule layers at batch 256, ~60 MB per request,
    ~1.9 GB at batch 32 and ~5.6 GB at batch 96 (golden fixture, cited in the file)."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "state_sizes.json")))
    for batch, gb in g["fp32_state_GB"].items():
        d = ssq.make_desc(ssq.SSQ_DELTA, "fp32", int(batch), g["heads"], g["dk"], g["dv"])
        total = g["layers"] * ssq.ssq_state_bytes(d)
        assert round(total / 2 ** 30, 1) == pytest.approx(gb, abs=1e-9)
    d = ssq.make_desc(ssq.SSQ_DELTA, "fp32", 256, g["heads"], g["dk"], g["dv"])
    assert g["layers"] * ssq.ssq_state_bytes(d) == 15 * 2 ** 30
    assert round(g["layers"] * ssq.ssq_state_bytes(d) / 256 / 2 ** 20) == g["per_request_MB_at_256"]


def test_quantized_footprints():
    # int4 asym Mamba-2 370m-shaped layer at batch 256: 524288 rows x (64 B codes + 8 B metadata),
    # plus the 256-byte region of the stochastic-rounding token counter
    d = ssq.make_desc(ssq.SSQ_MAMBA2, "int4_asym", 256, 32, 64)
    assert ssq.ssq_state_bytes(d) == 524288 * 72 + 256
    # int8 asym delta layer: 136 of 512 bytes per fp32 row
    d8 = ssq.make_desc(ssq.SSQ_DELTA, "int8_asym", 256, 32, 128)
    d32 = ssq.make_desc(ssq.SSQ_DELTA, "fp32", 256, 32, 128)
    assert (ssq.ssq_state_bytes(d8) - 256) * 512 == ssq.ssq_state_bytes(d32) * 136


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), ssq.SSQ_ERR_INVALID_ARG),
    (dict(nheads=-1), ssq.SSQ_ERR_INVALID_ARG),
    (dict(P=0), ssq.SSQ_ERR_INVALID_ARG),
    (dict(nheads=6, ngroups=4), ssq.SSQ_ERR_INVALID_ARG),
    (dict(N=64), ssq.SSQ_ERR_UNSUPPORTED),
    (dict(N=127), ssq.SSQ_ERR_UNSUPPORTED),
    (dict(P=24), ssq.SSQ_ERR_UNSUPPORTED),
    (dict(kind=ssq.SSQ_DELTA, P=64), ssq.SSQ_ERR_UNSUPPORTED),
    (dict(kind=ssq.SSQ_DELTA, P=128, ngroups=2), ssq.SSQ_ERR_INVALID_ARG),
    (dict(kind=7), ssq.SSQ_ERR_INVALID_ARG),
    (dict(fmt=9), ssq.SSQ_ERR_INVALID_ARG),
])
def test_invalid_descriptions_are_rejected(kw, status):
    d = desc(**kw)
    assert ssq.ssq_state_bytes(d) == 0
    lay = ssq.ssq_layout()
    assert ssq.lib.ssq_state_layout(ctypes.byref(d), ctypes.byref(lay)) == status
    assert ssq.ssq_last_error() != ""
    h = ctypes.c_void_p()
    assert ssq.lib.ssq_alloc_state(ctypes.byref(d), None, None, None, ctypes.byref(h)) == status
    assert h.value is None


def test_null_arguments_are_rejected_before_any_device_call():
    L = ssq.lib
    assert L.ssq_state_bytes(None) == 0
    assert L.ssq_state_layout(None, None) == ssq.SSQ_ERR_INVALID_ARG
    d = desc()
    assert L.ssq_alloc_state(ctypes.byref(d), None, None, None, None) == ssq.SSQ_ERR_INVALID_ARG
    # misaligned caller storage
    h = ctypes.c_void_p()
    assert L.ssq_alloc_state(ctypes.byref(d), ctypes.c_void_p(0x1000 + 16), None, None, ctypes.byref(h)) \
        == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_decode_step(None, None, None, None, None, None, None, None, 0, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_scan(None, 4, None, None, None, None, None, None, None, 0, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_prefill(None, 4, 2, None, None, None, None, None, None, None, 0, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_delta_step(None, None, None, None, None, None, None, 0, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_kda_step(None, None, None, None, None, None, None, 0, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_dequant(None, None, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_state_info(None, None, None, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_set_rounding(None, ssq.SSQ_ROUND_STOCHASTIC, 1, 0, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_get_rounding(None, None, None, None, None) == ssq.SSQ_ERR_INVALID_ARG
    assert L.ssq_free_state(None) == ssq.SSQ_OK


def test_forced_allocation_failure(monkeypatch):
    monkeypatch.setenv("SSQ_TEST_FAIL_ALLOC", "1")
    d = desc()
    h = ctypes.c_void_p()
    assert ssq.lib.ssq_alloc_state(ctypes.byref(d), None, None, None, ctypes.byref(h)) == ssq.SSQ_ERR_ALLOC
    assert "SSQ_TEST_FAIL_ALLOC" in ssq.ssq_last_error()
    assert h.value is None


def test_status_strings():
    for s in range(6):
        assert ssq.ssq_status_string(s).startswith("SSQ_")
    assert "unknown" in ssq.ssq_status_string(42)


def test_two_tier_layout():
    """SSQ_DAMP: uint8 rows (codes, scale, zero) for key rows 16..127 of each matrix, half rows
    for 0..15, 9.44 bits per value; a delta-rule format only."""
    d = ssq.make_desc(ssq.SSQ_DELTA, "damp", 3, 5, 128, 128)
    lay = ssq.ssq_state_layout(d)
    mats = 15
    lo = mats * 112
    assert lay.rows == mats * 128 and lay.row_bytes == 128
    assert lay.scale_offset >= lo * 128 and lay.zero_offset >= lay.scale_offset + 4 * lo
    assert lay.hi_offset >= lay.zero_offset + 4 * lo
    assert lay.counter_offset >= lay.hi_offset + mats * 16 * 128 * 2
    assert lay.total_bytes >= lay.counter_offset + 8
    for off in (lay.scale_offset, lay.zero_offset, lay.hi_offset, lay.counter_offset, lay.total_bytes):
        assert off % 256 == 0
    payload = lo * (128 + 8) + mats * 16 * 256
    assert lay.total_bytes - payload < 5 * 256
    assert payload * 8 / (mats * 128 * 128) == pytest.approx(9.4375)
    bad = ssq.make_desc(ssq.SSQ_MAMBA2, "damp", 1, 2, 64)
    h = ctypes.c_void_p()
    assert ssq.lib.ssq_alloc_state(ctypes.byref(bad), None, None, None, ctypes.byref(h)) == ssq.SSQ_ERR_UNSUPPORTED


def test_stream_copy_validates_before_launch():
    """Rejected copies return INVALID_ARG from the argument checks alone (no device work)."""
    import mamba_decode_amd as ssq
    vp = ctypes.c_void_p
    cases = [
        (None, vp(4096), 64),            # NULL dst
        (vp(4096), None, 64),            # NULL src
        (vp(4096 + 8), vp(1 << 20), 64),  # misaligned dst
        (vp(4096), vp(1 << 20), 40),     # not a multiple of 16
        (vp(4096), vp(4096 + 32), 64),   # overlapping
        (vp(4096 + 32), vp(4096), 64),   # overlapping the other way
    ]
    for dst, src, n in cases:
        assert ssq.lib.ssq_stream_copy(dst, src, n, None) == ssq.SSQ_ERR_INVALID_ARG, (dst, src, n)
        assert ssq.ssq_last_error()
