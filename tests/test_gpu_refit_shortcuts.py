"""The refit fast path's shortcuts as the library compiles them, checked exhaustively on the
GPU (tests/csrc/ssq_checks.hip, built by the same hipcc flags from the same device header):

* the step (max - min)/Q or max|h|/Q by one correction step, against IEEE division, for every
  fp32 numerator in the admitted range 2^-100 .. 2^100 and Q = 7, 15, 127, 255;
* the reciprocal 1/s from v_rcp_f32 and one Newton step, against IEEE division, for every
  fp32 s from 2^-110 to 2^100 (every step the admitted ranges produce);
* the reference quotients against the double quotient rounded once;
* two negative controls: each shortcut without its correction is wrong somewhere, so the
  comparisons do see a wrong result.
"""
import ctypes
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "libssq_checks.so")


def test_refit_shortcuts_exhaustive():
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is not built: run __graft_entry__.build()")
    print("refit shortcuts: exhaustive division and reciprocal checks", file=sys.stderr, flush=True)
    lib = ctypes.CDLL(LIB)
    lib.ssq_check_refit_shortcuts.restype = ctypes.c_int
    lib.ssq_check_refit_shortcuts.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    counts = torch.zeros(8, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    assert lib.ssq_check_refit_shortcuts(ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    c = counts.cpu().tolist()
    print(f"refit shortcuts: counts {c}", file=sys.stderr, flush=True)
    assert c[0:4] == [0, 0, 0, 0], "the division shortcut differs from IEEE division"
    assert c[4] == 0, "the reciprocal shortcut differs from IEEE division"
    assert c[5] == 0, "a reference quotient differs from the double quotient rounded once"
    assert c[6] > 0 and c[7] > 0, "a negative control found nothing: the comparison is not effective"
