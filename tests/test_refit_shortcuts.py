"""The refit fast path's division shortcut equals IEEE division on every input it admits.

The step kernels refit a row's step as q = a*r, fma(fma(-q, Q, a), r, q) with r = RN(1/Q),
Q = 2^b - 1 (asymmetric grid, a = max - min) or 2^(b-1) - 1 (symmetric grid, a = max |h|),
and take that path only for 2^-100 <= a <= 2^100.  This host test evaluates the same
three operations in C (fmaf, -ffp-contract=off) for every fp32 value of a in that range,
all 2^23 mantissas at each of the 200 binades plus 2^100 itself, for the four constants
Q = 7, 15, 127, 255, against the correctly rounded quotient a/Q of IEEE division.  The
shortcut is the one-correction-step division of Markstein ("IA-64 and elementary
functions", 2000) with a fixed divisor; its correctness over a range has to be checked,
and this is that check.  The compiled device functions are checked again on the GPU
(tests/test_gpu_refit_shortcuts.py).  Host arithmetic only; no GPU.
"""
import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <string.h>

static float from_bits(uint32_t b)
{
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

/* mismatches of fma(fma(-q, Q, a), r, q), q = a*r, r = RN(1/Q), against a/Q, over the
 * fp32 values a = m * 2^e, all 2^23 mantissas, e_lo <= e <= e_hi (normal binades);
 * correct = 0 leaves out the correction step (q alone) */
long long count_div_mismatch(int Q, int e_lo, int e_hi, int correct)
{
    const float qf = (float)Q;
    const float r = 1.0f / qf;
    long long bad = 0;
    int e;
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 1)
    for (e = e_lo; e <= e_hi; ++e) {
        uint32_t m;
        long long local = 0;
        for (m = 0; m < (1u << 23); ++m) {
            const float a = from_bits(((uint32_t)(e + 127) << 23) | m);
            const float q = a * r;
            const float got = correct ? fmaf(fmaf(-q, qf, a), r, q) : q;
            const float ref = a / qf;
            local += got != ref;
        }
        bad += local;
    }
    return bad;
}

long long count_div_mismatch_at(int Q, float a)
{
    const float qf = (float)Q;
    const float r = 1.0f / qf;
    const float q = a * r;
    return fmaf(fmaf(-q, qf, a), r, q) != a / qf;
}
"""


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    import ctypes
    d = tmp_path_factory.mktemp("divconst")
    src = d / "divconst.c"
    src.write_text(SRC)
    so = d / "libdivconst.so"
    cmd = ["gcc", "-O3", "-march=native", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", str(src), "-o", str(so), "-lm"]
    try:
        subprocess.check_call(cmd)
    except subprocess.CalledProcessError:
        cmd.remove("-fopenmp")
        subprocess.check_call(cmd)
    L = ctypes.CDLL(str(so))
    L.count_div_mismatch.restype = ctypes.c_longlong
    L.count_div_mismatch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.count_div_mismatch_at.restype = ctypes.c_longlong
    L.count_div_mismatch_at.argtypes = [ctypes.c_int, ctypes.c_float]
    return L


@pytest.mark.parametrize("Q", [7, 15, 127, 255])
def test_division_shortcut_is_exact_over_the_admitted_range(lib, Q):
    os.environ.setdefault("OMP_NUM_THREADS", str(min(8, os.cpu_count() or 1)))
    # 2^-100 <= a < 2^100: binades -100 .. 99, every mantissa; then 2^100 itself
    assert lib.count_div_mismatch(Q, -100, 99, 1) == 0
    assert lib.count_div_mismatch_at(Q, 2.0 ** 100) == 0


def test_the_check_can_fail(lib):
    """Without its correction step the shortcut is wrong on part of every binade, so the
    comparison above does see a wrong quotient."""
    for Q in (7, 15, 127, 255):
        assert lib.count_div_mismatch(Q, 0, 0, 0) > 0
