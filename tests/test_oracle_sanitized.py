"""The oracle's C under AddressSanitizer and UndefinedBehaviorSanitizer: ssq_oracle.c is built
again with both (float-to-int overflow included, every report fatal) and the oracle's pin
suites run against that build in a child process, which must pass with no report.  Host
only; nothing here touches a GPU.  (A read one past a row planted in a copy of the source
stops that child run with a heap-buffer-overflow report.)"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_SUITES = ["test_oracle_pins.py", "test_oracle_sr.py", "test_oracle_kda.py", "test_oracle_prefill.py",
              "test_oracle_damp.py"]
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
             "-fno-sanitize-recover=all"]


def test_pin_suites_pass_under_asan_and_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded; the sanitizer runtime has to come first")
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    so = str(tmp_path / "liboracle_san.so")
    flags = [f for f in oracle.CFLAGS if not f.startswith("-O")] + SAN_FLAGS
    subprocess.check_call(["gcc", *flags, oracle._SRC, "-o", so, "-lm"])

    env = dict(os.environ, SSQ_ORACLE_LIB=so, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    probe = ("import ctypes, oracle; L = oracle.lib(); "
             "print(L._name, hasattr(L, '__asan_init'), hasattr(L, '__ubsan_handle_float_cast_overflow_abort'))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == [so, "True", "True"], r.stdout  # the instrumented build is the one loaded

    # --capture=sys: a sanitizer report written to fd 2 reaches this process
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "--capture=sys", *[os.path.join(ROOT, "tests", f) for f in PIN_SUITES]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
