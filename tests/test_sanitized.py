"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, every report fatal.

- The oracle: ssq_oracle.c is built again with both (float-to-int overflow included) and the
  oracle's pin suites run against that build in a child process.  (A read one past a row
  planted in a copy of the source stops that child run with a heap-buffer-overflow report.)
- The library's host side: ssq_api.cpp (argument checks, layouts, handles, status text) is
  compiled with both for the host only, linked with the kernels' objects, and the ABI's host
  tests run against that build in a child process with the sanitizer runtime preloaded.

Nothing here touches a GPU."""
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


def _hip_objects(tmp_path):
    """The kernels' objects of the library build; compiled into tmp_path if not built yet."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("ssq_libbuild", os.path.join(ROOT, "mamba_decode_amd", "build.py"))
    libbuild = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(libbuild)
    objs = []
    for src in libbuild.SOURCES:
        if src == "ssq_api.cpp":
            continue
        obj = os.path.join(libbuild.BUILD_DIR, src.rsplit(".", 1)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(libbuild.CSRC, src)):
            obj = str(tmp_path / (src + ".o"))
            subprocess.check_call([libbuild.HIPCC, *libbuild.FLAGS, "-c", os.path.join(libbuild.CSRC, src), "-o", obj],
                                  stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        objs.append(obj)
    return libbuild, objs


def test_abi_host_tests_pass_with_the_host_side_sanitized(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded; the sanitizer runtime has to come first")
    rt = subprocess.check_output(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 text=True).strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not found:
            pytest.skip("no clang AddressSanitizer runtime here")
        rt = found[0]
    libbuild, objs = _hip_objects(tmp_path)
    api_obj = str(tmp_path / "ssq_api_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in libbuild.FLAGS if not f.startswith("-O")] + ["-O1", "-g"]
    subprocess.check_call([libbuild.HIPCC, *flags, *host_san, "-c", os.path.join(libbuild.CSRC, "ssq_api.cpp"),
                           "-o", api_obj], stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    so = str(tmp_path / "libssq_san.so")
    # the sanitizer symbols stay undefined in the library and resolve to the preloaded runtime
    subprocess.check_call([libbuild.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_obj, *objs, "-o", so])

    env = dict(os.environ, SSQ_LIBRARY=so, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    probe = "import mamba_decode_amd as m; print(m.LIB_PATH, m.lib._name)"
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == [so, so], r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "--capture=sys", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
