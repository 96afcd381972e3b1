"""Build ``tests/csrc/libssq_checks.so``: GPU check kernels over the library's device code
(test support, not part of the library).  Uses the library's own hipcc flags."""
from __future__ import annotations

import importlib.util
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libssq_checks.so")


def build() -> str:
    spec = importlib.util.spec_from_file_location("ssq_hip_build", os.path.join(ROOT, "mamba_decode_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    tmp = LIB + ".tmp"
    p = subprocess.run([mod.HIPCC, *mod.FLAGS, "-shared", os.path.join(HERE, "ssq_checks.hip"), "-o", tmp],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        # the host pass does not know the gfx950 feature name: that warning is harmless
        print("\n".join(ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln))
        raise RuntimeError("hipcc failed for ssq_checks.hip")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
