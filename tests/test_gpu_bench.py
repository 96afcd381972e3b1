"""GPU: bench.py end to end on a few layers of three workloads (decode, delta rule, scan), its one
JSON line checked for the fields and units the measurement contract names."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("workload,bound,limited", [("m2_370m_int4", "hbm", "valu_issue"),
                                                    ("delta_int8", "hbm", "valu_issue"),
                                                    ("m2_8b_int8sym", "hbm", "hbm"),
                                                    ("m2_130m_scan_int8asym", "alu", "valu_issue_on_chip")])
def test_bench_json_line(workload, bound, limited):
    print(f"bench {workload}", file=sys.stderr, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, "--layers", "2",
                        "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["unit"] == "GB/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["layers"] == 2 and d["config"]["layers_reduced_from"] > 2
    rf = d["roofline"]
    assert rf["bound"] == bound and rf["peak"] > 0 and 0 < rf["frac"] < 1.5
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["unit"] == ("GB/s" if bound == "hbm" else "T lane-ops/s")
    assert rf["limited_by"] == limited and rf["limited_by_evidence"]
    assert d["copy_GBps"] > 1000 and "cpu_baseline" not in d
