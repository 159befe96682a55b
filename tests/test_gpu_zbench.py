"""bench.py end to end on the GPU, on the tiny chain: one JSON line with the
contract's fields, a roofline object, and a CPU baseline whose same-run
parity check passes.  (Named to run after the other GPU tests.)"""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_bench_tiny_chain_line():
    print("[case] bench.py --workload tiny_chain --steps 8 --warmup 2", flush=True)
    r = _run("--workload", "tiny_chain", "--steps", "8", "--warmup", "2")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2
    assert d["config"]["workload"] == "tiny_chain" and d["value"] > 0
    assert d["dtype"] == "f32"
    rf = d["roofline"]
    assert rf["bound"] == "alu" and rf["peak"] > 0 and rf["avg_launch_us"] > 0
    ev = d["call_us_events"]
    assert 0 < ev["p10"] <= ev["median"] <= ev["p90"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["parity"]["ok"] and cb["parity"]["rows"] == 16
