"""Host logic of bench.py that runs without a GPU: the CPU-baseline sample
and the parity check of the same run (the oracle's sampled rows against a
given output).  The "GPU output" here is the oracle's own full result, as
stored by the device (f32, or rounded to f16 for the quantized path), so the
check must pass; a planted error in one element must fail it."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
from tree_masked_decode_amd import inputs  # noqa: E402


def _fp_full(c):
    mask = oracle.tree_mask(c["parents"], c["kv_seq_len"], c["mask_stride"])
    full = oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=c["n_kv_heads"],
                            kv_seq_len=c["kv_seq_len"], scale=c["scale"])
    return full.reshape(-1, full.shape[-1])


def _quant_full(c):
    full = oracle.quant_attention(
        c["q"], c["k_packed"], c["k_scales"], c["k_biases"], c["v_packed"], c["v_scales"],
        c["v_biases"], n_kv_heads=c["n_kv_heads"], kv_seq_len=c["kv_seq_len"], bits=c["bits"],
        group_size=c["group_size"], scale=c["scale"], sinks=c["sinks"],
        mask=np.ascontiguousarray(c["mask"]).ravel(), mask_head_stride=c["mask_head_stride"],
        mask_stride=c["mask_stride"])
    return full.reshape(-1, full.shape[-1])


def test_baseline_parity_fp32():
    c = inputs.fp_case("tiny_chain")
    got = _fp_full(c).astype(np.float32)
    r = bench.cpu_baseline("tiny_chain", c, bench.fp_alg(c), False, gpu_out=got, tol=1e-4)
    assert r["parity"]["ok"] and r["parity"]["rows"] == 16
    assert r["cores"] >= 1 and r["kind"] == "oracle" and r["value"] > 0
    # cores = the threads the oracle used; the host's own count beside it
    import os
    assert r["host_cores"] == len(os.sched_getaffinity(0))
    assert r["threads"] == r["cores"] == min(16, r["host_cores"])
    bad = got.copy()
    bad[5, 17] += 2e-4
    r = bench.cpu_baseline("tiny_chain", c, bench.fp_alg(c), False, gpu_out=bad, tol=1e-4)
    assert not r["parity"]["ok"]


def test_baseline_parity_quant_f16_half_ulp():
    # a short quantized problem of the 4-bit workload's shape family
    c = inputs.quant_case("quant_4bit", batch=1, kv_seq_len=256, kv_capacity=256)
    ref = _quant_full(c)
    got = ref.astype(np.float16).astype(np.float64)   # the contract's f16 rounding
    alg = bench.quant_alg(c)
    r = bench.cpu_baseline("quant_4bit", c, alg, True, gpu_out=got, tol=2e-3, out_elem="f16")
    assert r["parity"]["ok"], r["parity"]
    bad = got.copy()
    bad[3, 9] += 5e-3
    r = bench.cpu_baseline("quant_4bit", c, alg, True, gpu_out=bad, tol=2e-3, out_elem="f16")
    assert not r["parity"]["ok"]


@pytest.mark.parametrize("target,expect_all", [(1e-9, False), (1e9, True)])
def test_baseline_sample_size(monkeypatch, target, expect_all):
    # the pilot sizes the measured sample: a tiny target keeps the pilot's
    # rows, a huge one takes every row of the call
    c = inputs.fp_case("tiny_chain", q_l=4)
    monkeypatch.setattr(bench, "CPU_SAMPLE_S", target)
    monkeypatch.setattr(bench.os, "sched_getaffinity", lambda pid: {0, 1})
    r = bench.cpu_baseline("tiny_chain", c, bench.fp_alg(c), False)
    n = int(r["sample"].split(" of ")[0])
    total = c["n_heads"] * c["q_l"]
    if expect_all:
        assert n == total
    else:
        assert n == min(total, 4)
    assert r["parity"] is None


def test_bench_refuses_several_gpus():
    # one GPU only: the refusal comes before anything touches a device
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_traffic_record_only_for_the_source_it_was_taken_on(monkeypatch):
    # a committed HBM-traffic record is reported while the forward kernel's
    # sources hash to its key, and dropped (None) once they differ
    import json
    w = "dynamic_tree_32k"
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_%s.json" % w)))
    monkeypatch.setattr(bench, "source_sha", lambda files: rec["source_sha"])
    assert bench.measured_traffic(w, "f16") == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_sha", lambda files: "0" * 16)
    assert bench.measured_traffic(w, "f16") is None
    assert bench.measured_traffic("no_such_workload", "f16") is None
