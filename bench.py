#!/usr/bin/env python3
"""Benchmark of one tree-verify call (forward + log-sum-exp merge) on MI355X.

Default workload: the 32K-context dynamic-tree verify (n_heads=24,
n_kv_heads=4, head_dim=256, kv_seq_len=32768, kv_capacity=40960, q_l=64
random-tree nodes, fp16 K/V).  A step is one full verify call over one set
of inputs already resident in HBM; the timed steps rotate over identical
input copies totalling >= 1 GiB so that each call reads its K/V from HBM,
not from the 256 MB Infinity Cache (a warm, cache-resident figure is
reported separately).

Prints ONE JSON line.  value = effective HBM throughput of the whole call:
algorithmic bytes (K/V rows below kv_seq_len, Q, the mask once, the
output) / time per call.  roofline = the forward kernel's achieved rate,
timed with HIP events on its own stream, against the MI355X peak of the
unit that bounds it.  cpu_baseline = the CPU oracle timed on a sample of the
same workload on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per tree-verify call + effective HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0     # dense fp16 matrix
VALU_F32_PEAK_TFS = 157.3      # fp32 vector
ROTATE_BYTES = 1 << 30
EV_EVERY = 4                   # timed calls bracketed by HIP events: every 4th


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="dynamic_tree_32k")
    p.add_argument("--nwg", type=int, default=0, help="0 = library's pick")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain copy of known size (for PMC byte scaling)")
    p.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) "
                        "of a --copy-calibration run into profiles/traffic_<workload>.json "
                        "and exit")
    return p.parse_args()


# --------------------------------------------------------------------------
# algorithmic sizes
# --------------------------------------------------------------------------
def fp_alg(c):
    H, Hk, D = c["n_heads"], c["n_kv_heads"], c["head_dim"]
    L, q_l = c["kv_seq_len"], c["q_l"]
    esz = 2 if c["kv_dtype"] == "f16" else 4
    ws = c.get("window_start")
    mask = q_l * L * 4
    if ws is not None:   # decode: no mask buffer, keys from window_start on
        L -= ws
        mask = 0
    mws = c.get("mask_window_start")
    if mws:              # window as a mask: the mask is read whole, keys from mws on
        L -= mws
    kv = 2 * Hk * L * D * esz
    qb = H * q_l * D * 4
    out = q_l * H * D * 4
    flops = 4 * (q_l * H) * L * D
    return dict(bytes=kv + qb + mask + out, kv_bytes=kv, flops=flops)


def quant_alg(c):
    B, nQ, nKV, dim = c["batch"], c["n_q_heads"], c["n_kv_heads"], c["dim"]
    L, q_l, bits, G = c["kv_seq_len"], c["q_l"], c["bits"], c["group_size"]
    W = c.get("window_size", 0)
    if W:
        L = min(W, L)   # a sliding window reads only its last W tokens
    packed = 2 * B * nKV * L * dim * bits // 8
    sb = 4 * B * nKV * L * (dim // G) * 2
    esz = 4 if c.get("elem") == "f32" else 2   # bytes of a Q / scale / bias / out element
    sb = sb * esz // 2
    qb = B * nQ * q_l * dim * esz
    mask = 0 if c["mask"] is None else B * nQ * q_l * L * esz
    if c.get("mask_bool") is not None:
        mask = B * nQ * q_l * L * 4
    sinks = 0 if c["sinks"] is None else nQ * 4
    out = B * nQ * q_l * dim * esz
    flops = 4 * (B * nQ * q_l) * L * dim
    return dict(bytes=packed + sb + qb + mask + sinks + out, kv_bytes=packed + sb,
                flops=flops)


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


# (the split planner in abi.hip sets the partial-result bytes, so it keys
# the record too)
FWD_SOURCES = {"f16": ["tree_masked_decode_amd/csrc/fwd_f16.hip",
                       "tree_masked_decode_amd/csrc/fwd_wide.hip",
                       "tree_masked_decode_amd/csrc/fwd_wide_loop.inc",
                       "tree_masked_decode_amd/csrc/common.h",
                       "tree_masked_decode_amd/csrc/abi.hip"],
               "f32": ["tree_masked_decode_amd/csrc/fwd_f32.hip",
                       "tree_masked_decode_amd/csrc/common.h",
                       "tree_masked_decode_amd/csrc/abi.hip"],
               "quant": ["tree_masked_decode_amd/csrc/quant.hip",
                         "tree_masked_decode_amd/csrc/quant_impl.h",
                         "tree_masked_decode_amd/csrc/common.h",
                         "tree_masked_decode_amd/csrc/abi.hip"]}


def measured_traffic(workload, kind):
    """HBM bytes per forward launch from the committed PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(FWD_SOURCES[kind]):
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 256 << 20     # the --copy-calibration copy: reads and writes this much
CALIB_COPIES = 5           # ... this many times, right before the warm-up calls


def record_traffic(workload, fetch_csv, write_csv):
    """HBM bytes per forward launch from two rocprofv3 --pmc runs.

    FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by
    COPY_BYTES / (what the same counter reads for the calibration copy), so
    that a plain copy of known size counts exactly its size.  The forward
    kernel is the dispatch whose name holds "fwd_" or "quant_kernel"; its
    dispatches are averaged."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        return acc

    def is_copy(k):
        return "copy" in k.lower() or "elementwise" in k.lower()

    def is_fwd(k):
        return "fwd_" in k or "quant_kernel" in k

    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        acc = per_kernel(path, name)
        fwd_ids = [d for (k, d) in acc if is_fwd(k)]
        if not fwd_ids:
            raise SystemExit("record-traffic: no forward dispatches in %s" % path)
        first = min(fwd_ids)
        # the calibration copies are the CALIB_COPIES copy dispatches right
        # before the first forward (the input rotation copies come earlier
        # and can be larger)
        copies = sorted((d, v) for (k, d), v in acc.items() if is_copy(k) and d < first)
        copy = [v for _, v in copies[-CALIB_COPIES:]]
        fwd = [v for (k, _), v in acc.items() if is_fwd(k)]
        if len(copy) < CALIB_COPIES:
            raise SystemExit("record-traffic: no calibration copies in %s" % path)
        copy_kib = statistics.median(copy)
        scale = COPY_BYTES / (copy_kib * 1024.0)
        out[name] = {"kib_per_launch": statistics.fmean(fwd), "copy_kib": copy_kib,
                     "scale": scale, "dispatches": len(fwd)}
    from tree_masked_decode_amd import inputs
    kind = ("quant" if workload in inputs.QUANT_WORKLOADS
            else inputs.WORKLOADS[workload]["kv_dtype"])
    total = sum(v["kib_per_launch"] * 1024.0 * v["scale"] for v in out.values())
    rec = {"workload": workload, "kernel": "forward", "bytes_per_launch": round(total),
           "counters": out, "source_sha": source_sha(FWD_SOURCES[kind])}
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# --------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of rows
# --------------------------------------------------------------------------
CPU_SAMPLE_S = 12.0   # target wall time of the measured oracle sample


def cpu_baseline(name, c, alg, quant, gpu_out=None, tol=None, out_elem=None):
    """A pilot over a few rows sizes the sample; the measured run then takes
    evenly spaced rows for about CPU_SAMPLE_S seconds (all rows if fewer).
    With gpu_out (the GPU result of the same inputs, [rows, D]) the sampled
    rows are also compared with it: max-abs error against tol, plus half an
    ulp of the output type for fp16 / bf16 outputs."""
    import oracle
    import numpy as np
    # the host's cores available to this process; the oracle runs on at most
    # 16 of them (one GPU's share of the host)
    host_cores = len(os.sched_getaffinity(0))
    threads = max(1, min(16, host_cores))
    if quant:
        nrows = c["q"].shape[0] * c["q"].shape[1]
        to_row = lambda r: (r // c["q_l"], r % c["q_l"])
        mask = None if c["mask"] is None else np.ascontiguousarray(c["mask"]).ravel()
        mb = c.get("mask_bool")
        mb = None if mb is None else np.ascontiguousarray(mb).ravel()

        def run(rows):
            return oracle.quant_attention(c["q"], c["k_packed"], c["k_scales"], c["k_biases"],
                                   c["v_packed"], c["v_scales"], c["v_biases"],
                                   n_kv_heads=c["n_kv_heads"], kv_seq_len=c["kv_seq_len"],
                                   bits=c["bits"], group_size=c["group_size"],
                                   scale=c["scale"], sinks=c["sinks"], mask=mask,
                                   mask_bool=mb, mask_head_stride=c["mask_head_stride"],
                                   mask_stride=c["mask_stride"],
                                   window_size=c.get("window_size", 0),
                                   elem=c.get("elem", "f16"), rows=rows, nthreads=threads)
    else:
        H = c["n_heads"]
        nrows = H * c["q_l"]
        to_row = lambda r: (r // H, r % H)
        ws = c.get("window_start")
        mask = (None if ws is not None else
                oracle.tree_mask(c["parents"], c["kv_seq_len"], c["mask_stride"]))
        if c.get("mask_window_start"):
            mask[:, :c["mask_window_start"]] = -65504.0

        def run(rows):
            return oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=c["n_kv_heads"],
                             kv_seq_len=c["kv_seq_len"], scale=c["scale"],
                             window_start=ws or 0, rows=rows, nthreads=threads)

    def sample(n):
        step = max(1, nrows // max(1, n))
        return list(range(0, nrows, step))[:max(1, n)]

    flat = sample(min(nrows, 2 * threads))
    t = time.perf_counter()
    ref = run([to_row(r) for r in flat])
    dt = time.perf_counter() - t
    if dt < CPU_SAMPLE_S and len(flat) < nrows:
        n = min(nrows, max(len(flat) + 1, int(len(flat) * CPU_SAMPLE_S / max(dt, 1e-3))))
        flat = sample(n)
        t = time.perf_counter()
        ref = run([to_row(r) for r in flat])
        dt = time.perf_counter() - t
    rows = flat
    parity = None
    if gpu_out is not None:
        got = np.asarray(gpu_out, dtype=np.float64)[flat]
        ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
        diff = np.abs(got - ref)
        bound = np.full(ref.shape, float(tol))
        if out_elem == "f16":
            bound += 0.5 * np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        elif out_elem == "bf16":
            a = np.abs(ref).astype(np.float32)
            e = ((a.view(np.uint32) >> np.uint32(23)) & np.uint32(0xff)).astype(np.int64)
            bound += 0.5 * np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)
        parity = {"rows": len(flat), "max_abs_err": float(diff.max()), "tol": float(tol),
                  "ok": bool(np.all(np.isfinite(got)) and np.all(diff <= bound))}
    us_call = dt * 1e6 * nrows / len(rows)
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for l in f:
                k, _, v = l.partition(":")
                k = k.strip()
                if k in ("model name", "cpu family", "model", "stepping") and k not in info:
                    info[k] = v.strip()
                if not l.strip() and info:
                    break
    except OSError:
        pass
    model = None
    if info:
        model = "%s (family %s, model %s, stepping %s)" % (
            info.get("model name", "?"), info.get("cpu family", "?"), info.get("model", "?"),
            info.get("stepping", "?"))
    return {"value": round(alg["bytes"] / (us_call * 1e-6) / 1e9, 4), "unit": "GB/s",
            "cores": threads, "threads": threads, "host_cores": host_cores,
            "cpu_model": model, "kind": "oracle",
            "sample": "%d of %d output rows of %s (each row over all %d keys), "
                      "%.2f s wall; scaled to the whole call"
                      % (len(rows), nrows, name, c["kv_seq_len"], dt),
            "us_per_call": round(us_call, 1), "parity": parity}


# --------------------------------------------------------------------------
def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py: measures one GPU only; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_masked_decode_amd as ta
    from tree_masked_decode_amd import _lib, inputs

    lib = _lib.load()
    torch.cuda.set_device(0)
    quant = args.workload in inputs.QUANT_WORKLOADS
    if quant:
        c = inputs.quant_case(args.workload)
        alg = quant_alg(c)
        kind = "quant"
    else:
        c = inputs.fp_case(args.workload)
        alg = fp_alg(c)
        kind = c["kv_dtype"]

    # ---- device inputs, rotated over copies totalling >= 1 GiB ----
    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    ncopies = max(1, min(64, math.ceil(ROTATE_BYTES / alg["bytes"])))
    if quant:
        names = ("q", "k_packed", "k_scales", "k_biases", "v_packed", "v_scales", "v_biases")
        elem_t = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[
            c.get("elem", "f16")]
        q_dtype = {"f16": 1, "bf16": 2, "f32": 0}[c.get("elem", "f16")]

        def to_dev_e(a):   # bf16 arrays hold bit patterns (uint16)
            t = to_dev(a)
            return t.view(torch.bfloat16) if c.get("elem") == "bf16" else t
        base = {n: (to_dev if n == "k_packed" or n == "v_packed" else to_dev_e)(c[n])
                for n in names}
        base["sinks"] = None if c["sinks"] is None else to_dev(c["sinks"])
        base["mask"] = (None if c["mask"] is None else
                        to_dev_e(np.ascontiguousarray(c["mask"]).ravel()))
        mask_kind = 0 if c["mask"] is None else 1
        if c.get("mask_bool") is not None:
            base["mask"] = to_dev(np.ascontiguousarray(c["mask_bool"]).ravel().view(np.int32))
            mask_kind = 2
        window = c.get("window_size", 0)
        B, nQ, nKV, dim = c["batch"], c["n_q_heads"], c["n_kv_heads"], c["dim"]
        L, q_l = c["kv_seq_len"], c["q_l"]
        span = min(window, L) if window else L
        nwg = args.nwg or ta.quant_pick_nwg(B, nQ, nKV, dim, span, q_l, bits=c["bits"],
                                            group_size=c["group_size"],
                                            mask_kind=mask_kind, q_dtype=q_dtype)
        nrows, D = B * nQ * q_l, dim
        out_dtype = elem_t
    else:
        base = {"q": to_dev(c["q"]), "k": to_dev(c["k"]), "v": to_dev(c["v"])}
        ws = c.get("window_start")
        base["mask"] = (None if ws is not None else
                        ta.build_tree_mask(c["parents"], c["kv_seq_len"], c["mask_stride"]))
        if c.get("mask_window_start"):
            base["mask"][:, :c["mask_window_start"]] = ta.MASKED
        H, Hk, D = c["n_heads"], c["n_kv_heads"], c["head_dim"]
        L, q_l = c["kv_seq_len"], c["q_l"]
        nwg = args.nwg or c.get("nwg") or ta.pick_nwg(H, Hk, D, L - (ws or 0), q_l,
                                                       1 if kind == "f16" else 0)
        nrows = H * q_l
        out_dtype = torch.float32
    copies = [base] + [{n: (None if t is None else t.clone()) for n, t in base.items()}
                       for _ in range(ncopies - 1)]
    # (plus the tail tree_attn_forward may use for the live-key scan of a mask)
    part = torch.empty(max(1, (ta.partials_bytes(nrows, D, 1, nwg) + ta.RANGE_BYTES) // 4),
                       dtype=torch.float32, device="cuda")
    out = torch.empty((nrows, D), dtype=out_dtype, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    # Pre-marshalled C calls (keeps host launch cost far below the GPU time).
    import ctypes
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    nb = lambda t: 0 if t is None else t.numel() * t.element_size()
    P = part if nwg > 1 else None
    O = out if nwg == 1 else None
    calls = []
    for cp in copies:
        if quant:
            kvb = (ctypes.c_size_t * 6)(*[nb(cp[n]) for n in names[1:]])
            head = (vp(cp["q"]), q_dtype, nb(cp["q"]), vp(cp["k_packed"]), vp(cp["k_scales"]),
                    vp(cp["k_biases"]), vp(cp["v_packed"]), vp(cp["v_scales"]),
                    vp(cp["v_biases"]), kvb, vp(cp["sinks"]), nb(cp["sinks"]),
                    vp(cp["mask"]))
            tail = (vp(P), nb(P), vp(O), nb(O), B, nQ, nKV, dim, L, c["kv_capacity"],
                    q_l, c["bits"], c["group_size"], c["scale"], nwg,
                    ctypes.c_void_p(sptr))
            if mask_kind == 2 or window:
                fargs = head + (mask_kind, nb(cp["mask"]), c["mask_head_stride"],
                                c["mask_stride"], window) + tail
                calls.append((lib.tree_attn_quant_forward_ex, fargs))
            else:
                fargs = head + (nb(cp["mask"]), c["mask_head_stride"],
                                c["mask_stride"]) + tail
                calls.append((lib.tree_attn_quant_forward, fargs))
        elif ws is not None:
            fargs = (vp(cp["q"]), nb(cp["q"]), vp(cp["k"]), vp(cp["v"]),
                     1 if kind == "f16" else 0, nb(cp["k"]), vp(P), nb(P), vp(O), nb(O),
                     H, Hk, D, L, c["kv_capacity"], q_l, ws, c["scale"], nwg,
                     ctypes.c_void_p(sptr))
            calls.append((lib.tree_attn_decode, fargs))
        else:
            fargs = (vp(cp["q"]), nb(cp["q"]), vp(cp["k"]), vp(cp["v"]),
                     1 if kind == "f16" else 0, nb(cp["k"]), vp(cp["mask"]), nb(cp["mask"]),
                     vp(P), nb(P), vp(O), nb(O), H, Hk, D, L, c["kv_capacity"], q_l,
                     c["mask_stride"], c["scale"], nwg, ctypes.c_void_p(sptr))
            calls.append((lib.tree_attn_forward, fargs))
    rargs = (vp(part), nb(part), vp(out),
             {torch.float16: 1, torch.bfloat16: 2}.get(out_dtype, 0),
             nb(out), nrows, D, nwg, ctypes.c_void_p(sptr))

    def step(i, ev=None):
        fn, fa = calls[i % len(calls)]
        if ev is not None:
            ev[0].record(stream)
        rc = fn(*fa)
        if ev is not None:
            ev[1].record(stream)
        if rc != 0:
            raise RuntimeError("forward failed: %s" % _lib.last_error())
        if nwg > 1:
            rc = lib.tree_attn_reduce(*rargs)
            if rc != 0:
                raise RuntimeError("reduce failed: %s" % _lib.last_error())
        if ev is not None:
            ev[2].record(stream)

    if args.copy_calibration:
        # a plain device copy of known size, for scaling the PMC byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(CALIB_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy calibration: 5 copies of %d bytes" % src.numel(), file=sys.stderr)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print("warmup done: %d steps, nwg=%d, %d input copies" % (args.warmup, nwg, ncopies),
          file=sys.stderr, flush=True)

    # ---- timed region (cold: rotating copies) ----
    K = args.steps
    # HIP events bracket every EV_EVERY-th call (forward, and forward + merge):
    # recording them on every call costs enough host time to make calls of a
    # few tens of µs host-bound
    evs = {i: tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for i in range(0, K, EV_EVERY)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs.values()]
    call_ms = [e[0].elapsed_time(e[2]) for e in evs.values()]
    fwd_avg_ms = statistics.fmean(fwd_ms)

    def spread(ms):
        q = np.percentile(np.asarray(ms) * 1e3, [50, 10, 90])
        return {"median": round(float(q[0]), 2), "p10": round(float(q[1]), 2),
                "p90": round(float(q[2]), 2)}
    print("timed: %d steps, %.3f ms/step" % (K, ms_step), file=sys.stderr, flush=True)

    # ---- warm: one input set, back to back (cache-resident) ----
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    for _ in range(K):
        step(0)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - tw0) * 1e3 / K

    # ---- context: what HIP events read around a kernel that does nothing ----
    # (a one-element fill on the same stream, recorded like the forward): the
    # part of avg_launch_us that is launch and event overhead rather than the
    # forward's own run, which matters for kernels of a few tens of µs
    tiny = torch.empty(1, dtype=torch.float32, device="cuda")
    floor = []
    for i in range(40):
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        tiny.fill_(float(i))
        b_ev.record(stream)
        floor.append((a_ev, b_ev))
    torch.cuda.synchronize()
    event_floor_us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in floor[5:])

    # ---- context: streaming bandwidth of this GPU ----
    # a device-to-device copy of 1 GiB (reads and writes every byte once),
    # reported as (read + write bytes) / time, best of five
    src = torch.ones(ROTATE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    rd = []
    for _ in range(5):
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_ev.record(stream)
        dst.copy_(src)
        b_ev.record(stream)
        b_ev.synchronize()
        rd.append(a_ev.elapsed_time(b_ev))
    copy_gbs = 2 * ROTATE_BYTES / (min(rd) * 1e-3) / 1e9
    del src, dst

    us_call = ms_step * 1e3
    gbs = alg["bytes"] / (ms_step * 1e-3) / 1e9
    fwd_s = fwd_avg_ms * 1e-3
    fwd_gbs = alg["bytes"] / fwd_s / 1e9
    fwd_tfs = alg["flops"] / fwd_s / 1e12
    hbm_frac = fwd_gbs / HBM_PEAK_GBS
    if kind == "f32":
        bound, achieved, peak, unit = "alu", fwd_tfs, VALU_F32_PEAK_TFS, "TFLOP/s"
    elif alg["flops"] / alg["bytes"] > MFMA_F16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9):
        bound, achieved, peak, unit = "mfma", fwd_tfs, MFMA_F16_PEAK_TFS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", fwd_gbs, HBM_PEAK_GBS, "GB/s"

    # ---- aside: the tree-mask build (setup, not part of a verify call) ----
    mask_us = None
    if not quant and c.get("window_start") is None:
        m_out = torch.empty_like(base["mask"])
        ta.build_tree_mask(c["parents"], c["kv_seq_len"], c["mask_stride"], out=m_out)
        torch.cuda.synchronize()
        mt = []
        for _ in range(10):
            a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_ev.record(stream)
            ta.build_tree_mask(c["parents"], c["kv_seq_len"], c["mask_stride"], out=m_out)
            b_ev.record(stream)
            b_ev.synchronize()
            mt.append(a_ev.elapsed_time(b_ev) * 1e3)
        mask_us = round(statistics.median(mt), 2)
        del m_out

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (c.get("elem", "f16") if quant else "f16" if kind == "f16" else "f32"),
        "data": "synthetic (seeded normal Q/K/V, random tree)",
        "config": {"workload": args.workload, "nwg": nwg, "input_copies": ncopies,
                   "alg_bytes": alg["bytes"], "alg_flops": alg["flops"],
                   "parallelism": "single GPU"},
        "us_per_call": round(us_call, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "warm_us_per_call": round(warm_ms * 1e3, 2),
        "call_us_events": spread(call_ms),
        "forward_us_events": spread(fwd_ms),
        "copy_1GiB_GBs": round(copy_gbs, 1),
        "build_tree_mask_us": mask_us,
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(args.workload, kind),
                     "kernel": "forward", "avg_launch_us": round(fwd_avg_ms * 1e3, 2),
                     "event_floor_us": round(event_floor_us, 2),
                     "hbm_frac": round(hbm_frac, 4),
                     "mfma_frac": round(fwd_tfs / MFMA_F16_PEAK_TFS, 4)},
    }
    if not args.no_cpu_baseline:
        # the last call above ran on the base input set: compare it with the
        # oracle on the baseline's sample of rows
        torch.cuda.synchronize()
        gpu_out = out.float().cpu().numpy()
        elem = c.get("elem", "f16") if quant else None
        tol = 1e-4 if kind == "f32" else 2e-3
        result["cpu_baseline"] = cpu_baseline(args.workload, c, alg, quant, gpu_out=gpu_out,
                                              tol=tol, out_elem=elem)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
