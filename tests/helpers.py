"""Shared helpers for the GPU tests: device transfer and comparison."""

from __future__ import annotations

import sys

import numpy as np


def dev(a):
    """numpy array -> contiguous torch tensor on cuda:0 (same dtype)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    return t.detach().cpu().numpy()


def note(msg):
    """Name the case on stdout before a GPU step (flushed), so a failure that
    takes the process down still says which case was running."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (7 stored mantissa bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64)).astype(np.float32)
    e = ((a.view(np.uint32) >> np.uint32(23)) & np.uint32(0xff)).astype(np.int64)
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


def assert_close(got, ref, tol, what="", f16_out=False, out_elem=None):
    """max |got - ref| <= tol.  With f16_out (or out_elem "f16" / "bf16") the
    result was rounded to that type by contract, so each element may also
    carry that rounding: half an ulp of the exact value is added to its
    bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output " + what
    diff = np.abs(got - ref)
    bound = np.full(ref.shape, float(tol))
    if f16_out or out_elem == "f16":
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        bound = bound + 0.5 * ulp
    elif out_elem == "bf16":
        bound = bound + 0.5 * bf16_ulp(ref)
    worst = int(np.argmax(diff - bound)) if diff.size else 0
    ok = bool(np.all(diff <= bound))
    assert ok, "%s error %.3e > bound %.3e at flat index %d (max-abs %.3e)" % (
        what, diff.flat[worst], bound.flat[worst], worst, float(diff.max()))
    return float(diff.max()) if diff.size else 0.0


def sample_rows(q_l, n_heads, n, seed=0):
    """A fixed sample of (node, head) pairs: the first and last node, every
    head of node 0 and random others."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (q_l - 1, n_heads - 1), (q_l - 1, 0), (0, n_heads - 1)}
    while len(rows) < min(n, q_l * n_heads):
        rows.add((int(rng.integers(q_l)), int(rng.integers(n_heads))))
    return sorted(rows)
