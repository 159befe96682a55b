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


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output " + what
    err = max_abs(got, ref)
    assert err <= tol, "%s max-abs error %.3e > %.1e" % (what, err, tol)
    return err


def sample_rows(q_l, n_heads, n, seed=0):
    """A fixed sample of (node, head) pairs: the first and last node, every
    head of node 0 and random others."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (q_l - 1, n_heads - 1), (q_l - 1, 0), (0, n_heads - 1)}
    while len(rows) < min(n, q_l * n_heads):
        rows.add((int(rng.integers(q_l)), int(rng.integers(n_heads))))
    return sorted(rows)
