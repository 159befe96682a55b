"""Pins for the oracle's building blocks: f16 decode and the tree mask.

The oracle is test infrastructure; these tests tie it to facts outside itself
(numpy's own binary16 decoder, hand-written fixtures, brute-force ancestor
walks), so that a slip in it cannot hide behind a matching GPU result.
"""

import os

import numpy as np
import pytest

import oracle
from tree_masked_decode_amd import inputs

MASKED = np.float32(-65504.0)


def test_f16_decode_exhaustive():
    # Every binary16 bit pattern against numpy's float16 -> float64.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _read_mask_fixture(path):
    rows, meta = [], {}
    for line in open(path):
        line = line.rstrip("\n")
        if line.startswith("# q_l="):
            for kv in line[2:].split():
                k, v = kv.split("=")
                meta[k] = int(v)
        elif line.startswith("# parents="):
            meta["parents"] = [int(x) for x in line.split("=")[1].split(",")]
        elif line and not line.startswith("#"):
            rows.append([0.0 if c == "." else -65504.0 for c in line])
    return meta, np.array(rows, dtype=np.float32)


def test_tree_mask_golden_heap7(golden_dir):
    meta, expect = _read_mask_fixture(os.path.join(golden_dir, "tree_mask_heap7.txt"))
    got = oracle.tree_mask(meta["parents"], meta["kv_seq_len"], meta["mask_stride"])
    assert got.shape == expect.shape == (meta["q_l"], meta["mask_stride"])
    assert np.array_equal(got, expect)
    # the generator's heap tree is the fixture's tree
    assert list(inputs.parents_binary(7)) == meta["parents"]


def _ancestors(parents, i):
    out = {i}
    while parents[i] >= 0:
        i = int(parents[i])
        out.add(i)
    return out


@pytest.mark.parametrize("kind,q_l,L,stride", [
    ("chain", 4, 256, 256), ("binary", 16, 40, 45), ("dynamic", 64, 100, 128),
    ("dynamic", 1, 5, 5), ("binary", 9, 9, 9)])
def test_tree_mask_brute_force(kind, q_l, L, stride):
    parents = inputs.parents_for(kind, q_l, seed=3)
    m = oracle.tree_mask(parents, L, stride)
    base = L - q_l
    for i in range(q_l):
        anc = _ancestors(parents, i)
        for j in range(stride):
            visible = j < base or (base <= j < L and (j - base) in anc)
            assert m[i, j] == (0.0 if visible else MASKED), (i, j)


def test_chain_mask_equals_implicit_causal():
    # Implicit rule of "tree_attention.metal" header: row i sees j <= L - q_l + i.
    for q_l, L in [(1, 1), (4, 256), (8, 77), (33, 40)]:
        m = oracle.tree_mask(inputs.parents_chain(q_l), L)
        i = np.arange(q_l)[:, None]
        j = np.arange(L)[None, :]
        expect = np.where(j <= L - q_l + i, 0.0, -65504.0).astype(np.float32)
        assert np.array_equal(m, expect)


def test_heap_tree_row15_attends_its_path():
    # The 16-node binary tree of the fixed-tree workload: node 15's root path
    # is 15 -> 7 -> 3 -> 1 -> 0.
    L = 4096
    m = oracle.tree_mask(inputs.parents_binary(16), L)
    tail = np.nonzero(m[15, L - 16:] == 0.0)[0]
    assert list(tail) == [0, 1, 3, 7, 15]
    assert np.all(m[15, :L - 16] == 0.0)


@pytest.mark.parametrize("parents,L,stride", [
    ([0, 0, 1], 8, 8),        # root must have parent -1
    ([-1, 1, 0], 8, 8),       # parent must precede the node
    ([-1, 0, -1], 8, 8),      # only node 0 is a root
    ([-1, 0, 1], 2, 2),       # more nodes than KV positions
    ([-1, 0, 1], 8, 7),       # stride below kv_seq_len
])
def test_tree_mask_rejects_invalid(parents, L, stride):
    with pytest.raises(oracle.OracleError):
        oracle.tree_mask(parents, L, stride)


def test_dynamic_tree_generator_spans():
    p = inputs.parents_dynamic(64, seed=0)
    assert p[0] == -1
    for i in range(1, 64):
        assert max(0, i - 8) <= p[i] <= i - 1
