"""GPU parity of the fp path (tree mask, forward, reduce) against the oracle.

Tolerances are the contract's: max-abs 1e-4 for fp32 K/V, 2e-3 for fp16
K/V.  An explicit chain mask must reproduce the implicit causal path byte
for byte ("tree_attention.metal" header: the "tree=1" parity gate).
"""

import math

import numpy as np
import pytest

import oracle
from tree_masked_decode_amd import inputs

from helpers import assert_close, dev, host, note, sample_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "f16": 2e-3}


@pytest.fixture(scope="module")
def ta():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import tree_masked_decode_amd as ta
    ta._api()  # the HIP library must load
    return ta


def gpu_case(c, mask_np):
    return (dev(c["q"]), dev(c["k"]), dev(c["v"]),
            None if mask_np is None else dev(mask_np))


def run_verify(ta, c, mask_np, nwg=None, **kw):
    import torch
    q, k, v, m = gpu_case(c, mask_np)
    out = ta.verify(q, k, v, m, kv_seq_len=c["kv_seq_len"], scale=c["scale"],
                    nwg=nwg, **kw)
    torch.cuda.synchronize()
    return host(out)


def small_case(seed, H, Hk, D, L, q_l, kvd, tree="dynamic", cap=None, stride=None,
               scale=None):
    return inputs.fp_case(dict(n_heads=H, n_kv_heads=Hk, head_dim=D, kv_seq_len=L,
                               kv_capacity=cap or L + 7, q_l=q_l, tree=tree,
                               mask_stride=stride or L, kv_dtype=kvd, kv_std=1.0,
                               scale=scale),
                          seed=seed)


# --------------------------------------------------------------------------
# tree mask
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,q_l,L,stride", [
    ("chain", 4, 256, 256), ("binary", 16, 4096, 4096), ("dynamic", 64, 32768, 32768),
    ("chain", 8, 1000, 1003), ("dynamic", 1, 1, 1), ("dynamic", 300, 300, 301),
    ("binary", 1024, 5000, 5000)])
def test_tree_mask_bit_exact(ta, kind, q_l, L, stride):
    import torch
    note("tree_mask %s q_l=%d L=%d stride=%d" % (kind, q_l, L, stride))
    parents = inputs.parents_for(kind, q_l, seed=0)
    got = ta.build_tree_mask(parents, L, stride)
    torch.cuda.synchronize()
    ref = oracle.tree_mask(parents, L, stride)
    assert np.array_equal(host(got), ref)


# --------------------------------------------------------------------------
# forward + reduce parity on small shapes (several tiles, ragged tails)
# --------------------------------------------------------------------------
SMALL = [
    # seed, H, Hk, D, L, q_l, kv dtype, nwg
    (0, 4, 2, 128, 333, 5, "f32", 1),
    (1, 4, 2, 128, 333, 5, "f32", 3),
    (2, 8, 2, 256, 1000, 7, "f32", None),
    (3, 4, 4, 512, 257, 3, "f32", 2),
    (4, 4, 2, 128, 1000, 5, "f16", 1),
    (5, 12, 2, 256, 777, 16, "f16", 4),
    (6, 24, 4, 256, 1500, 16, "f16", None),
    (7, 8, 8, 512, 611, 9, "f16", 3),
    (8, 6, 1, 128, 2049, 33, "f16", 5),   # 198 rows: 4 row tiles, last ragged
    (9, 2, 1, 256, 65, 1, "f16", 7),      # more splits than tiles
    # launch plans and mask-tile heights of the fp16 kernel
    (10, 12, 2, 128, 700, 32, "f16", None),  # d 128, 3 row blocks (192 rows), 32 mask rows
    (11, 4, 2, 128, 900, 100, "f16", 3),     # d 128, 2 row blocks, 128 mask rows
    (12, 2, 1, 128, 500, 190, "f16", 2),     # d 128, 3 row blocks, 192 mask rows
    (13, 4, 4, 256, 600, 100, "f16", 2),     # d 256, group 1: 128 mask rows
    (14, 16, 8, 512, 700, 40, "f16", 4),     # d 512: 80 rows in 2 row tiles, 64 mask rows
]


@pytest.mark.parametrize("seed,H,Hk,D,L,q_l,kvd,nwg", SMALL)
def test_forward_parity_small(ta, seed, H, Hk, D, L, q_l, kvd, nwg):
    note("fp small seed=%d H=%d Hk=%d D=%d L=%d q_l=%d %s nwg=%s" %
         (seed, H, Hk, D, L, q_l, kvd, nwg))
    c = small_case(seed, H, Hk, D, L, q_l, kvd)
    mask = oracle.tree_mask(c["parents"], L, c["mask_stride"])
    got = run_verify(ta, c, mask, nwg=nwg)
    ref = oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=Hk,
                           kv_seq_len=L, scale=c["scale"])
    assert_close(got, ref, TOL[kvd], "small %d" % seed)


# --------------------------------------------------------------------------
# the workloads at full size
# --------------------------------------------------------------------------
def test_workload_tiny_chain(ta):
    note("workload tiny_chain")
    c = inputs.fp_case("tiny_chain")
    mask = oracle.tree_mask(c["parents"], c["kv_seq_len"], c["mask_stride"])
    got = run_verify(ta, c, mask, nwg=c["nwg"])
    ref = oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=c["n_kv_heads"],
                           kv_seq_len=c["kv_seq_len"], scale=c["scale"])
    assert_close(got, ref, TOL["f32"], "tiny_chain")
    # byte identity with the implicit causal path
    implicit = run_verify(ta, c, None, nwg=c["nwg"])
    assert np.array_equal(got.view(np.uint32), implicit.view(np.uint32))


def test_workload_fixed_tree(ta):
    note("workload fixed_tree")
    c = inputs.fp_case("fixed_tree")
    mask = oracle.tree_mask(c["parents"], c["kv_seq_len"], c["mask_stride"])
    got = run_verify(ta, c, mask)
    ref = oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=c["n_kv_heads"],
                           kv_seq_len=c["kv_seq_len"], scale=c["scale"])
    assert_close(got, ref, TOL["f16"], "fixed_tree")


def _sampled(ta, name, nrows, gpu_mask=True):
    """Run a workload at full size in bench.py's launch configuration and
    compare nrows (node, head) rows with the oracle (every row if nrows is
    None)."""
    import torch
    c = inputs.fp_case(name)
    L, H = c["kv_seq_len"], c["n_heads"]
    mask_np = oracle.tree_mask(c["parents"], L, c["mask_stride"])
    q, k, v, _ = gpu_case(c, None)
    m = ta.build_tree_mask(c["parents"], L, c["mask_stride"])
    nwg = ta.pick_nwg(H, c["n_kv_heads"], c["head_dim"], L, c["q_l"], 1)
    out = ta.verify(q, k, v, m, kv_seq_len=L, scale=c["scale"], nwg=nwg)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(np.isfinite(got))
    if nrows is None:
        ref = oracle.attention(c["q"], c["k"], c["v"], mask_np, n_kv_heads=c["n_kv_heads"],
                               kv_seq_len=L, scale=c["scale"])
        assert_close(got, ref, TOL["f16"], name)
    else:
        rows = sample_rows(c["q_l"], H, nrows)
        ref = oracle.attention(c["q"], c["k"], c["v"], mask_np, n_kv_heads=c["n_kv_heads"],
                               kv_seq_len=L, scale=c["scale"], rows=rows)
        sel = np.stack([got[i, h] for i, h in rows])
        assert_close(sel, ref, TOL["f16"], name)
    return c, (q, k, v, m), nwg, got


def test_workload_dynamic_tree_32k(ta):
    note("workload dynamic_tree_32k (every row)")
    _sampled(ta, "dynamic_tree_32k", None)


def test_workload_long_context_128k(ta):
    import torch
    note("workload long_context_128k (sampled rows) + byte identity")
    c, (q, k, v, m), nwg, got = _sampled(ta, "long_context_128k", 64)
    implicit = ta.verify(q, k, v, None, kv_seq_len=c["kv_seq_len"], scale=c["scale"],
                         nwg=nwg)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), host(implicit).view(np.uint32))


# --------------------------------------------------------------------------
# byte identity, poison, determinism, edges
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kvd,D,nwg", [("f32", 128, 3), ("f16", 256, 4), ("f16", 512, 1),
                                       ("f16", 128, 1)])
def test_chain_mask_byte_identical_to_implicit(ta, kvd, D, nwg):
    note("byte identity %s D=%d nwg=%d" % (kvd, D, nwg))
    c = small_case(11, 8, 2, D, 517, 9, kvd, tree="chain")
    mask = oracle.tree_mask(c["parents"], 517, 517)
    a = run_verify(ta, c, mask, nwg=nwg)
    b = run_verify(ta, c, None, nwg=nwg)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("kvd", ["f32", "f16"])
def test_unread_regions_poisoned(ta, kvd):
    import torch
    note("poison %s" % kvd)
    L, stride, cap = 700, 709, 900
    c = small_case(12, 8, 2, 256, L, 9, kvd, cap=cap, stride=stride)
    mask = oracle.tree_mask(c["parents"], L, stride)
    clean = run_verify(ta, c, mask, nwg=3)
    # K/V capacity tail -> NaN; mask padding -> 0 ("attended" if it were read)
    p = dict(c)
    p["k"] = c["k"].copy()
    p["v"] = c["v"].copy()
    p["k"][:, L:] = np.nan
    p["v"][:, L:] = np.nan
    pm = mask.copy()
    pm[:, L:] = 0.0
    q, k, v, m = gpu_case(p, pm)
    H, q_l, D = c["q"].shape
    # partial scratch pre-filled with NaN; output with a canary tail
    import tree_masked_decode_amd as T
    part = torch.full((T.partials_bytes(H, D, q_l, 3) // 4,), float("nan"), device="cuda")
    flat = torch.full((q_l * H * D + 64,), 12345.0, device="cuda")
    out = flat[: q_l * H * D].view(q_l, H, D)
    T.verify(q, k, v, m, kv_seq_len=L, scale=c["scale"], nwg=3, out=out, partials=part)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), clean.view(np.uint32))
    assert torch.all(flat[q_l * H * D:] == 12345.0)


def test_deterministic(ta):
    note("determinism")
    c = small_case(13, 24, 4, 256, 3000, 16, "f16", tree="binary")
    mask = oracle.tree_mask(c["parents"], 3000)
    a = run_verify(ta, c, mask)
    b = run_verify(ta, c, mask)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("kvd", ["f32", "f16"])
def test_edges(ta, kvd):
    note("edges %s" % kvd)
    tol = TOL[kvd]
    # one key
    c = small_case(14, 4, 2, 128, 1, 1, kvd, tree="chain", cap=1)
    got = run_verify(ta, c, None, nwg=1)
    ref = oracle.attention(c["q"], c["k"], c["v"], None, n_kv_heads=2, kv_seq_len=1,
                           scale=c["scale"])
    assert_close(got, ref, tol, "L=1")
    # whole cache is the tree (no prefix), implicit rule with q_l > L
    c = small_case(15, 4, 1, 256, 40, 40, kvd)
    m = oracle.tree_mask(c["parents"], 40)
    assert_close(run_verify(ta, c, m, nwg=2),
                 oracle.attention(c["q"], c["k"], c["v"], m, n_kv_heads=1, kv_seq_len=40,
                                  scale=c["scale"]), tol, "q_l=L")
    c = small_case(16, 2, 1, 128, 5, 9, kvd, tree="chain")
    assert_close(run_verify(ta, c, None, nwg=2),
                 oracle.attention(c["q"], c["k"], c["v"], None, n_kv_heads=1, kv_seq_len=5,
                                  scale=c["scale"]), tol, "q_l>L implicit")
    # rows with no visible key -> 0; fully masked prefix -> ancestors only
    c = small_case(17, 8, 2, 256, 1200, 12, kvd)
    m = oracle.tree_mask(c["parents"], 1200)
    m[:, :1200 - 12] = -65504.0
    m[3, :] = -65504.0
    got = run_verify(ta, c, m, nwg=4)
    assert np.all(got[3] == 0.0)
    assert_close(got, oracle.attention(c["q"], c["k"], c["v"], m, n_kv_heads=2,
                                       kv_seq_len=1200, scale=c["scale"]), tol, "masked")
    # additive (non-sentinel) mask values
    c = small_case(18, 4, 2, 128, 300, 4, kvd)
    m = np.random.default_rng(3).uniform(-4, 1, size=(4, 300)).astype(np.float32)
    assert_close(run_verify(ta, c, m, nwg=2),
                 oracle.attention(c["q"], c["k"], c["v"], m, n_kv_heads=2, kv_seq_len=300,
                                  scale=c["scale"]), tol, "additive")


@pytest.mark.parametrize("H,D,nwg", [(2, 128, 1), (2, 512, 2), (8, 256, 1), (8, 256, 3)])
def test_implicit_rows_before_the_cache(ta, H, D, nwg):
    # q_l > kv_seq_len under the implicit rule: nodes 0..35 have their last
    # visible key before key 0, see nothing and must come out as zeros (the
    # fast-tile bound of the first workgroup is negative there)
    note("implicit q_l=100 L=64 H=%d D=%d nwg=%d" % (H, D, nwg))
    c = small_case(21, H, 1, D, 64, 100, "f16", tree="chain")
    got = run_verify(ta, c, None, nwg=nwg)
    ref = oracle.attention(c["q"], c["k"], c["v"], None, n_kv_heads=1, kv_seq_len=64,
                           scale=c["scale"])
    assert np.all(got[:36] == 0.0)
    assert_close(got, ref, TOL["f16"], "q_l=100 L=64")


@pytest.mark.parametrize("kvd", ["f32", "f16"])
def test_dead_band_inside_one_split(ta, kvd):
    # live tiles, then whole tiles masked for every row (skipped), then live
    # tiles again, all in one split: the tile after the band must be fetched
    # although the band's arithmetic was skipped
    note("dead band inside one split %s" % kvd)
    c = small_case(20, 8, 2, 128, 700, 6, kvd)
    m = oracle.tree_mask(c["parents"], 700)
    m[:, 96:352] = -65504.0      # tiles 3..10 of 32 keys (and 6..21 of 16)
    ref = oracle.attention(c["q"], c["k"], c["v"], m, n_kv_heads=2, kv_seq_len=700,
                           scale=c["scale"])
    for nwg in (1, 2):
        assert_close(run_verify(ta, c, m, nwg=nwg), ref, TOL[kvd], "band nwg=%d" % nwg)


def test_unaligned_mask_stride(ta):
    note("odd mask stride (scalar mask path)")
    c = small_case(19, 8, 2, 256, 501, 6, "f16", stride=503)
    m = oracle.tree_mask(c["parents"], 501, 503)
    assert_close(run_verify(ta, c, m, nwg=2),
                 oracle.attention(c["q"], c["k"], c["v"], m, n_kv_heads=2, kv_seq_len=501,
                                  scale=c["scale"]), TOL["f16"], "stride 503")


def test_reduce_alone_on_oracle_partials(ta):
    """Feed exact partials from the oracle's split into the reduce kernel."""
    import torch
    note("reduce alone")
    c = small_case(20, 4, 2, 128, 90, 3, "f32")
    m = oracle.tree_mask(c["parents"], 90)
    bounds = [0, 0, 17, 50, 50, 90]
    o_un, s, mx = oracle.attention_partials(c["q"], c["k"], c["v"], m, bounds,
                                            n_kv_heads=2, kv_seq_len=90, scale=c["scale"])
    nrows, nw, D = o_un.shape
    # this library's layout: O[w][row][D], then (S, M) [w][row][2], M in base 2
    po = np.transpose(o_un, (1, 0, 2)).astype(np.float32).ravel()
    sm = np.stack([s.T, mx.T * (1.0 / math.log(2.0))], axis=-1).astype(np.float32).ravel()
    part = dev(np.concatenate([po, sm]))
    import tree_masked_decode_amd as T
    for dt, tol in ((torch.float32, 1e-5), (torch.float16, 2e-3)):
        out = torch.empty((nrows, D), dtype=dt, device="cuda")
        T.tree_attn_reduce(part, out, nrows=nrows, head_dim=D, nwg=nw)
        torch.cuda.synchronize()
        assert_close(host(out), oracle.lse_combine(o_un, s, mx), tol, "reduce")


# --------------------------------------------------------------------------
# the wide fp16 forward (head dim 256, at least 192 rows per kv head: one
# wavefront per SIMD with 48 rows, 192-row tiles, 4-stage K/V ring, mask
# cells classified per tile)
# --------------------------------------------------------------------------
WIDE = [
    # seed, H, Hk, L, q_l, tree, nwg, softmax scale (None: 1/sqrt(256))
    (60, 24, 4, 1000, 64, "dynamic", 3, None),    # 384 rows: two row tiles; ragged tail
    (61, 12, 2, 2049, 40, "dynamic", 5, None),    # 240 rows: the second tile has 3 padding waves
    (62, 16, 4, 777, 64, "dynamic", None, None),  # group 4: two mask copies per wavefront
    (63, 24, 4, 3000, 64, "binary", 2, 0.125),    # logits twice as wide: the reference max moves
    (64, 24, 4, 40, 32, "dynamic", 1, None),      # one partial tile, direct output
    (65, 24, 4, 5000, 64, "chain", 7, None),
    (66, 12, 2, 33, 32, "dynamic", 2, None),      # two tiles, the second holds one key
    (67, 48, 8, 1500, 16, "binary", None, None),  # group 6, 96 rows: not wide (reference plan)
]


@pytest.mark.parametrize("seed,H,Hk,L,q_l,tree,nwg,scale", WIDE)
def test_wide_forward_parity(ta, seed, H, Hk, L, q_l, tree, nwg, scale):
    note("wide seed=%d H=%d Hk=%d L=%d q_l=%d %s nwg=%s scale=%s" %
         (seed, H, Hk, L, q_l, tree, nwg, scale))
    c = small_case(seed, H, Hk, 256, L, q_l, "f16", tree=tree, scale=scale)
    mask = oracle.tree_mask(c["parents"], L, c["mask_stride"])
    got = run_verify(ta, c, mask, nwg=nwg)
    ref = oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=Hk,
                           kv_seq_len=L, scale=c["scale"])
    assert_close(got, ref, TOL["f16"], "wide %d" % seed)


@pytest.mark.parametrize("nwg", [1, 4])
def test_wide_chain_byte_identical_to_implicit(ta, nwg):
    note("wide byte identity nwg=%d" % nwg)
    L, q_l = 1500, 40
    c = small_case(68, 24, 4, 256, L, q_l, "f16", tree="chain")
    mask = oracle.tree_mask(c["parents"], L, L)
    a = run_verify(ta, c, mask, nwg=nwg)
    b = run_verify(ta, c, None, nwg=nwg)
    ref = oracle.attention(c["q"], c["k"], c["v"], None, n_kv_heads=4, kv_seq_len=L,
                           scale=c["scale"])
    assert_close(b, ref, TOL["f16"], "wide implicit")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("ws,nwg", [(100, 3), (31, 2), (1990, 5), (0, None)])
def test_wide_decode_window(ta, ws, nwg):
    note("wide decode ws=%d nwg=%s" % (ws, nwg))
    L, q_l = 2000, 40
    c = small_case(69, 24, 4, 256, L, q_l, "f16", tree="chain")
    got = run_decode(ta, c, ws, nwg)
    ref = oracle.attention(c["q"], c["k"], c["v"], None, n_kv_heads=4, kv_seq_len=L,
                           scale=c["scale"], window_start=ws)
    assert_close(got, ref, TOL["f16"], "wide decode ws=%d" % ws)
    abs_pos = L - q_l + np.arange(q_l)
    assert np.all(got[abs_pos < ws] == 0.0)


def test_wide_masks(ta):
    note("wide masked rows, masked band, additive cells")
    L, q_l = 1200, 40
    c = small_case(70, 24, 4, 256, L, q_l, "f16")
    m = oracle.tree_mask(c["parents"], L)
    m[:, 96:352] = -65504.0           # a band of whole tiles masked for every row
    m[3, :] = -65504.0                # a row that sees nothing
    m[:, 500:510] = -np.inf           # -inf cells are excluded as well
    got = run_verify(ta, c, m, nwg=3)
    assert np.all(got[3] == 0.0)
    assert_close(got, oracle.attention(c["q"], c["k"], c["v"], m, n_kv_heads=4,
                                       kv_seq_len=L, scale=c["scale"]), TOL["f16"], "band")
    # additive (non-sentinel) mask values everywhere: every tile takes the
    # per-cell path
    m2 = np.random.default_rng(5).uniform(-4, 1, size=(q_l, L)).astype(np.float32)
    assert_close(run_verify(ta, c, m2, nwg=2),
                 oracle.attention(c["q"], c["k"], c["v"], m2, n_kv_heads=4, kv_seq_len=L,
                                  scale=c["scale"]), TOL["f16"], "additive")
    # prefix fully masked: only ancestors and self
    m3 = oracle.tree_mask(c["parents"], L)
    m3[:, :L - q_l] = -65504.0
    assert_close(run_verify(ta, c, m3, nwg=4),
                 oracle.attention(c["q"], c["k"], c["v"], m3, n_kv_heads=4, kv_seq_len=L,
                                  scale=c["scale"]), TOL["f16"], "masked prefix")


def test_wide_poisoned_and_deterministic(ta):
    import torch
    note("wide poison + determinism")
    L, stride, cap, q_l = 1100, 1108, 1300, 40
    c = small_case(71, 24, 4, 256, L, q_l, "f16", cap=cap, stride=stride)
    mask = oracle.tree_mask(c["parents"], L, stride)
    clean = run_verify(ta, c, mask, nwg=3)
    again = run_verify(ta, c, mask, nwg=3)
    assert np.array_equal(clean.view(np.uint32), again.view(np.uint32))
    p = dict(c)
    p["k"] = c["k"].copy()
    p["v"] = c["v"].copy()
    p["k"][:, L:] = np.nan
    p["v"][:, L:] = np.nan
    pm = mask.copy()
    pm[:, L:] = 0.0
    q, k, v, m = gpu_case(p, pm)
    H = c["q"].shape[0]
    import tree_masked_decode_amd as T
    part = torch.full((T.partials_bytes(H, 256, q_l, 3) // 4,), float("nan"), device="cuda")
    out = torch.full((q_l, H, 256), 12345.0, device="cuda")
    T.verify(q, k, v, m, kv_seq_len=L, scale=c["scale"], nwg=3, out=out, partials=part)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), clean.view(np.uint32))


# --------------------------------------------------------------------------
# causal decode with a sliding-window start (tree_attn_decode)
# --------------------------------------------------------------------------
DECODE = [
    # seed, H, Hk, D, L, q_l, kv dtype, window_start, nwg
    (40, 4, 2, 128, 333, 5, "f32", 0, 3),
    (41, 4, 2, 128, 333, 5, "f32", 5, 3),
    (42, 8, 2, 256, 517, 9, "f16", 31, 4),
    (43, 8, 2, 256, 517, 9, "f16", 32, 4),      # window starts on a tile edge
    (44, 8, 2, 256, 517, 9, "f16", 33, None),
    (45, 8, 1, 512, 700, 3, "f16", 300, 2),
    (46, 4, 4, 128, 1000, 1, "f16", 999, 1),     # the last key only
    (47, 4, 2, 512, 257, 4, "f32", 100, 2),      # fp32, 16-key tiles
    (48, 6, 2, 128, 2000, 16, "f16", 1990, 5),   # early nodes see nothing
    (49, 24, 4, 256, 4096, 16, "f16", 1000, None),
]


def run_decode(ta, c, ws, nwg=None):
    import torch
    q, k, v, _ = gpu_case(c, None)
    out = ta.decode(q, k, v, kv_seq_len=c["kv_seq_len"], scale=c["scale"],
                    window_start=ws, nwg=nwg)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("seed,H,Hk,D,L,q_l,kvd,ws,nwg", DECODE)
def test_decode_window_parity(ta, seed, H, Hk, D, L, q_l, kvd, ws, nwg):
    note("decode seed=%d H=%d Hk=%d D=%d L=%d q_l=%d %s ws=%d nwg=%s"
         % (seed, H, Hk, D, L, q_l, kvd, ws, nwg))
    c = small_case(seed, H, Hk, D, L, q_l, kvd, tree="chain")
    got = run_decode(ta, c, ws, nwg)
    ref = oracle.attention(c["q"], c["k"], c["v"], None, n_kv_heads=Hk, kv_seq_len=L,
                           scale=c["scale"], window_start=ws)
    assert_close(got, ref, TOL[kvd], "decode %d" % seed)
    abs_pos = L - q_l + np.arange(q_l)
    assert np.all(got[abs_pos < ws] == 0.0)


@pytest.mark.parametrize("kvd,D,ws,nwg", [("f32", 128, 3, 3), ("f16", 256, 17, 4),
                                          ("f16", 512, 31, 2), ("f16", 128, 0, 5)])
def test_decode_window_in_first_tile_byte_identical_to_explicit(ta, kvd, D, ws, nwg):
    note("decode byte identity %s D=%d ws=%d nwg=%d" % (kvd, D, ws, nwg))
    L, q_l = 517, 9
    c = small_case(50, 8, 2, D, L, q_l, kvd, tree="chain")
    i = np.arange(q_l)[:, None]
    j = np.arange(L)[None, :]
    mask = np.where((j >= ws) & (j <= L - q_l + i), 0.0, -65504.0).astype(np.float32)
    a = run_verify(ta, c, mask, nwg=nwg)
    b = run_decode(ta, c, ws, nwg)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---- the live-key scan of an explicit mask (K/V >= 64 MiB, mask <= 1/32) ----
RANGE = [
    # seed, H, Hk, D, L, q_l, kv dtype, window start, nwg   (kernel)
    (80, 8, 2, 512, 32768, 4, "f16", 24576, 8),     # fp16, one row block per wave
    (81, 8, 2, 512, 32768, 4, "f16", 24577, 5),     # window inside a tile
    (82, 24, 1, 256, 65536, 8, "f16", 49152, 16),   # wide (192 rows)
    (83, 4, 2, 128, 65536, 2, "f32", 40960, 6),     # fp32
]


def _window_mask(L, q_l, ws):
    i = np.arange(q_l)[:, None]
    j = np.arange(L)[None, :]
    return np.where((j >= ws) & (j <= L - q_l + i), 0.0, -65504.0).astype(np.float32)


@pytest.mark.parametrize("seed,H,Hk,D,L,q_l,kvd,ws,nwg", RANGE)
def test_explicit_window_live_range(ta, seed, H, Hk, D, L, q_l, kvd, ws, nwg):
    note("live range seed=%d H=%d Hk=%d D=%d L=%d q_l=%d %s ws=%d nwg=%d"
         % (seed, H, Hk, D, L, q_l, kvd, ws, nwg))
    c = small_case(seed, H, Hk, D, L, q_l, kvd, tree="chain", cap=L)
    mask = _window_mask(L, q_l, ws)
    got = run_verify(ta, c, mask, nwg=nwg)
    ref = oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=Hk, kv_seq_len=L,
                           scale=c["scale"])
    assert_close(got, ref, TOL[kvd], "explicit window %d" % seed)
    # a window that starts on a tile edge splits exactly the tiles the
    # implicit rule's window start does: the same bytes as tree_attn_decode
    bn = 32 if kvd == "f16" else (16 if D == 512 else 32)
    if ws % bn == 0:
        b = run_decode(ta, c, ws, nwg)
        assert np.array_equal(got.view(np.uint32), b.view(np.uint32))


def test_explicit_mask_live_range_edges(ta):
    # fp16 d=512, 64 MiB of K/V: a dead band in the middle (kept, skipped per
    # tile), every cell dead (zeros), one live key at the very end
    H, Hk, D, L, q_l = 8, 1, 512, 32768, 3
    c = small_case(84, H, Hk, D, L, q_l, "f16", tree="chain", cap=L)
    for name, mask in (
            ("band", np.where((np.arange(L) // 1000) % 7 == 3, -65504.0, 0.0)
             .astype(np.float32)[None, :].repeat(q_l, 0)),
            ("dead", np.full((q_l, L), -65504.0, np.float32)),
            ("last key", np.where(np.arange(L) == L - 1, 0.0, -65504.0)
             .astype(np.float32)[None, :].repeat(q_l, 0))):
        note("live range edges: %s" % name)
        got = run_verify(ta, c, mask, nwg=7)
        ref = oracle.attention(c["q"], c["k"], c["v"], mask, n_kv_heads=Hk, kv_seq_len=L,
                               scale=c["scale"])
        assert_close(got, ref, TOL["f16"], name)
        if name == "dead":
            assert np.all(got == 0.0)


def test_workload_decode_window_128k(ta):
    note("workload decode_window_128k (sampled rows)")
    c = inputs.fp_case("decode_window_128k")
    L, H, ws = c["kv_seq_len"], c["n_heads"], c["window_start"]
    got = run_decode(ta, c, ws)
    assert np.all(np.isfinite(got))
    rows = sample_rows(c["q_l"], H, 16)
    ref = oracle.attention(c["q"], c["k"], c["v"], None, n_kv_heads=c["n_kv_heads"],
                           kv_seq_len=L, scale=c["scale"], window_start=ws, rows=rows)
    sel = np.stack([got[i, h] for i, h in rows])
    assert_close(sel, ref, TOL["f16"], "decode_window_128k")
