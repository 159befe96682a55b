"""Pins for the oracle's fp-path attention and its split/merge rule.

Each test checks the oracle against something it does not compute itself:
a numpy brute force in matrix form, closed forms, invariants of softmax
attention, and the page statements they come from ("tree_attention.metal",
mlx-native 0.9.1: explicit mask, implicit causal rule, GQA head mapping,
split-KV with a merge pass; "ops/tree_attention.rs", mlx-native 0.9.2:
query-outer output layout, mask sentinels).
"""

import numpy as np
import pytest

import oracle
from tree_masked_decode_amd import inputs

MASKED = -65504.0


def brute(q, k, v, mask, n_kv_heads, L, scale):
    """softmax(scale*Q K^T + mask, with masked cells removed) V, matrix form."""
    H, q_l, D = q.shape
    g = H // n_kv_heads
    out = np.zeros((q_l, H, D))
    for h in range(H):
        K = k[h // g, :L].astype(np.float64)
        V = v[h // g, :L].astype(np.float64)
        mk = mask[:, :L].astype(np.float64)
        z = scale * (q[h].astype(np.float64) @ K.T) + mk
        z[mk <= MASKED] = -np.inf
        mx = z.max(axis=1, keepdims=True)
        ok = np.isfinite(mx[:, 0])
        w = np.zeros_like(z)
        w[ok] = np.exp(z[ok] - mx[ok])
        s = w.sum(axis=1, keepdims=True)
        o = np.zeros((q_l, D))
        o[ok] = (w[ok] @ V) / s[ok]
        out[:, h, :] = o
    return out


def causal(q_l, L, stride=None):
    stride = stride or L
    i = np.arange(q_l)[:, None]
    j = np.arange(stride)[None, :]
    return np.where(j <= L - q_l + i, 0.0, MASKED).astype(np.float32)


def small(seed=0, H=4, Hk=2, D=128, L=37, cap=None, q_l=5, tree="dynamic",
          kv_dtype="f32", stride=None):
    cap = cap or L + 3
    return inputs.fp_case(dict(n_heads=H, n_kv_heads=Hk, head_dim=D,
                               kv_seq_len=L, kv_capacity=cap, q_l=q_l,
                               tree=tree, mask_stride=stride or L,
                               kv_dtype=kv_dtype, kv_std=1.0), seed=seed)


def run(c, mask, **kw):
    return oracle.attention(c["q"], c["k"], c["v"], mask,
                            n_kv_heads=c["n_kv_heads"],
                            kv_seq_len=c["kv_seq_len"], scale=c["scale"], **kw)


@pytest.mark.parametrize("seed,H,Hk,D,L,q_l,tree,kvd", [
    (0, 4, 2, 128, 37, 5, "dynamic", "f32"),
    (1, 6, 3, 64, 300, 8, "binary", "f16"),
    (2, 4, 1, 128, 17, 1, "chain", "f32"),
    (3, 8, 2, 32, 64, 7, "dynamic", "f16"),
])
def test_matches_brute_force(seed, H, Hk, D, L, q_l, tree, kvd):
    c = small(seed, H, Hk, D, L, None, q_l, tree, kvd)
    mask = oracle.tree_mask(c["parents"], L)
    got = run(c, mask)
    ref = brute(c["q"], c["k"], c["v"], mask, Hk, L, c["scale"])
    assert got.shape == (q_l, H, D)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_single_key_returns_that_value():
    c = small(4, L=1, cap=4, q_l=1, tree="chain")
    got = run(c, None)
    for h in range(c["n_heads"]):
        hk = h // (c["n_heads"] // c["n_kv_heads"])
        np.testing.assert_array_equal(got[0, h], c["v"][hk, 0].astype(np.float64))


def test_zero_query_is_mean_of_visible_values():
    c = small(5, L=50, q_l=6)
    c["q"][:] = 0.0
    mask = oracle.tree_mask(c["parents"], 50)
    got = run(c, mask)
    g = c["n_heads"] // c["n_kv_heads"]
    for i in range(6):
        vis = np.nonzero(mask[i, :50] == 0.0)[0]
        for h in range(c["n_heads"]):
            expect = c["v"][h // g, vis].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(got[i, h], expect, rtol=0, atol=1e-13)


def test_constant_values_pass_through():
    c = small(6, L=80, q_l=4)
    c["v"][:] = np.float32(0.375)
    got = run(c, oracle.tree_mask(c["parents"], 80))
    np.testing.assert_allclose(got, 0.375, rtol=0, atol=1e-14)


def test_two_keys_logistic():
    c = small(7, H=2, Hk=1, D=16, L=2, q_l=1, tree="chain")
    got = run(c, None)
    K = c["k"][0, :2].astype(np.float64)
    V = c["v"][0, :2].astype(np.float64)
    for h in range(2):
        l0, l1 = c["scale"] * (K @ c["q"][h, 0].astype(np.float64))
        p0 = 1.0 / (1.0 + np.exp(l1 - l0))
        np.testing.assert_allclose(got[0, h], p0 * V[0] + (1 - p0) * V[1],
                                   rtol=0, atol=1e-13)


def test_chain_mask_equals_implicit_exactly():
    for seed, L, q_l in [(8, 256, 4), (9, 33, 8), (10, 12, 12)]:
        c = small(seed, L=L, q_l=q_l, tree="chain")
        explicit = run(c, oracle.tree_mask(c["parents"], L))
        implicit = run(c, None)
        assert np.array_equal(explicit, implicit)


def test_fully_masked_prefix_leaves_only_ancestors():
    L, q_l = 90, 9
    c = small(11, L=L, q_l=q_l)
    mask = oracle.tree_mask(c["parents"], L)
    mask[:, :L - q_l] = MASKED
    got = run(c, mask)
    # Same problem restricted to the q_l tree positions, mask on the tree only.
    sub = dict(c)
    sub["k"] = np.ascontiguousarray(c["k"][:, L - q_l:L])
    sub["v"] = np.ascontiguousarray(c["v"][:, L - q_l:L])
    sub["kv_seq_len"] = q_l
    tree_only = oracle.tree_mask(c["parents"], q_l)
    ref = run(sub, tree_only)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)
    # and node 0 (the root) sees only itself
    g = c["n_heads"] // c["n_kv_heads"]
    for h in range(c["n_heads"]):
        np.testing.assert_allclose(got[0, h], c["v"][h // g, L - q_l], atol=1e-14)


def test_mask_shift_invariance():
    L = 70
    c = small(12, L=L, q_l=6)
    mask = oracle.tree_mask(c["parents"], L)
    shifted = np.where(mask == 0.0, np.float32(-3.25), mask).astype(np.float32)
    np.testing.assert_allclose(run(c, shifted), run(c, mask), rtol=0, atol=1e-13)


def test_additive_mask_values_enter_the_logit():
    # A bias of log(2) on one key doubles its weight relative to the others.
    c = small(13, H=1, Hk=1, D=8, L=3, q_l=1, tree="chain")
    c["q"][:] = 0.0
    mask = np.zeros((1, 3), dtype=np.float32)
    mask[0, 1] = np.float32(np.log(2.0))
    got = run(c, mask)
    V = c["v"][0, :3].astype(np.float64)
    w = np.array([1.0, float(np.exp(np.float64(mask[0, 1]))), 1.0])
    np.testing.assert_allclose(got[0, 0], (w @ V) / w.sum(), atol=1e-14)


def test_key_permutation_invariance():
    L = 64
    c = small(14, L=L, cap=L, q_l=5)
    mask = oracle.tree_mask(c["parents"], L)
    perm = np.random.default_rng(0).permutation(L)
    p = dict(c)
    p["k"] = np.ascontiguousarray(c["k"][:, perm])
    p["v"] = np.ascontiguousarray(c["v"][:, perm])
    np.testing.assert_allclose(run(p, np.ascontiguousarray(mask[:, perm])),
                               run(c, mask), rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    L = 40
    c = small(15, H=6, Hk=2, L=L, q_l=4)
    mask = oracle.tree_mask(c["parents"], L)
    m = dict(c)
    m["k"] = np.repeat(c["k"], 3, axis=0)
    m["v"] = np.repeat(c["v"], 3, axis=0)
    m["n_kv_heads"] = 6
    assert np.array_equal(run(m, mask), run(c, mask))


def test_output_layout_is_query_outer():
    # "ops/tree_attention.rs": out[i, h, :], not Q's [h, i, :].
    L = 30
    c = small(16, H=4, Hk=4, L=L, q_l=3)
    mask = oracle.tree_mask(c["parents"], L)
    full = run(c, mask)
    for i in range(3):
        for h in range(4):
            row = run(c, mask, rows=[(i, h)])
            assert np.array_equal(row[0], full[i, h])


def test_f16_kv_equals_f32_fed_decoded_values():
    L = 50
    c = small(17, L=L, q_l=4, kv_dtype="f16")
    mask = oracle.tree_mask(c["parents"], L)
    d = dict(c)
    d["k"] = c["k"].astype(np.float32)
    d["v"] = c["v"].astype(np.float32)
    assert np.array_equal(run(c, mask), run(d, mask))


def test_unread_regions_never_touched():
    L, stride, cap = 45, 52, 60
    c = small(18, L=L, cap=cap, q_l=5, stride=stride)
    mask = oracle.tree_mask(c["parents"], L, stride)
    ref = run(c, mask)
    poisoned = mask.copy()
    poisoned[:, L:] = np.nan
    c2 = dict(c)
    c2["k"] = c["k"].copy()
    c2["v"] = c["v"].copy()
    c2["k"][:, L:] = np.nan
    c2["v"][:, L:] = np.nan
    got = run(c2, poisoned)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, ref)


def test_row_with_no_visible_key_is_zero():
    L = 20
    c = small(19, L=L, q_l=3)
    mask = oracle.tree_mask(c["parents"], L)
    mask[1, :] = MASKED
    got = run(c, mask)
    assert np.all(got[1] == 0.0)
    assert np.any(got[0] != 0.0)


def test_implicit_mask_when_q_l_exceeds_visible_prefix():
    # Implicit rule with q_l > L: rows whose last visible key is negative see
    # nothing and produce zero.
    c = small(20, L=3, cap=3, q_l=5, tree="chain")
    got = run(c, None)
    ref = brute(c["q"], c["k"], c["v"], causal(5, 3), c["n_kv_heads"], 3, c["scale"])
    np.testing.assert_allclose(got, ref, atol=1e-13)
    assert np.all(got[:2] == 0.0)


@pytest.mark.parametrize("bounds", [
    [0, 37], [0, 10, 37], [0, 0, 5, 5, 36, 37], [0, 1, 2, 3, 30, 37]])
def test_split_partials_merge_to_direct(bounds):
    L = 37
    c = small(21, L=L, q_l=5)
    mask = oracle.tree_mask(c["parents"], L)
    o_un, s, m = oracle.attention_partials(c["q"], c["k"], c["v"], mask, bounds,
                                           n_kv_heads=c["n_kv_heads"],
                                           kv_seq_len=L, scale=c["scale"])
    merged = oracle.lse_combine(o_un, s, m).reshape(5, c["n_heads"], -1)
    np.testing.assert_allclose(merged, run(c, mask), rtol=0, atol=1e-12)
    # empty parts carry (0, 0, -inf)
    for w in range(len(bounds) - 1):
        if bounds[w] == bounds[w + 1]:
            assert np.all(s[:, w] == 0.0) and np.all(np.isneginf(m[:, w]))
            assert np.all(o_un[:, w] == 0.0)


def test_merge_of_hand_partials():
    # Two parts with known (O, S, M): result = (O1 e^M1 + O2 e^M2)/(S1 e^M1 + S2 e^M2)
    o = np.array([[[1.0, 2.0], [3.0, -1.0]]])
    s = np.array([[2.0, 4.0]])
    m = np.array([[0.5, -1.5]])
    got = oracle.lse_combine(o, s, m)
    e1, e2 = np.exp(0.5), np.exp(-1.5)
    expect = (o[0, 0] * e1 + o[0, 1] * e2) / (2.0 * e1 + 4.0 * e2)
    np.testing.assert_allclose(got[0], expect, rtol=1e-15)
    # all parts empty -> zero
    z = oracle.lse_combine(np.zeros((1, 2, 2)), np.zeros((1, 2)),
                           np.full((1, 2), -np.inf))
    assert np.all(z == 0.0)


# ---- implicit causal rule with a sliding-window start (R8W) ----

def windowed(q_l, L, ws, stride=None):
    """The explicit mask the "tree_attention.metal" header pairs with the
    implicit rule: 0 on [window_start, abs_pos], -65504 elsewhere."""
    stride = stride or L
    i = np.arange(q_l)[:, None]
    j = np.arange(stride)[None, :]
    return np.where((j >= ws) & (j <= L - q_l + i), 0.0, MASKED).astype(np.float32)


@pytest.mark.parametrize("L,q_l,ws,kvd", [(37, 5, 0, "f32"), (37, 5, 10, "f16"),
                                          (64, 3, 31, "f32"), (100, 8, 92, "f16")])
def test_window_start_matches_brute_force(L, q_l, ws, kvd):
    c = small(21, H=4, Hk=2, D=128, L=L, q_l=q_l, kv_dtype=kvd)
    got = run(c, None, window_start=ws)
    ref = brute(c["q"], c["k"], c["v"], windowed(q_l, L, ws), 2, L, c["scale"])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_window_start_equals_explicit_window_mask_exactly():
    c = small(22, H=4, Hk=1, D=128, L=50, q_l=4)
    for ws in (0, 1, 17, 46):
        assert np.array_equal(run(c, None, window_start=ws),
                              run(c, windowed(4, 50, ws)))


def test_window_start_zero_is_plain_implicit():
    c = small(23, H=2, Hk=2, D=128, L=33, q_l=6)
    assert np.array_equal(run(c, None, window_start=0), run(c, None))


def test_window_start_at_last_row_position_is_one_value():
    # the last node sees exactly one key when window_start = abs_pos = L - 1
    L, q_l = 40, 3
    c = small(24, H=2, Hk=1, D=128, L=L, q_l=q_l)
    got = run(c, None, window_start=L - 1)
    np.testing.assert_array_equal(got[q_l - 1, 0], c["v"][0, L - 1].astype(np.float64))
    # earlier nodes' abs_pos < window_start: nothing visible, zeros (R2)
    assert np.array_equal(got[: q_l - 1], np.zeros_like(got[: q_l - 1]))


def test_window_start_with_mask_is_rejected():
    c = small(25, H=2, Hk=1, D=128, L=20, q_l=2)
    with pytest.raises(oracle.OracleError):
        run(c, causal(2, 20), window_start=3)
