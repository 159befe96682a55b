"""Pins for the oracle's affine-quantized K/V attention.

Source: "ffai/flash_quantized_sdpa.rs" (metaltile-std 0.1.0) -- layout doc,
base kernel macro (dequant x = scale_g * code + bias_g, GQA q_idx/repeat,
sink initialisation, final o / l), float-mask macro (additive bias),
bool-mask macro (a zero u32 drops the token) and the sliding-window gate
(token t kept iff t + window > tokens - 1).
"""

import os

import numpy as np
import pytest

import oracle
from tree_masked_decode_amd import inputs


def qcase(seed=0, B=2, nQ=4, nKV=2, dim=64, L=40, cap=None, q_l=1, bits=4, G=32,
          sinks=False, mask=None, window=0):
    return inputs.quant_case(dict(batch=B, n_q_heads=nQ, n_kv_heads=nKV, dim=dim,
                                  kv_seq_len=L, kv_capacity=cap or L, q_l=q_l,
                                  bits=bits, group_size=G, sinks=sinks,
                                  mask=mask, window_size=window), seed=seed)


def qrun(c, **kw):
    args = dict(n_kv_heads=c["n_kv_heads"], kv_seq_len=c["kv_seq_len"],
                bits=c["bits"], group_size=c["group_size"], scale=c["scale"],
                sinks=c["sinks"], mask=c["mask"], mask_bool=c.get("mask_bool"),
                mask_head_stride=c["mask_head_stride"],
                mask_stride=c["mask_stride"], window_size=c.get("window_size", 0))
    args.update(kw)
    return oracle.quant_attention(c["q"], c["k_packed"], c["k_scales"],
                                  c["k_biases"], c["v_packed"], c["v_scales"],
                                  c["v_biases"], **args)


def _word_fixture(golden_dir):
    rows = []
    for line in open(os.path.join(golden_dir, "quant_word_order.txt")):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        rows.append((int(parts[0]), int(parts[1], 16), [int(x) for x in parts[2:]]))
    return rows


def test_word_order_golden(golden_dir):
    # One key (so the output IS the dequantised value row), scale 1, bias 0.
    for bits, word, codes in _word_fixture(golden_dir):
        dim = 32 // bits
        c = qcase(B=1, nQ=1, nKV=1, dim=dim, L=1, bits=bits, G=dim)
        c["v_packed"][:] = np.uint32(word)
        c["v_scales"][:] = np.float16(1.0)
        c["v_biases"][:] = np.float16(0.0)
        got = qrun(c)
        assert np.array_equal(got[0, 0], np.array(codes, dtype=np.float64))
        # the generator packs in the same order
        assert int(inputs.pack_codes(np.array([codes]), bits)[0, 0]) == word


def test_affine_dequant_per_group():
    # single key: out = s_g * code + b_g, group g = d // G
    c = qcase(1, B=1, nQ=2, nKV=1, dim=64, L=1, bits=4, G=16)
    got = qrun(c)
    pf = 8
    words = c["v_packed"][0, 0]
    sc = c["v_scales"][0, 0].astype(np.float64)
    bi = c["v_biases"][0, 0].astype(np.float64)
    for d in range(64):
        code = (int(words[d // pf]) >> ((d % pf) * 4)) & 15
        expect = sc[d // 16] * code + bi[d // 16]
        assert got[0, 0, d] == expect and got[1, 0, d] == expect


def test_eight_bit_unit_affine_equals_fp_path():
    # 8-bit codes with scale 1, bias 0 are exactly the integers; the fp-path
    # oracle fed those integers (and the same Q) must agree.
    B, nQ, nKV, dim, L = 1, 4, 2, 64, 33
    c = qcase(2, B=B, nQ=nQ, nKV=nKV, dim=dim, L=L, bits=8, G=64)
    rng = np.random.default_rng(5)
    kc = rng.integers(0, 256, size=(nKV, L, dim), dtype=np.uint32)
    vc = rng.integers(0, 256, size=(nKV, L, dim), dtype=np.uint32)
    c["k_packed"] = inputs.pack_codes(kc, 8)
    c["v_packed"] = inputs.pack_codes(vc, 8)
    for n in ("k_scales", "v_scales"):
        c[n][:] = np.float16(1.0)
    for n in ("k_biases", "v_biases"):
        c[n][:] = np.float16(0.0)
    c["scale"] = 1.0 / 512.0
    got = qrun(c)  # [nQ, 1, dim]
    ref = oracle.attention(c["q"][:, 0:1, :].astype(np.float32),
                           kc.astype(np.float32), vc.astype(np.float32), None,
                           n_kv_heads=nKV, kv_seq_len=L, scale=c["scale"])
    np.testing.assert_allclose(got[:, 0, :], ref[0], rtol=0, atol=1e-10)


def _brute_quant(c):
    """Dequantise everything with numpy, then softmax in matrix form."""
    bits, G = c["bits"], c["group_size"]
    pf = 32 // bits
    def deq(packed, sc, bi):
        S, N, W = packed.shape
        shifts = (np.arange(pf, dtype=np.uint32) * bits)
        codes = (packed[..., None] >> shifts) & np.uint32((1 << bits) - 1)
        codes = codes.reshape(S, N, W * pf).astype(np.float64)
        s = np.repeat(sc.astype(np.float64), G, axis=2)
        b = np.repeat(bi.astype(np.float64), G, axis=2)
        return s * codes + b
    K = deq(c["k_packed"], c["k_scales"], c["k_biases"])
    V = deq(c["v_packed"], c["v_scales"], c["v_biases"])
    BnQ, q_l, dim = c["q"].shape
    nQ = c["n_q_heads"]
    rep = nQ // c["n_kv_heads"]
    L = c["kv_seq_len"]
    out = np.zeros((BnQ, q_l, dim))
    W = c.get("window_size", 0)
    keep = np.ones((q_l, L), dtype=bool)
    if W:
        keep &= (np.arange(L) + W > L - 1)[None, :]
    for qi in range(BnQ):
        kv = qi // rep
        z = c["scale"] * (c["q"][qi].astype(np.float64) @ K[kv, :L].T)
        if c["mask"] is not None:
            z = z + c["mask"].reshape(BnQ, q_l, -1)[qi, :, :L].astype(np.float64)
        k = keep.copy()
        if c.get("mask_bool") is not None:
            k &= c["mask_bool"].reshape(BnQ, q_l, -1)[qi, :, :L] != 0
        elif c["mask"] is None and q_l > 1:
            k &= np.arange(L)[None, :] <= L - q_l + np.arange(q_l)[:, None]
        z = np.where(k, z, -np.inf)
        cols = [z]
        vals = [V[kv, :L]]
        if c["sinks"] is not None:
            cols.append(np.full((q_l, 1), float(c["sinks"][qi % nQ])))
            vals.append(np.zeros((1, dim)))
        z = np.concatenate(cols, axis=1)
        Vx = np.concatenate(vals, axis=0)
        zmax = z.max(axis=1, keepdims=True)
        live = np.isfinite(zmax[:, 0])
        w = np.exp(z - np.where(np.isfinite(zmax), zmax, 0.0))
        o = (w @ Vx) / np.where(live, w.sum(axis=1), 1.0)[:, None]
        out[qi] = np.where(live[:, None], o, 0.0)   # no visible key: zeros
    return out


@pytest.mark.parametrize("bits,G,sinks,alibi,dim", [
    (4, 32, False, False, 64), (4, 64, True, True, 64), (8, 32, True, False, 64),
    (8, 16, False, True, 64), (4, 32, True, True, 96), (8, 32, False, False, 96)])
def test_matches_brute_force(bits, G, sinks, alibi, dim):
    c = qcase(3, B=2, nQ=4, nKV=2, dim=dim, L=57, bits=bits, G=G, sinks=sinks,
              mask="alibi" if alibi else None)
    np.testing.assert_allclose(qrun(c), _brute_quant(c), rtol=0, atol=1e-12)


def test_sink_closed_form_single_key():
    # Q = 0 and one key: logit 0, so out = V0 * 1 / (1 + e^sink).
    c = qcase(4, B=1, nQ=2, nKV=1, dim=32, L=1, bits=4, G=32, sinks=True)
    c["q"][:] = np.float16(0.0)
    no_sink = qrun(c, sinks=None)
    got = qrun(c)
    for h in range(2):
        f = 1.0 / (1.0 + np.exp(np.float64(c["sinks"][h])))
        np.testing.assert_allclose(got[h, 0], no_sink[h, 0] * f, rtol=1e-14)


def test_far_negative_sink_is_no_sink():
    c = qcase(5, sinks=True)
    c["sinks"][:] = np.float32(-1e4)
    assert np.array_equal(qrun(c), qrun(c, sinks=None))


def test_sink_scales_output_by_mass_ratio():
    # O_sink = O_nosink * A / (A + e^s), A = sum of the key weights, all
    # relative to the same max; checked through two sinks on the same row.
    c = qcase(6, B=1, nQ=1, nKV=1, dim=32, L=10, bits=4, G=32, sinks=True)
    base = qrun(c, sinks=None)[0, 0]
    s1 = np.array([0.3], dtype=np.float32)
    s2 = np.array([1.7], dtype=np.float32)
    o1 = qrun(c, sinks=s1)[0, 0]
    o2 = qrun(c, sinks=s2)[0, 0]
    # base/o = 1 + e^s / A  ->  (base/o1 - 1) e^(s2 - s1) = base/o2 - 1
    idx = np.argmax(np.abs(base))
    r1 = base[idx] / o1[idx] - 1.0
    r2 = base[idx] / o2[idx] - 1.0
    np.testing.assert_allclose(
        r1 * np.exp(np.float64(s2[0]) - np.float64(s1[0])), r2, rtol=1e-10)


def test_additive_mask_shift_invariance_without_sinks():
    # Bias values on a 1/8 grid are exact in f16 before and after the shift.
    c = qcase(7, B=1, nQ=2, nKV=1, dim=32, L=30, bits=4, G=32)
    grid = np.random.default_rng(1).integers(-40, 1, size=(2, 1, 30))
    c["mask"] = (grid / 8.0).astype(np.float16)
    c["mask_head_stride"] = 30
    c["mask_stride"] = 30
    shifted = dict(c)
    shifted["mask"] = ((grid - 16) / 8.0).astype(np.float16)
    np.testing.assert_allclose(qrun(shifted), qrun(c), rtol=0, atol=1e-13)
    np.testing.assert_allclose(qrun(c), _brute_quant(c), rtol=0, atol=1e-12)
    # with a sink the shift is NOT neutral (the sink logit is not biased)
    c["sinks"] = shifted["sinks"] = np.zeros(2, dtype=np.float32)
    assert not np.allclose(qrun(shifted), qrun(c), atol=1e-6)


def test_gqa_mapping_repeat():
    # q_idx uses stream q_idx // (nQ/nKV) within its batch ([FQS] kv_idx).
    c = qcase(8, B=2, nQ=4, nKV=2, dim=32, L=20, bits=4, G=32)
    m = dict(c)
    for n in ("k_packed", "k_scales", "k_biases", "v_packed", "v_scales", "v_biases"):
        m[n] = np.repeat(c[n], 2, axis=0)  # MHA with each stream repeated
    m["n_kv_heads"] = 4
    assert np.array_equal(qrun(m), qrun(c))


def test_masked_cells_excluded_and_implicit_causal_rows():
    c = qcase(9, B=1, nQ=2, nKV=1, dim=32, L=24, q_l=3, bits=4, G=32)
    implicit = qrun(c)
    # the implicit rule as an explicit f16 mask (0 / -65504) gives the same rows
    i = np.arange(3)[:, None]
    t = np.arange(24)[None, :]
    m = np.where(t <= 24 - 3 + i, 0.0, -65504.0).astype(np.float16)
    c2 = dict(c)
    c2["mask"] = np.broadcast_to(m, (2, 3, 24)).copy()
    c2["mask_head_stride"] = 3 * 24
    c2["mask_stride"] = 24
    assert np.array_equal(qrun(c2), implicit)
    # broadcast tree mask (head stride 0) is the same thing
    c3 = dict(c)
    c3["mask"] = m.copy()
    c3["mask_head_stride"] = 0
    c3["mask_stride"] = 24
    assert np.array_equal(qrun(c3), implicit)


def test_quant_rows_selection_matches_full():
    c = qcase(10, B=2, nQ=4, nKV=2, dim=64, L=30, q_l=2, bits=8, G=64, sinks=True)
    full = qrun(c)
    rows = [(0, 0), (5, 1), (7, 0)]
    sel = qrun(c, rows=rows)
    for r, (qi, i) in enumerate(rows):
        assert np.array_equal(sel[r], full[qi, i])


# ---- bool mask and sliding window ----

@pytest.mark.parametrize("bits,G,sinks,q_l,window", [
    (4, 32, False, 1, 0), (4, 64, True, 2, 0), (8, 32, True, 1, 0),
    (8, 16, False, 3, 0), (4, 32, True, 1, 21), (8, 64, False, 2, 7)])
def test_bool_mask_matches_brute_force(bits, G, sinks, q_l, window):
    c = qcase(11, B=2, nQ=4, nKV=2, dim=64, L=57, q_l=q_l, bits=bits, G=G,
              sinks=sinks, mask="bool", window=window)
    assert c["mask_bool"].dtype == np.uint32 and (c["mask_bool"] == 0).any()
    np.testing.assert_allclose(qrun(c), _brute_quant(c), rtol=0, atol=1e-12)


def test_bool_mask_only_zero_versus_nonzero_matters():
    c = qcase(12, B=1, nQ=2, nKV=1, dim=32, L=33, q_l=2, bits=4, G=32,
              sinks=True, mask="bool")
    d = dict(c)
    d["mask_bool"] = np.where(c["mask_bool"] != 0, np.uint32(1), np.uint32(0))
    assert np.array_equal(qrun(c), qrun(d))


def test_bool_mask_all_visible_equals_no_mask_at_q_l_1():
    # q_l = 1: the implicit rule (no mask) attends every token
    c = qcase(13, B=2, nQ=4, nKV=2, dim=64, L=40, bits=8, G=64, sinks=True,
              mask="bool")
    c["mask_bool"][:] = np.uint32(7)
    assert np.array_equal(qrun(c), qrun(c, mask_bool=None))


def test_bool_mask_equals_float_mask_of_zero_and_sentinel():
    c = qcase(14, B=1, nQ=2, nKV=1, dim=32, L=29, q_l=2, bits=4, G=16,
              mask="bool")
    f = np.where(c["mask_bool"] != 0, 0.0, -65504.0).astype(np.float16)
    assert np.array_equal(qrun(c), qrun(c, mask_bool=None, mask=f))


def test_bool_mask_row_with_nothing_visible():
    # R2: no visible key gives zeros; with a sink (value zero) also zeros
    c = qcase(15, B=1, nQ=2, nKV=1, dim=32, L=20, bits=4, G=32, mask="bool")
    c["mask_bool"][1] = 0
    got = qrun(c)
    assert np.array_equal(got[1], np.zeros_like(got[1]))
    assert np.abs(got[0]).max() > 0
    got_s = qrun(c, sinks=np.array([0.5, -0.25], dtype=np.float32))
    assert np.array_equal(got_s[1], np.zeros_like(got_s[1]))


def test_window_of_one_token_is_last_value_row():
    # one visible token: softmax weight 1, so out = dequantised V[L - 1]
    c = qcase(16, B=1, nQ=2, nKV=1, dim=64, L=23, bits=4, G=32, window=1)
    got = qrun(c)
    pf, G = 8, 32
    w = c["v_packed"][0, 22]
    sc = c["v_scales"][0, 22].astype(np.float64)
    bi = c["v_biases"][0, 22].astype(np.float64)
    expect = np.array([sc[d // G] * ((int(w[d // pf]) >> ((d % pf) * 4)) & 15) + bi[d // G]
                       for d in range(64)])
    for h in range(2):
        assert np.array_equal(got[h, 0], expect)


def test_window_equals_problem_cut_to_last_tokens():
    # keeping the last W tokens is the same as a problem of W tokens that
    # start at L - W (q_l = 1, no mask, with sinks)
    L, W = 45, 13
    c = qcase(17, B=2, nQ=4, nKV=2, dim=64, L=L, bits=8, G=32, sinks=True, window=W)
    cut = dict(c)
    for name in ("k_packed", "k_scales", "k_biases", "v_packed", "v_scales", "v_biases"):
        cut[name] = np.ascontiguousarray(c[name][:, L - W:L])
    cut["kv_seq_len"] = W
    cut["window_size"] = 0
    cut["mask_stride"] = W
    np.testing.assert_allclose(qrun(c), qrun(cut), rtol=0, atol=1e-14)
    np.testing.assert_allclose(qrun(c), _brute_quant(c), rtol=0, atol=1e-12)


def test_window_not_shorter_than_sequence_is_no_window():
    c = qcase(18, B=1, nQ=2, nKV=1, dim=32, L=30, bits=4, G=32, sinks=True,
              mask="alibi")
    for W in (30, 31, 1000):
        assert np.array_equal(qrun(c, window_size=W), qrun(c))
    assert not np.array_equal(qrun(c, window_size=29), qrun(c))


# ---- element types bf16 and f32 (the page's kernels are generic in T) ----

def test_bf16_decode_known_patterns():
    # bfloat16 = the upper half of an IEEE binary32
    known = {0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x4049: 3.140625,
             0x3E80: 0.25, 0x0000: 0.0, 0x7F7F: 3.3895313892515355e38,
             0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x42F6: 123.0}
    for bits, val in known.items():
        assert oracle.bf16_to_f64(bits) == val, hex(bits)
    assert oracle.bf16_to_f64(0x7F80) == np.inf
    assert np.isnan(oracle.bf16_to_f64(0x7FC0))


def test_bf16_decode_exhaustive_against_f32_upper_half():
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):   # NaN patterns
        ref = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def _as(c, elem):
    """The same values re-expressed in another element type (exact)."""
    d = dict(c)
    for n in ("q", "k_scales", "k_biases", "v_scales", "v_biases", "mask"):
        if d.get(n) is None:
            continue
        x = np.asarray(d[n], dtype=np.float32)
        d[n] = inputs.to_bf16_bits(x) if elem == "bf16" else x.astype(np.float32)
    d["elem"] = elem
    return d


def qrun_e(c, **kw):
    return qrun(c, elem=c.get("elem", "f16"), **kw)


@pytest.mark.parametrize("elem", ["bf16", "f32"])
def test_element_types_agree_on_values_all_can_hold(elem):
    # values with 8 significant bits and a modest exponent are exact in f16,
    # bf16 and f32 alike: the three element types must give the same result
    c = qcase(30, B=1, nQ=4, nKV=2, dim=64, L=41, q_l=2, bits=4, G=32,
              sinks=True, mask="alibi")
    for n in ("q", "k_scales", "k_biases", "v_scales", "v_biases", "mask"):
        x = np.asarray(c[n], dtype=np.float32)
        x = np.where(np.abs(x) < 2.0 ** -14, 0.0, x).astype(np.float32)  # f16 normals only
        b = inputs.to_bf16_bits(x).astype(np.uint32) << np.uint32(16)
        c[n] = b.view(np.float32).astype(np.float16)    # 8 significant bits
    assert np.array_equal(qrun_e(_as(c, elem)), qrun_e(c))


@pytest.mark.parametrize("elem,bits,G", [("bf16", 4, 32), ("bf16", 8, 64), ("f32", 4, 64),
                                         ("f32", 8, 32)])
def test_element_types_match_brute_force(elem, bits, G):
    c = qcase(31, B=2, nQ=4, nKV=2, dim=64, L=53, q_l=2, bits=bits, G=G,
              sinks=True, mask="alibi")
    c = inputs.quant_case(dict(batch=2, n_q_heads=4, n_kv_heads=2, dim=64,
                               kv_seq_len=53, kv_capacity=53, q_l=2, bits=bits,
                               group_size=G, sinks=True, mask="alibi", elem=elem),
                          seed=31)
    ref = _brute_quant(_decoded(c))
    np.testing.assert_allclose(qrun_e(c), ref, rtol=0, atol=1e-12)


def _decoded(c):
    """float64 copies of the T-typed arrays for the numpy brute force."""
    d = dict(c)
    for n in ("q", "k_scales", "k_biases", "v_scales", "v_biases", "mask"):
        if d.get(n) is None:
            continue
        x = np.asarray(d[n])
        if c["elem"] == "bf16":
            x = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
        d[n] = x.astype(np.float64)
    return d
