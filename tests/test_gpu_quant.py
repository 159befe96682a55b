"""GPU parity of the affine-quantized K/V path against the oracle.

"ffai/flash_quantized_sdpa.rs" (metaltile-std 0.1.0): 4/8-bit codes with
per-group f16 scales and biases, optional sinks, optional additive f16 mask
or u32 visibility mask (bool-mask macro), optional sliding window.
Output is f16: each element must be within 2e-3 of the exact result plus
half an fp16 ulp of it (the rounding the f16 output type itself imposes).
"""

import numpy as np
import pytest

import oracle
from tree_masked_decode_amd import inputs

from helpers import assert_close, dev, host, note

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def ta():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import tree_masked_decode_amd as ta
    ta._api()
    return ta


def qcase(seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask, cap=None, window=0,
          elem="f16"):
    return inputs.quant_case(dict(batch=B, n_q_heads=nQ, n_kv_heads=nKV, dim=dim,
                                  kv_seq_len=L, kv_capacity=cap or (L + 5 + (L + 5) % 2), q_l=q_l,
                                  bits=bits, group_size=G, sinks=sinks, mask=mask,
                                  window_size=window, elem=elem),
                             seed=seed)


def dev_e(a, elem):
    """A T-typed array on the device (bf16 arrays hold uint16 bit patterns)."""
    import torch
    t = dev(a)
    return t.view(torch.bfloat16) if elem == "bf16" else t


def host_f(t):
    """Device result -> float64 numpy (bf16 widens exactly through fp32)."""
    import torch
    return host(t.float() if t.dtype == torch.bfloat16 else t).astype(np.float64)


def gpu_run(ta, c, nwg=None):
    import torch
    e = c.get("elem", "f16")
    t = {k: (dev(c[k]) if k.endswith("packed") else dev_e(c[k], e))
         for k in ("q", "k_packed", "k_scales", "k_biases", "v_packed", "v_scales",
                   "v_biases")}
    sinks = None if c["sinks"] is None else dev(c["sinks"])
    mask = None if c["mask"] is None else dev_e(np.ascontiguousarray(c["mask"]).ravel(), e)
    mb = c.get("mask_bool")
    mb = None if mb is None else dev(np.ascontiguousarray(mb).ravel().view(np.int32))
    out = ta.quant_verify(t["q"], t["k_packed"], t["k_scales"], t["k_biases"],
                          t["v_packed"], t["v_scales"], t["v_biases"],
                          n_kv_heads=c["n_kv_heads"], kv_seq_len=c["kv_seq_len"],
                          bits=c["bits"], group_size=c["group_size"], scale=c["scale"],
                          nwg=nwg, sinks=sinks, mask=mask, mask_bool=mb,
                          mask_head_stride=c["mask_head_stride"],
                          mask_stride=c["mask_stride"],
                          window_size=c.get("window_size", 0))
    torch.cuda.synchronize()
    return host_f(out)


def ref_run(c, rows=None):
    return oracle.quant_attention(
        c["q"], c["k_packed"], c["k_scales"], c["k_biases"], c["v_packed"],
        c["v_scales"], c["v_biases"], n_kv_heads=c["n_kv_heads"],
        kv_seq_len=c["kv_seq_len"], bits=c["bits"], group_size=c["group_size"],
        scale=c["scale"], sinks=c["sinks"],
        mask=None if c["mask"] is None else np.ascontiguousarray(c["mask"]).ravel(),
        mask_bool=None if c.get("mask_bool") is None else np.ascontiguousarray(c["mask_bool"]).ravel(),
        mask_head_stride=c["mask_head_stride"], mask_stride=c["mask_stride"],
        window_size=c.get("window_size", 0), elem=c.get("elem", "f16"), rows=rows)


SMALL = [
    # seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask, nwg
    (0, 1, 4, 1, 128, 100, 1, 4, 64, False, None, 1),
    (1, 2, 8, 2, 128, 333, 1, 4, 64, True, "alibi", 3),
    (2, 1, 4, 4, 64, 257, 1, 8, 32, True, None, 2),
    (3, 2, 6, 2, 256, 190, 1, 4, 128, False, "alibi", None),
    (4, 1, 8, 2, 128, 500, 1, 8, 64, True, "alibi", 4),
    (5, 1, 2, 1, 512, 97, 1, 4, 32, True, None, 2),
    (6, 1, 2, 2, 512, 65, 1, 8, 128, False, "alibi", 1),
    (7, 1, 4, 2, 64, 1000, 3, 4, 64, False, None, 5),      # implicit causal, q_l = 3
    (8, 3, 4, 1, 128, 77, 5, 4, 32, True, "alibi", 2),     # 20 rows: 2 row tiles
    (9, 1, 2, 1, 128, 40, 1, 4, 64, False, None, 9),       # more splits than tiles
    (10, 1, 2, 1, 64, 101, 1, 4, 64, True, "alibi", 2),   # one group per token
    (11, 2, 4, 2, 64, 99, 2, 8, 64, False, None, 3),
    (12, 1, 4, 1, 96, 333, 1, 4, 32, True, "alibi", 3),    # 1.5 KB K/V tiles
    (13, 2, 4, 2, 96, 190, 2, 8, 32, False, None, 2),
    (14, 3, 8, 2, 96, 1000, 1, 4, 32, True, None, None),
]


@pytest.mark.parametrize("seed,B,nQ,nKV,dim,L,q_l,bits,G,sinks,mask,nwg", SMALL)
def test_quant_parity_small(ta, seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask, nwg):
    note("quant small seed=%d dim=%d L=%d q_l=%d bits=%d G=%d sinks=%s mask=%s nwg=%s"
         % (seed, dim, L, q_l, bits, G, sinks, mask, nwg))
    c = qcase(seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask)
    assert_close(gpu_run(ta, c, nwg), ref_run(c), TOL, "quant %d" % seed, f16_out=True)


def test_quant_workload_4bit(ta):
    note("workload quant_4bit (full)")
    c = inputs.quant_case("quant_4bit", f16_out=True)
    got = gpu_run(ta, c)
    assert_close(got, ref_run(c), TOL, "quant_4bit", f16_out=True)


def test_quant_workload_8bit_sampled(ta):
    note("workload quant_4bit shape at 8 bits (sampled rows)")
    c = inputs.quant_case("quant_4bit", bits=8)
    got = gpu_run(ta, c)
    rows = [(qi, 0) for qi in (0, 1, 31, 32, 64, 100, 127)]
    sel = np.stack([got[qi, i] for qi, i in rows])
    assert_close(sel, ref_run(c, rows), TOL, "quant_8bit", f16_out=True)


def test_quant_tree_mask_broadcast(ta):
    note("quant with a broadcast tree mask (q_l = 16, head stride 0)")
    c = qcase(10, 1, 8, 2, 128, 600, 16, 4, 64, True, None)
    tm = oracle.tree_mask(inputs.parents_binary(16), 600).astype(np.float16)
    c["mask"] = tm
    c["mask_head_stride"] = 0
    c["mask_stride"] = 600
    assert_close(gpu_run(ta, c, 3), ref_run(c), TOL, "tree mask", f16_out=True)


def test_quant_masked_rows_and_poison(ta):
    note("quant masked rows + poisoned capacity tail")
    c = qcase(11, 1, 4, 1, 128, 300, 2, 4, 64, True, None, cap=400)
    m = np.zeros((4, 2, 300), dtype=np.float16)
    m[1, 1, :] = -65504.0        # row with no visible key -> sink only -> zeros
    m[2, :, :250] = -np.inf      # -inf excludes as well
    c["mask"] = m
    c["mask_head_stride"] = 600
    c["mask_stride"] = 300
    ref = ref_run(c)
    got = gpu_run(ta, c, 4)
    assert np.all(got[1, 1] == 0.0)
    assert_close(got, ref, TOL, "masked", f16_out=True)
    # scales/biases past kv_seq_len -> NaN must not leak
    for k in ("k_scales", "k_biases", "v_scales", "v_biases"):
        c[k] = c[k].copy()
        c[k][:, 300:] = np.nan
    got2 = gpu_run(ta, c, 4)
    assert np.array_equal(got2.view(np.uint16), got.view(np.uint16))


def test_quant_deterministic(ta):
    note("quant determinism")
    c = qcase(12, 2, 8, 2, 128, 2000, 1, 4, 64, True, "alibi")
    a = gpu_run(ta, c)
    b = gpu_run(ta, c)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


# ---- u32 visibility mask and sliding window ----

GATED = [
    # seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask, window, nwg
    (20, 1, 4, 1, 128, 100, 1, 4, 64, False, "bool", 0, 1),
    (21, 2, 8, 2, 128, 333, 1, 4, 64, True, "bool", 0, 3),
    (22, 1, 4, 4, 64, 257, 1, 8, 32, True, "bool", 0, 2),
    (23, 2, 6, 2, 256, 190, 1, 4, 128, False, "bool", 0, None),
    (24, 1, 2, 1, 512, 97, 1, 8, 32, True, "bool", 0, 2),
    (25, 3, 4, 1, 128, 77, 5, 4, 32, True, "bool", 0, 2),      # 20 rows: 2 row tiles
    (26, 1, 2, 1, 64, 101, 2, 8, 64, False, "bool", 0, 9),     # splits past the tiles
    (27, 1, 4, 1, 128, 500, 1, 4, 64, True, "alibi", 1, None),  # one token
    (28, 1, 4, 1, 128, 500, 1, 4, 64, False, None, 31, 2),     # window inside one tile
    (29, 1, 4, 1, 128, 500, 1, 8, 64, True, "bool", 33, 3),    # window crosses a tile edge
    (30, 2, 4, 2, 64, 1000, 1, 4, 32, True, "alibi", 320, 4),  # window on tile edges
    (31, 1, 2, 1, 256, 333, 3, 4, 64, False, "bool", 100, 2),
    (32, 1, 4, 1, 128, 300, 1, 4, 64, True, "alibi", 299, 5),  # one token short of all
    (33, 1, 4, 1, 128, 300, 1, 4, 64, True, None, 300, 5),     # window == L: no window
    (34, 1, 4, 1, 128, 300, 1, 4, 64, True, "bool", 5000, 5),  # window > L
    (35, 1, 2, 1, 512, 161, 2, 4, 128, True, None, 70, 3),
    (38, 1, 4, 2, 96, 300, 1, 4, 32, True, "bool", 0, 2),
    (39, 1, 4, 1, 96, 500, 1, 8, 32, False, "alibi", 77, 3),
]


@pytest.mark.parametrize("seed,B,nQ,nKV,dim,L,q_l,bits,G,sinks,mask,window,nwg", GATED)
def test_quant_gated_parity(ta, seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask,
                            window, nwg):
    note("quant gated seed=%d dim=%d L=%d q_l=%d bits=%d G=%d sinks=%s mask=%s W=%d nwg=%s"
         % (seed, dim, L, q_l, bits, G, sinks, mask, window, nwg))
    c = qcase(seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask, window=window)
    assert_close(gpu_run(ta, c, nwg), ref_run(c), TOL, "gated %d" % seed, f16_out=True)


def test_quant_workload_bool(ta):
    note("workload quant_4bit_bool (full)")
    c = inputs.quant_case("quant_4bit_bool")
    assert_close(gpu_run(ta, c), ref_run(c), TOL, "quant_4bit_bool", f16_out=True)


def test_quant_workload_window(ta):
    note("workload quant_4bit_window (full)")
    c = inputs.quant_case("quant_4bit_window")
    assert_close(gpu_run(ta, c), ref_run(c), TOL, "quant_4bit_window", f16_out=True)


@pytest.mark.parametrize("L", [203, 204])   # 4-byte and 16-byte mask copies
def test_quant_bool_edge_rows_and_tail_cells(ta, L):
    note("quant bool mask: empty rows, high-bit words, garbage past kv_seq_len, L=%d" % L)
    stride = 256
    c = qcase(36, 1, 4, 1, 128, L, 2, 4, 64, True, "bool")
    mb = np.zeros((4, 2, stride), dtype=np.uint32)
    mb[:, :, :L] = c["mask_bool"]
    mb[:, :, L:] = 0xFFFFFFFF          # never read
    mb[1, 0, :] = 0                    # nothing visible: zeros (the sink value is 0)
    mb[2, 1, :L] = 0x80000000          # only the top bit set: visible
    c["mask_bool"] = mb
    c["mask_stride"] = stride
    c["mask_head_stride"] = 2 * stride
    got = gpu_run(ta, c, 3)
    assert np.all(got[1, 0] == 0.0)
    assert_close(got, ref_run(c), TOL, "bool edges", f16_out=True)


def test_quant_ex_entry_matches_plain_entry(ta):
    note("quant: forward_ex(F16, no window) is the plain entry, byte for byte")
    import torch
    c = qcase(37, 2, 8, 2, 128, 700, 1, 4, 64, True, "alibi")
    t = {k: dev(c[k]) for k in ("q", "k_packed", "k_scales", "k_biases", "v_packed",
                                "v_scales", "v_biases")}
    mask = dev(np.ascontiguousarray(c["mask"]).ravel())
    sinks = dev(c["sinks"])
    args = (t["q"], t["k_packed"], t["k_scales"], t["k_biases"], t["v_packed"],
            t["v_scales"], t["v_biases"])
    kw = dict(n_kv_heads=2, kv_seq_len=700, bits=4, group_size=64, scale=c["scale"],
              nwg=1, sinks=sinks, mask=mask, mask_head_stride=c["mask_head_stride"],
              mask_stride=c["mask_stride"])
    o1 = torch.empty((16, 1, 128), dtype=torch.float16, device="cuda")
    o2 = torch.empty_like(o1)
    ta.tree_attn_quant_forward(*args, out=o1, **kw)
    ta.tree_attn_quant_forward_ex(*args, out=o2, mask_kind=ta.TA_MASK_F16,
                                  window_size=0, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ---- bf16 and fp32 element types ----

ELEM = [
    # seed, elem, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask, window, nwg
    (60, "bf16", 1, 4, 1, 128, 100, 1, 4, 64, False, None, 0, 1),       # direct bf16 out
    (61, "bf16", 2, 8, 2, 128, 333, 1, 4, 64, True, "alibi", 0, 3),
    (62, "bf16", 1, 4, 4, 64, 257, 2, 8, 32, True, "bool", 0, 2),
    (63, "bf16", 2, 6, 2, 256, 190, 1, 4, 128, False, "alibi", 0, None),
    (64, "bf16", 1, 2, 1, 512, 97, 1, 8, 32, True, None, 0, 2),
    (65, "bf16", 1, 4, 2, 96, 300, 1, 4, 32, True, "alibi", 77, 3),
    (66, "bf16", 1, 2, 1, 64, 101, 1, 4, 64, True, "alibi", 0, 2),      # one group per token
    (70, "f32", 1, 4, 1, 128, 100, 1, 4, 64, False, None, 0, 1),        # direct f32 out
    (71, "f32", 2, 8, 2, 128, 333, 1, 4, 64, True, "alibi", 0, 3),
    (72, "f32", 1, 4, 4, 64, 257, 2, 8, 32, True, "bool", 0, 2),
    (73, "f32", 2, 6, 2, 256, 190, 1, 4, 32, False, "alibi", 0, None),  # 4-byte mask copies
    (74, "f32", 1, 2, 1, 512, 97, 1, 8, 32, True, "alibi", 0, 2),       # 16-byte scale copies
    (75, "f32", 1, 4, 2, 96, 300, 3, 4, 32, True, None, 77, 3),
    (76, "f32", 1, 2, 1, 64, 101, 1, 4, 64, True, "alibi", 0, 2),
]


@pytest.mark.parametrize("seed,elem,B,nQ,nKV,dim,L,q_l,bits,G,sinks,mask,window,nwg", ELEM)
def test_quant_element_types(ta, seed, elem, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask,
                             window, nwg):
    note("quant %s seed=%d dim=%d L=%d q_l=%d bits=%d G=%d sinks=%s mask=%s W=%d nwg=%s"
         % (elem, seed, dim, L, q_l, bits, G, sinks, mask, window, nwg))
    c = qcase(seed, B, nQ, nKV, dim, L, q_l, bits, G, sinks, mask, window=window, elem=elem)
    assert_close(gpu_run(ta, c, nwg), ref_run(c), TOL, "%s %d" % (elem, seed), out_elem=elem)


@pytest.mark.parametrize("name", ["quant_4bit_bf16", "quant_4bit_f32"])
def test_quant_workload_element_types(ta, name):
    note("workload %s (full)" % name)
    c = inputs.quant_case(name)
    assert_close(gpu_run(ta, c), ref_run(c), TOL, name, out_elem=c["elem"])
