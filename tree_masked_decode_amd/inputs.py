"""Seeded synthetic inputs for tree-masked decode attention.

This module is shared by the tests, the benchmark and the smoke check.  It
holds NO arithmetic of the method itself: it only draws random tensors, tree
topologies and the synthetic additive bias of the quantized workload, and
packs random integer codes into 32-bit words.  Both the HIP path and the CPU
oracle receive exactly these arrays.

Workloads (all seed 0, numpy ``default_rng``):

* ``tiny_chain``      H=4, Hk=2, D=128, L=cap=256, q_l=4 chain, fp32 K/V, nwg=4
* ``fixed_tree``      H=24, Hk=4, D=256, L=4096, cap=4608, q_l=16 heap-ordered
                      complete binary tree, fp16 K/V
* ``dynamic_tree_32k`` H=24, Hk=4, D=256, L=32768, cap=40960, q_l=64 random
                      tree (parent of i uniform in [max(0, i-8), i-1]),
                      fp16 K/V scaled by 0.5
* ``long_context_128k`` H=32, Hk=8, D=512, L=cap=131072, q_l=8 chain, fp16 K/V
* ``quant_4bit``      B=4, nQ=32, nKV=8, dim=128, tokens=16384, 4-bit codes,
                      group 64, f16 scales U(0.01, 0.1), biases N(0, 0.5),
                      f32 sinks N(0, 1), ALiBi-style f16 bias, f16 Q/out

Q is always N(0, 1); scale is 1/sqrt(head_dim).  Tensors are drawn one KV
head (or one KV stream) at a time so that the 2 GiB workload never needs a
full float32 copy on the host.
"""

from __future__ import annotations

import math

import numpy as np

WORKLOADS = {
    "tiny_chain": dict(n_heads=4, n_kv_heads=2, head_dim=128, kv_seq_len=256,
                       kv_capacity=256, q_l=4, tree="chain", mask_stride=256,
                       kv_dtype="f32", kv_std=1.0, nwg=4),
    "fixed_tree": dict(n_heads=24, n_kv_heads=4, head_dim=256, kv_seq_len=4096,
                       kv_capacity=4608, q_l=16, tree="binary",
                       mask_stride=4096, kv_dtype="f16", kv_std=1.0, nwg=None),
    "dynamic_tree_32k": dict(n_heads=24, n_kv_heads=4, head_dim=256,
                             kv_seq_len=32768, kv_capacity=40960, q_l=64,
                             tree="dynamic", mask_stride=32768, kv_dtype="f16",
                             kv_std=0.5, nwg=None),
    "long_context_128k": dict(n_heads=32, n_kv_heads=8, head_dim=512,
                              kv_seq_len=131072, kv_capacity=131072, q_l=8,
                              tree="chain", mask_stride=131072, kv_dtype="f16",
                              kv_std=1.0, nwg=None),
    # causal decode without a mask buffer over the last 32768 of 131072 keys
    # (implicit rule with a sliding-window start), long-context shape
    "decode_window_128k": dict(n_heads=32, n_kv_heads=8, head_dim=512,
                               kv_seq_len=131072, kv_capacity=131072, q_l=8,
                               tree="chain", mask_stride=131072, kv_dtype="f16",
                               kv_std=1.0, nwg=None, window_start=98304),
    # the same window written as an explicit mask (chain rule, keys below
    # 98304 at -65504) and sent through the masked forward
    "window_mask_128k": dict(n_heads=32, n_kv_heads=8, head_dim=512,
                             kv_seq_len=131072, kv_capacity=131072, q_l=8,
                             tree="chain", mask_stride=131072, kv_dtype="f16",
                             kv_std=1.0, nwg=None, mask_window_start=98304),
}

QUANT_WORKLOADS = {
    "quant_4bit": dict(batch=4, n_q_heads=32, n_kv_heads=8, dim=128,
                       kv_seq_len=16384, kv_capacity=16384, q_l=1, bits=4,
                       group_size=64, sinks=True, mask="alibi", nwg=None),
    # the bool-mask variant of the same decode: one u32 visibility word per
    # (query, token), 75% visible
    "quant_4bit_bool": dict(batch=4, n_q_heads=32, n_kv_heads=8, dim=128,
                            kv_seq_len=16384, kv_capacity=16384, q_l=1, bits=4,
                            group_size=64, sinks=True, mask="bool", nwg=None),
    # the same decode with 8-bit codes (4 per word)
    "quant_8bit": dict(batch=4, n_q_heads=32, n_kv_heads=8, dim=128,
                       kv_seq_len=16384, kv_capacity=16384, q_l=1, bits=8,
                       group_size=64, sinks=True, mask="alibi", nwg=None),
    # the 4-bit decode with bfloat16 / fp32 queries, scales, biases, bias and
    # output (the page's kernels are generic in that type)
    "quant_4bit_bf16": dict(batch=4, n_q_heads=32, n_kv_heads=8, dim=128,
                            kv_seq_len=16384, kv_capacity=16384, q_l=1, bits=4,
                            group_size=64, sinks=True, mask="alibi", nwg=None,
                            elem="bf16"),
    "quant_4bit_f32": dict(batch=4, n_q_heads=32, n_kv_heads=8, dim=128,
                           kv_seq_len=16384, kv_capacity=16384, q_l=1, bits=4,
                           group_size=64, sinks=True, mask="alibi", nwg=None,
                           elem="f32"),
    # sliding-window decode: only the last 4096 of 16384 tokens are attended
    "quant_4bit_window": dict(batch=4, n_q_heads=32, n_kv_heads=8, dim=128,
                              kv_seq_len=16384, kv_capacity=16384, q_l=1, bits=4,
                              group_size=64, sinks=True, mask="alibi",
                              window_size=4096, nwg=None),
}


# --------------------------------------------------------------------------
# tree topologies (parent arrays; parent[0] = -1, 0 <= parent[i] < i)
# --------------------------------------------------------------------------
def parents_chain(q_l: int) -> np.ndarray:
    """Linear chain: node i's parent is i-1."""
    return np.arange(-1, q_l - 1, dtype=np.int32)


def parents_binary(q_l: int) -> np.ndarray:
    """Complete binary tree in heap order: parent of i is (i-1)//2."""
    p = (np.arange(q_l, dtype=np.int64) - 1) // 2
    p[0] = -1
    return p.astype(np.int32)


def parents_dynamic(q_l: int, seed: int = 0, span: int = 8) -> np.ndarray:
    """Random asymmetric tree: parent of i uniform in [max(0, i-span), i-1]."""
    rng = np.random.default_rng(seed)
    p = np.empty(q_l, dtype=np.int32)
    p[0] = -1
    for i in range(1, q_l):
        p[i] = rng.integers(max(0, i - span), i)
    return p


def parents_for(kind: str, q_l: int, seed: int = 0) -> np.ndarray:
    if kind == "chain":
        return parents_chain(q_l)
    if kind == "binary":
        return parents_binary(q_l)
    if kind == "dynamic":
        return parents_dynamic(q_l, seed)
    raise ValueError("unknown tree kind %r" % kind)


# --------------------------------------------------------------------------
# fp path
# --------------------------------------------------------------------------
def _normal_heads(rng, n_heads, rows, dim, std, dtype):
    out = np.empty((n_heads, rows, dim), dtype=dtype)
    for h in range(n_heads):
        x = rng.standard_normal((rows, dim), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[h] = x.astype(dtype)
    return out


def fp_case(workload="tiny_chain", seed: int = 0, **overrides) -> dict:
    """Draw one fp-path problem.

    Returns a dict with q [H, q_l, D] f32, k/v [Hk, cap, D] (f32 or f16),
    parents [q_l] i32 and the shape parameters.  ``overrides`` replaces any
    workload field (used by the tests for small and ragged shapes).
    """
    cfg = dict(WORKLOADS[workload]) if isinstance(workload, str) else dict(workload)
    cfg.update(overrides)
    H, Hk, D = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    L, cap, q_l = cfg["kv_seq_len"], cfg["kv_capacity"], cfg["q_l"]
    if cfg.get("mask_stride") is None:
        cfg["mask_stride"] = L
    kv_dtype = np.float16 if cfg["kv_dtype"] == "f16" else np.float32
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, q_l, D), dtype=np.float32)
    std = float(cfg.get("kv_std", 1.0))
    k = _normal_heads(rng, Hk, cap, D, std, kv_dtype)
    v = _normal_heads(rng, Hk, cap, D, std, kv_dtype)
    parents = parents_for(cfg["tree"], q_l, seed)
    cfg.update(q=q, k=k, v=v, parents=parents,
               scale=float(cfg.get("scale") or 1.0 / math.sqrt(D)))
    return cfg


# --------------------------------------------------------------------------
# quantized path
# --------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack unsigned codes [..., dim] into uint32 words [..., dim*bits/32],
    element d at bits [(d % pf)*bits, +bits) of word d // pf (pf = 32/bits)."""
    pf = 32 // bits
    c = codes.astype(np.uint32).reshape(codes.shape[:-1] + (codes.shape[-1] // pf, pf))
    words = np.zeros(c.shape[:-1], dtype=np.uint32)
    for e in range(pf):
        words |= c[..., e] << np.uint32(e * bits)
    return words


def to_bf16_bits(x) -> np.ndarray:
    """float -> bfloat16 bit patterns (uint16), rounded to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def to_elem(x, elem: str) -> np.ndarray:
    """Round values to the element type of the quantized path's Q, scales,
    biases and float mask: "f16" (float16), "bf16" (uint16 bit patterns) or
    "f32" (float32)."""
    if elem == "f16":
        return np.asarray(x).astype(np.float16)
    if elem == "bf16":
        return to_bf16_bits(np.asarray(x, dtype=np.float32))
    return np.asarray(x).astype(np.float32)


def alibi_bias(n_q_heads: int, batch: int, tokens: int, q_l: int = 1,
               elem: str = "f16") -> np.ndarray:
    """Synthetic ALiBi-style additive bias [batch*nQ, q_l, tokens] in the
    element type: slope_h = 2^(-8 (h+1) / nQ), bias = slope_h * (t - (tokens
    - q_l + i))."""
    h = np.arange(n_q_heads, dtype=np.float64)
    slope = 2.0 ** (-8.0 * (h + 1.0) / n_q_heads)
    t = np.arange(tokens, dtype=np.float64)
    out = None
    for i in range(q_l):
        pos = tokens - q_l + i
        b = to_elem(slope[:, None] * (t[None, :] - pos), elem)
        if out is None:
            out = np.empty((batch * n_q_heads, q_l, tokens), dtype=b.dtype)
        out[:, i, :] = np.tile(b, (batch, 1))
    return out


def bool_mask(rows: int, q_l: int, tokens: int, rng, density: float) -> np.ndarray:
    """u32 visibility cells [rows, q_l, tokens]: each cell is visible with
    probability `density`, and a visible cell holds an arbitrary non-zero
    word (1, 0xFFFFFFFF, 0x80000000 or a random one), since only zero versus
    non-zero is meaningful."""
    vis = rng.random((rows, q_l, tokens)) < density
    words = rng.integers(1, 1 << 32, size=(rows, q_l, tokens), dtype=np.uint64)
    pick = rng.integers(0, 4, size=(rows, q_l, tokens))
    words = np.where(pick == 0, 1, np.where(pick == 1, 0xFFFFFFFF,
                                            np.where(pick == 2, 0x80000000, words)))
    return np.where(vis, words, 0).astype(np.uint32)


def quant_case(workload="quant_4bit", seed: int = 0, **overrides) -> dict:
    """Draw one affine-quantized problem (layouts of the quantized SDPA page).

    Returns q [B*nQ, q_l, dim] f16, k_packed/v_packed [B*nKV, cap, dim/pf]
    u32, k/v scales and biases [B*nKV, cap, dim/G] f16, sinks [nQ] f32 or
    None, mask f16 [B*nQ, q_l, tokens] or None, mask_bool u32 [B*nQ, q_l,
    tokens] or None (mask="bool"), window_size, and the shape parameters.
    """
    cfg = dict(QUANT_WORKLOADS[workload]) if isinstance(workload, str) else dict(workload)
    cfg.update(overrides)
    B, nQ, nKV = cfg["batch"], cfg["n_q_heads"], cfg["n_kv_heads"]
    dim, L, cap = cfg["dim"], cfg["kv_seq_len"], cfg["kv_capacity"]
    q_l, bits, G = cfg["q_l"], cfg["bits"], cfg["group_size"]
    elem = cfg.setdefault("elem", "f16")
    rng = np.random.default_rng(seed)
    q = to_elem(rng.standard_normal((B * nQ, q_l, dim), dtype=np.float32), elem)
    pf = 32 // bits
    out = {}
    for name in ("k", "v"):
        packed = np.empty((B * nKV, cap, dim // pf), dtype=np.uint32)
        edt = to_elem(np.zeros(1), elem).dtype
        scales = np.empty((B * nKV, cap, dim // G), dtype=edt)
        biases = np.empty((B * nKV, cap, dim // G), dtype=edt)
        for s in range(B * nKV):
            codes = rng.integers(0, 1 << bits, size=(cap, dim), dtype=np.uint32)
            packed[s] = pack_codes(codes, bits)
            scales[s] = to_elem(rng.uniform(0.01, 0.1, size=(cap, dim // G)), elem)
            biases[s] = to_elem(rng.normal(0.0, 0.5, size=(cap, dim // G)), elem)
        out[name + "_packed"] = packed
        out[name + "_scales"] = scales
        out[name + "_biases"] = biases
    sinks = rng.standard_normal(nQ).astype(np.float32) if cfg.get("sinks") else None
    mode = cfg.get("mask")
    if mode == "alibi":
        mask = alibi_bias(nQ, B, L, q_l, elem)
        if cfg.get("mask_stride") is None:
            cfg["mask_stride"] = L
        cfg["mask_head_stride"] = q_l * cfg["mask_stride"]
    elif mode is None or mode == "bool":
        mask = None
        cfg["mask_stride"] = L
        cfg["mask_head_stride"] = 0
    else:
        mask = mode  # caller-supplied f16 array
    mask_bool = None
    if mode == "bool":
        mask_bool = bool_mask(B * nQ, q_l, L, rng, cfg.get("bool_density", 0.75))
        cfg["mask_head_stride"] = q_l * L
    cfg.setdefault("window_size", 0)
    cfg.update(q=q, sinks=sinks, mask=mask, mask_bool=mask_bool,
               scale=float(cfg.get("scale") or 1.0 / math.sqrt(dim)), **out)
    return cfg
