"""tree_masked_decode_amd -- tree-masked decode attention for AMD MI355X.

Python face of libtreeattn.so (C ABI: include/tree_attn.h).  The functions
below only marshal torch tensors (device memory) and torch's current HIP
stream into the C entry points of the same names; every step of the path
runs in the library's HIP kernels.  There is no CPU or PyTorch fallback: if
the library is missing or a call fails, an exception is raised.

Sources: "tree_attention.metal" (mlx-native 0.9.1), "ops/tree_attention.rs"
(mlx-native 0.9.2) and "ffai/flash_quantized_sdpa.rs" (metaltile-std 0.1.0).
The ``inputs`` submodule (seeded synthetic workloads) does not load the
library.
"""

from __future__ import annotations

import ctypes

MASKED = -65504.0   # mask cell that excludes a key ("ops/tree_attention.rs")
ATTENDED = 0.0
TA_F32 = 0
TA_F16 = 1
TA_BF16 = 2
TA_MASK_NONE = 0
TA_MASK_F16 = 1
TA_MASK_BOOL = 2

__all__ = [
    "MASKED", "ATTENDED", "TreeAttnError", "partials_bytes", "pick_nwg",
    "quant_pick_nwg", "tree_attn_forward", "tree_attn_reduce",
    "tree_attn_quant_forward", "tree_attn_quant_forward_ex", "build_tree_mask",
    "tree_attn_decode", "tree_attn_forward_noalloc", "verify", "decode", "quant_verify",
]


class TreeAttnError(RuntimeError):
    """A C entry point returned an error code (message from the library)."""

    def __init__(self, code, message):
        super().__init__("%s (code %d)" % (message, code))
        self.code = code


def _api():
    from . import _lib as L
    return L.load()


def _check(rc):
    if rc != 0:
        from . import _lib as L
        raise TreeAttnError(rc, L.last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dense(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _kv_dtype(t):
    import torch
    if t.dtype == torch.float16:
        return TA_F16
    if t.dtype == torch.float32:
        return TA_F32
    raise TreeAttnError(-4, "k/v dtype must be float32 or float16, got %s" % t.dtype)


def _elem_dtype(t):
    """TA_* code of a quantized-path element tensor (queries, scales, biases,
    float mask, output): float16, bfloat16 or float32; -1 otherwise (the
    library then rejects the call)."""
    import torch
    return {torch.float16: TA_F16, torch.bfloat16: TA_BF16,
            torch.float32: TA_F32}.get(t.dtype, -1)


def partials_bytes(n_heads, head_dim, q_l, nwg) -> int:
    return int(_api().tree_attn_partials_bytes(n_heads, head_dim, q_l, nwg))


def pick_nwg(n_heads, n_kv_heads, head_dim, kv_seq_len, q_l, kv_dtype,
             num_cus=0) -> int:
    return int(_api().tree_attn_pick_nwg(n_heads, n_kv_heads, head_dim,
                                         kv_seq_len, q_l, kv_dtype, num_cus))


def quant_pick_nwg(batch, n_q_heads, n_kv_heads, dim, kv_seq_len, q_l,
                   num_cus=0, bits=None, group_size=None, mask_kind=None,
                   q_dtype=TA_F16) -> int:
    """Split count for the quantized forward; with bits, group_size and
    mask_kind it accounts for how many workgroups of that variant fit a CU
    (tree_attn_quant_pick_nwg_ex)."""
    if bits is None:
        return int(_api().tree_attn_quant_pick_nwg(batch, n_q_heads, n_kv_heads,
                                                   dim, kv_seq_len, q_l, num_cus))
    return int(_api().tree_attn_quant_pick_nwg_ex(
        batch, n_q_heads, n_kv_heads, dim, kv_seq_len, q_l, bits, group_size,
        TA_MASK_F16 if mask_kind is None else mask_kind, q_dtype, num_cus))


def tree_attn_forward(q, k, v, mask, *, kv_seq_len, scale, nwg, out=None,
                      partials=None, mask_stride=None, stream=None):
    """Forward pass.  q [H, q_l, D] f32; k, v [Hk, cap, D] f32/f16; mask
    [q_l, stride] f32 or None (implicit causal).  nwg == 1 writes ``out``
    ([q_l, H, D] f32); nwg > 1 writes ``partials`` (flat f32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (mask, "mask"), (out, "out"),
                 (partials, "partials")):
        _dense(t, n)
    H, q_l, D = q.shape
    Hk, cap, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or v.dtype != k.dtype or Dk != D:
        raise ValueError("k and v must share shape and dtype, head_dim must match q")
    if mask is not None and mask_stride is None:
        mask_stride = mask.shape[-1]
    rc = _api().tree_attn_forward(
        _ptr(q), _nbytes(q), _ptr(k), _ptr(v), _kv_dtype(k), _nbytes(k),
        _ptr(mask), _nbytes(mask), _ptr(partials), _nbytes(partials),
        _ptr(out), _nbytes(out), H, Hk, D, kv_seq_len, cap, q_l,
        mask_stride or 0, float(scale), nwg, _stream(stream))
    _check(rc)


def tree_attn_reduce(partials, out, *, nrows, head_dim, nwg, stream=None):
    """Merge split partials into ``out`` ([nrows, head_dim], f32 or f16)."""
    import torch
    _dense(partials, "partials")
    _dense(out, "out")
    out_dtype = _elem_dtype(out)
    rc = _api().tree_attn_reduce(_ptr(partials), _nbytes(partials), _ptr(out),
                                 out_dtype, _nbytes(out), nrows, head_dim, nwg,
                                 _stream(stream))
    _check(rc)


NOALLOC_SCRATCH_BYTES = 64 << 20
# Tail after the partials that tree_attn_forward may use for the live-key
# scan of an explicit mask (TA_RANGE_BYTES).
RANGE_BYTES = 2048


def tree_attn_forward_noalloc(q, k, v, mask, *, kv_seq_len, scale, nwg, out,
                              mask_stride=None, stream=None):
    """Forward plus merge into ``out`` ([q_l, H, D] f32) with the split
    partials in the library's static device buffer (no allocation in the
    call).  Calls that overlap on one GPU race on that buffer."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (mask, "mask"), (out, "out")):
        _dense(t, n)
    H, q_l, D = q.shape
    Hk, cap, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or v.dtype != k.dtype or Dk != D:
        raise ValueError("k and v must share shape and dtype, head_dim must match q")
    if mask is not None and mask_stride is None:
        mask_stride = mask.shape[-1]
    rc = _api().tree_attn_forward_noalloc(
        _ptr(q), _nbytes(q), _ptr(k), _ptr(v), _kv_dtype(k), _nbytes(k),
        _ptr(mask), _nbytes(mask), _ptr(out), _nbytes(out), H, Hk, D, kv_seq_len,
        cap, q_l, mask_stride or 0, float(scale), nwg, _stream(stream))
    _check(rc)


def build_tree_mask(parents, kv_seq_len, mask_stride=None, *, out=None,
                    device=None, stream=None):
    """Explicit [q_l, mask_stride] f32 mask built on the device from a host
    parent array (parents[0] = -1, 0 <= parents[i] < i)."""
    import numpy as np
    import torch
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    q_l = int(par.shape[0])
    stride = int(mask_stride or kv_seq_len)
    if out is None:
        out = torch.empty((q_l, stride), dtype=torch.float32,
                          device=device or "cuda")
    _dense(out, "out")
    rc = _api().build_tree_mask(par.ctypes.data_as(ctypes.c_void_p), q_l,
                                kv_seq_len, stride, _ptr(out), _nbytes(out),
                                _stream(stream))
    _check(rc)
    return out


def tree_attn_decode(q, k, v, *, kv_seq_len, scale, nwg, window_start=0,
                     out=None, partials=None, stream=None):
    """Causal decode with a sliding-window start (no mask buffer).  q [H,
    q_l, D] f32; k, v [Hk, cap, D] f32/f16.  nwg == 1 writes ``out`` ([q_l,
    H, D] f32); nwg > 1 writes ``partials``."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (partials, "partials")):
        _dense(t, n)
    H, q_l, D = q.shape
    Hk, cap, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or v.dtype != k.dtype or Dk != D:
        raise ValueError("k and v must share shape and dtype, head_dim must match q")
    rc = _api().tree_attn_decode(
        _ptr(q), _nbytes(q), _ptr(k), _ptr(v), _kv_dtype(k), _nbytes(k),
        _ptr(partials), _nbytes(partials), _ptr(out), _nbytes(out), H, Hk, D,
        kv_seq_len, cap, q_l, int(window_start), float(scale), nwg, _stream(stream))
    _check(rc)


def decode(q, k, v, *, kv_seq_len, scale, window_start=0, nwg=None, out=None,
           partials=None, stream=None):
    """Causal (sliding-window) decode plus the merge; returns ``out``
    [q_l, H, D] f32."""
    import torch
    H, q_l, D = q.shape
    if nwg is None:
        nwg = pick_nwg(H, k.shape[0], D, kv_seq_len - window_start, q_l, _kv_dtype(k))
    if out is None:
        out = torch.empty((q_l, H, D), dtype=torch.float32, device=q.device)
    if nwg > 1 and partials is None:
        partials = torch.empty(partials_bytes(H, D, q_l, nwg) // 4,
                               dtype=torch.float32, device=q.device)
    tree_attn_decode(q, k, v, kv_seq_len=kv_seq_len, scale=scale, nwg=nwg,
                     window_start=window_start, out=out if nwg == 1 else None,
                     partials=partials if nwg > 1 else None, stream=stream)
    if nwg > 1:
        tree_attn_reduce(partials, out, nrows=H * q_l, head_dim=D, nwg=nwg,
                         stream=stream)
    return out


def verify(q, k, v, mask, *, kv_seq_len, scale, nwg=None, out=None,
           partials=None, mask_stride=None, stream=None):
    """One tree-verify call: forward, then the merge when nwg > 1.
    Returns ``out`` [q_l, H, D] f32."""
    import torch
    H, q_l, D = q.shape
    if nwg is None:
        nwg = pick_nwg(H, k.shape[0], D, kv_seq_len, q_l, _kv_dtype(k))
    if out is None:
        out = torch.empty((q_l, H, D), dtype=torch.float32, device=q.device)
    if nwg > 1 and partials is None:
        # (with the live-key scan's tail: see RANGE_BYTES)
        partials = torch.empty((partials_bytes(H, D, q_l, nwg) + RANGE_BYTES) // 4,
                               dtype=torch.float32, device=q.device)
    tree_attn_forward(q, k, v, mask, kv_seq_len=kv_seq_len, scale=scale,
                      nwg=nwg, out=out if nwg == 1 else None,
                      partials=partials if nwg > 1 else None,
                      mask_stride=mask_stride, stream=stream)
    if nwg > 1:
        tree_attn_reduce(partials, out, nrows=H * q_l, head_dim=D, nwg=nwg,
                         stream=stream)
    return out


def tree_attn_quant_forward(q, k_packed, k_scales, k_biases, v_packed,
                            v_scales, v_biases, *, n_kv_heads, kv_seq_len,
                            bits, group_size, scale, nwg, sinks=None,
                            mask=None, mask_head_stride=0, mask_stride=None,
                            out=None, partials=None, stream=None):
    """Quantized forward.  q [B*nQ, q_l, dim] f16; packed [B*nKV, cap,
    dim/(32/bits)] int32/uint32 bits; scales/biases [B*nKV, cap, dim/G] f16;
    sinks [nQ] f32 or None; mask flat f16 or None."""
    bufs = (q, k_packed, k_scales, k_biases, v_packed, v_scales, v_biases,
            sinks, mask, out, partials)
    for t in bufs:
        _dense(t, "buffer")
    BnQ, q_l, dim = q.shape
    BnKV, cap, _ = k_packed.shape
    batch = BnKV // n_kv_heads
    nq = BnQ // batch
    kvb = (ctypes.c_size_t * 6)(*[_nbytes(t) for t in (
        k_packed, k_scales, k_biases, v_packed, v_scales, v_biases)])
    rc = _api().tree_attn_quant_forward(
        _ptr(q), _elem_dtype(q),
        _nbytes(q), _ptr(k_packed), _ptr(k_scales), _ptr(k_biases),
        _ptr(v_packed), _ptr(v_scales), _ptr(v_biases), kvb, _ptr(sinks),
        _nbytes(sinks), _ptr(mask), _nbytes(mask), int(mask_head_stride),
        int(mask_stride or kv_seq_len), _ptr(partials), _nbytes(partials),
        _ptr(out), _nbytes(out), batch, nq, n_kv_heads, dim, kv_seq_len, cap,
        q_l, bits, group_size, float(scale), nwg, _stream(stream))
    _check(rc)


def tree_attn_quant_forward_ex(q, k_packed, k_scales, k_biases, v_packed,
                               v_scales, v_biases, *, n_kv_heads, kv_seq_len,
                               bits, group_size, scale, nwg, sinks=None,
                               mask=None, mask_kind=None, mask_head_stride=0,
                               mask_stride=None, window_size=0, out=None,
                               partials=None, stream=None):
    """Quantized forward with a mask kind (TA_MASK_NONE / TA_MASK_F16 /
    TA_MASK_BOOL; default: F16 for an f16 tensor, BOOL for a 4-byte integer
    tensor) and a sliding window (0 = none)."""
    bufs = (q, k_packed, k_scales, k_biases, v_packed, v_scales, v_biases,
            sinks, mask, out, partials)
    for t in bufs:
        _dense(t, "buffer")
    if mask_kind is None:
        mask_kind = (TA_MASK_NONE if mask is None else
                     TA_MASK_F16 if mask.is_floating_point() else TA_MASK_BOOL)
    BnQ, q_l, dim = q.shape
    BnKV, cap, _ = k_packed.shape
    batch = BnKV // n_kv_heads
    nq = BnQ // batch
    kvb = (ctypes.c_size_t * 6)(*[_nbytes(t) for t in (
        k_packed, k_scales, k_biases, v_packed, v_scales, v_biases)])
    rc = _api().tree_attn_quant_forward_ex(
        _ptr(q), _elem_dtype(q),
        _nbytes(q), _ptr(k_packed), _ptr(k_scales), _ptr(k_biases),
        _ptr(v_packed), _ptr(v_scales), _ptr(v_biases), kvb, _ptr(sinks),
        _nbytes(sinks), _ptr(mask), int(mask_kind), _nbytes(mask),
        int(mask_head_stride), int(mask_stride or kv_seq_len), int(window_size),
        _ptr(partials), _nbytes(partials), _ptr(out), _nbytes(out), batch, nq,
        n_kv_heads, dim, kv_seq_len, cap, q_l, bits, group_size, float(scale), nwg,
        _stream(stream))
    _check(rc)


def quant_verify(q, k_packed, k_scales, k_biases, v_packed, v_scales,
                 v_biases, *, n_kv_heads, kv_seq_len, bits, group_size, scale,
                 nwg=None, sinks=None, mask=None, mask_bool=None,
                 mask_head_stride=0, mask_stride=None, window_size=0, out=None,
                 partials=None, stream=None):
    """Quantized forward plus merge; returns ``out`` [B*nQ, q_l, dim] f16.
    ``mask`` is an f16 additive bias, ``mask_bool`` u32 visibility words
    (at most one); ``window_size`` > 0 keeps the last window_size tokens."""
    import torch
    BnQ, q_l, dim = q.shape
    BnKV = k_packed.shape[0]
    batch = BnKV // n_kv_heads
    if mask is not None and mask_bool is not None:
        raise ValueError("quant_verify: give at most one of mask and mask_bool")
    if nwg is None:
        span = min(window_size, kv_seq_len) if window_size else kv_seq_len
        kind = (TA_MASK_BOOL if mask_bool is not None else
                TA_MASK_F16 if mask is not None else TA_MASK_NONE)
        nwg = quant_pick_nwg(batch, BnQ // batch, n_kv_heads, dim, span, q_l,
                             bits=bits, group_size=group_size, mask_kind=kind,
                             q_dtype=_elem_dtype(q))
    if out is None:
        out = torch.empty((BnQ, q_l, dim), dtype=q.dtype, device=q.device)
    if nwg > 1 and partials is None:
        partials = torch.empty(partials_bytes(BnQ, dim, q_l, nwg) // 4,
                               dtype=torch.float32, device=q.device)
    common = dict(n_kv_heads=n_kv_heads, kv_seq_len=kv_seq_len, bits=bits,
                  group_size=group_size, scale=scale, nwg=nwg, sinks=sinks,
                  mask_head_stride=mask_head_stride, mask_stride=mask_stride,
                  out=out if nwg == 1 else None,
                  partials=partials if nwg > 1 else None, stream=stream)
    if mask_bool is None and not window_size:
        tree_attn_quant_forward(q, k_packed, k_scales, k_biases, v_packed,
                                v_scales, v_biases, mask=mask, **common)
    else:
        m = mask_bool if mask_bool is not None else mask
        kind = (TA_MASK_BOOL if mask_bool is not None else
                TA_MASK_F16 if mask is not None else TA_MASK_NONE)
        tree_attn_quant_forward_ex(q, k_packed, k_scales, k_biases, v_packed,
                                   v_scales, v_biases, mask=m, mask_kind=kind,
                                   window_size=window_size, **common)
    if nwg > 1:
        tree_attn_reduce(partials, out, nrows=BnQ * q_l, head_dim=dim, nwg=nwg,
                         stream=stream)
    return out
