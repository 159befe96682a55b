"""CPU oracle for tree-masked decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or runs it, and it shares no code
with that path.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, plain loops,
direct two-pass softmax); this module only marshals numpy arrays into it.
Each function cites the page and section it follows:

* "tree_attention.metal" (mlx-native 0.9.1) -- header comment and
  ``tree_attention_impl``: explicit-mask attention, implicit causal rule.
* "ops/tree_attention.rs" (mlx-native 0.9.2) -- mask constants, buffer
  layouts (output is query-outer, head-inner).
* "ffai/flash_quantized_sdpa.rs" (metaltile-std 0.1.0) -- affine dequant,
  sinks, additive float mask.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, invariants, the pages' printed constants); none
is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

MASKED = -65504.0  # "ops/tree_attention.rs", mask constants (-MAXHALF)
ATTENDED = 0.0


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc -O2 (never fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or (
        os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", "-std=c11", "-Wall", "-o", tmp, _SRC,
               "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # A test may point the wrapper at a deliberately broken build of
            # oracle.c to check that the pins catch the mistake.
            path = os.environ.get("TREEATTN_ORACLE_LIB")
            if not path:
                path = build()
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            U = ctypes.c_uint32
            lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_f16_to_f64.restype = ctypes.c_double
            lib.orc_tree_mask.argtypes = [P, U, U, U, P]
            lib.orc_tree_mask.restype = ctypes.c_int
            lib.orc_attention.argtypes = [P, P, P, ctypes.c_int, P, U, U, U, U,
                                          U, U, U, ctypes.c_double, P, U, P,
                                          ctypes.c_int]
            lib.orc_attention.restype = ctypes.c_int
            lib.orc_attention_ex.argtypes = [P, P, P, ctypes.c_int, P, U, U, U, U,
                                             U, U, U, ctypes.c_double, U, P, U, P,
                                             ctypes.c_int]
            lib.orc_attention_ex.restype = ctypes.c_int
            lib.orc_attention_partials.argtypes = [P, P, P, ctypes.c_int, P, U,
                                                   U, U, U, U, U, U,
                                                   ctypes.c_double, P, U, P, P,
                                                   P, ctypes.c_int]
            lib.orc_attention_partials.restype = ctypes.c_int
            lib.orc_lse_combine.argtypes = [P, P, P, U, U, U, P]
            lib.orc_lse_combine.restype = ctypes.c_int
            lib.orc_quant_attention.argtypes = [P, P, P, P, P, P, P, P, P,
                                                ctypes.c_uint64, U, U, U, U, U,
                                                U, U, U, U, U, ctypes.c_double,
                                                P, U, P, ctypes.c_int]
            lib.orc_quant_attention.restype = ctypes.c_int
            lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_bf16_to_f64.restype = ctypes.c_double
            lib.orc_quant_attention_ex.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, P, P, P,
                                                   ctypes.c_uint64, U, U, U, U,
                                                   U, U, U, U, U, U, U,
                                                   ctypes.c_double, P, U, P,
                                                   ctypes.c_int]
            lib.orc_quant_attention_ex.restype = ctypes.c_int
            _lib = lib
    return _lib


def _threads(n):
    if n is not None:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class OracleError(ValueError):
    pass


def f16_to_f64(bits: int) -> float:
    """Exact binary16 decode from the bit pattern (used for every f16 input)."""
    return _load().orc_f16_to_f64(int(bits) & 0xFFFF)


def tree_mask(parents, kv_seq_len: int, mask_stride: int | None = None):
    """Explicit [q_l, mask_stride] f32 mask from a parent array.

    "tree_attention.metal" header: every tree shape reduces to such a mask,
    0 = attended, -65504 = masked.  Node i is at position
    kv_seq_len - q_l + i; it sees the whole prefix, its ancestors and itself.
    """
    parents = _c(parents, np.int32)
    q_l = parents.shape[0]
    stride = kv_seq_len if mask_stride is None else int(mask_stride)
    out = np.empty((q_l, stride), dtype=np.float32)
    rc = _load().orc_tree_mask(_ptr(parents), q_l, kv_seq_len, stride, _ptr(out))
    if rc != 0:
        raise OracleError("invalid tree topology or sizes")
    return out


def attention(q, k, v, mask, *, n_kv_heads, kv_seq_len, scale, mask_stride=None,
              window_start=0, rows=None, nthreads=None):
    """fp-path attention in double ("tree_attention.metal", impl; reading R1/R2).

    q: [n_heads, q_l, D] float32.  k, v: [n_kv_heads, kv_capacity, D], float32
    or float16.  mask: [q_l, mask_stride] float32 or None (implicit causal;
    with window_start, row i sees keys window_start .. kv_seq_len - q_l + i,
    the "tree_attention.metal" header's implicit causal / sliding-window rule).
    Returns [q_l, n_heads, D] float64, or [len(rows), D] when ``rows`` is a
    list of (node i, head h) pairs.
    """
    q = _c(q, np.float32)
    H, q_l, D = q.shape
    assert k.shape == v.shape and k.dtype == v.dtype
    kv_f16 = 1 if k.dtype == np.float16 else 0
    kdt = np.float16 if kv_f16 else np.float32
    k = _c(k, kdt)
    v = _c(v, kdt)
    Hk, cap, Dk = k.shape
    assert Dk == D and Hk == n_kv_heads
    if mask is not None:
        mask = _c(mask, np.float32)
        stride = mask.shape[1] if mask_stride is None else int(mask_stride)
    else:
        stride = kv_seq_len if mask_stride is None else int(mask_stride)
    if rows is None:
        sel, nsel = None, 0
        out = np.empty((q_l, H, D), dtype=np.float64)
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.uint32).reshape(-1, 2))
        nsel = sel.shape[0]
        out = np.empty((nsel, D), dtype=np.float64)
    rc = _load().orc_attention_ex(_ptr(q), _ptr(k), _ptr(v), kv_f16, _ptr(mask), H,
                                  Hk, D, kv_seq_len, cap, q_l, stride, float(scale),
                                  int(window_start), _ptr(sel), nsel, _ptr(out),
                                  _threads(nthreads))
    if rc != 0:
        raise OracleError("invalid attention problem")
    return out


def attention_partials(q, k, v, mask, bounds, *, n_kv_heads, kv_seq_len, scale,
                       mask_stride=None, nthreads=None):
    """Split-KV partials over the key partition ``bounds`` (exact arithmetic).

    Returns (o_un [nrows, nparts, D], s [nrows, nparts], m [nrows, nparts]);
    rows are r = i * n_heads + h; m is in natural-log units, -inf for an
    empty part ("tree_attention.metal" header: split-KV with a merge pass).
    """
    q = _c(q, np.float32)
    H, q_l, D = q.shape
    kv_f16 = 1 if k.dtype == np.float16 else 0
    kdt = np.float16 if kv_f16 else np.float32
    k = _c(k, kdt)
    v = _c(v, kdt)
    Hk, cap, _ = k.shape
    if mask is not None:
        mask = _c(mask, np.float32)
        stride = mask.shape[1] if mask_stride is None else int(mask_stride)
    else:
        stride = kv_seq_len if mask_stride is None else int(mask_stride)
    bounds = np.ascontiguousarray(np.asarray(bounds, dtype=np.uint32))
    nparts = bounds.shape[0] - 1
    nrows = H * q_l
    o_un = np.empty((nrows, nparts, D), dtype=np.float64)
    s = np.empty((nrows, nparts), dtype=np.float64)
    m = np.empty((nrows, nparts), dtype=np.float64)
    rc = _load().orc_attention_partials(_ptr(q), _ptr(k), _ptr(v), kv_f16,
                                        _ptr(mask), H, Hk, D, kv_seq_len, cap,
                                        q_l, stride, float(scale), _ptr(bounds),
                                        nparts, _ptr(o_un), _ptr(s), _ptr(m),
                                        _threads(nthreads))
    if rc != 0:
        raise OracleError("invalid partials problem")
    return o_un, s, m


def lse_combine(o_un, s, m):
    """Merge split partials (the reduce pass): returns [nrows, D] float64."""
    o_un = _c(o_un, np.float64)
    s = _c(s, np.float64)
    m = _c(m, np.float64)
    nrows, nparts, D = o_un.shape
    out = np.empty((nrows, D), dtype=np.float64)
    _load().orc_lse_combine(_ptr(o_un), _ptr(s), _ptr(m), nrows, D, nparts,
                            _ptr(out))
    return out


def bf16_to_f64(bits):
    """bfloat16 bit pattern -> float64, exactly (the oracle's decoder)."""
    return _load().orc_bf16_to_f64(int(bits))


def quant_attention(q, k_packed, k_scales, k_biases, v_packed, v_scales,
                    v_biases, *, n_kv_heads, kv_seq_len, bits, group_size, scale,
                    sinks=None, mask=None, mask_bool=None, mask_head_stride=0,
                    mask_stride=None, window_size=0, elem="f16", rows=None,
                    nthreads=None):
    """Affine-quantized K/V attention in double ("ffai/flash_quantized_sdpa.rs").

    q: [B*nQ, q_l, dim] float16.  k_packed: [B*nKV, cap, dim/(32/bits)] uint32.
    k_scales/k_biases: [B*nKV, cap, dim/G] float16.  V the same.
    sinks: [nQ] float32 or None.  mask: float16 array (flat), cell
    (q_idx, i, t) at q_idx*mask_head_stride + i*mask_stride + t, or None.
    mask_bool: uint32 array with the same cell layout (0 drops the key), or
    None; at most one of mask and mask_bool.  window_size: W > 0 keeps only
    tokens t with t + W > kv_seq_len - 1 (the bool- and float-mask macros'
    sliding-window gate); 0 keeps all.
    elem: the element type of q, the scales, biases and float mask -- "f16"
    (float16 arrays), "bf16" (uint16 arrays of bfloat16 bit patterns) or
    "f32" (float32 arrays).
    Returns [B*nQ, q_l, dim] float64 or [len(rows), dim] for (q_idx, i) rows.
    """
    code = {"f16": 0, "bf16": 1, "f32": 2}[elem]
    et = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32}[elem]
    q = _c(q, et)
    BnQ, q_l, dim = q.shape
    k_packed = _c(k_packed, np.uint32)
    v_packed = _c(v_packed, np.uint32)
    k_scales = _c(k_scales, et)
    k_biases = _c(k_biases, et)
    v_scales = _c(v_scales, et)
    v_biases = _c(v_biases, et)
    BnKV, cap, _ = k_packed.shape
    batch = BnKV // n_kv_heads
    nq = BnQ // batch
    if sinks is not None:
        sinks = _c(sinks, np.float32)
    if mask is not None:
        mask = _c(mask, et)
    if mask_bool is not None:
        mask_bool = _c(mask_bool, np.uint32)
    stride = kv_seq_len if mask_stride is None else int(mask_stride)
    if rows is None:
        sel, nsel = None, 0
        out = np.empty((BnQ, q_l, dim), dtype=np.float64)
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.uint32).reshape(-1, 2))
        nsel = sel.shape[0]
        out = np.empty((nsel, dim), dtype=np.float64)
    h = lambda a: a
    rc = _load().orc_quant_attention_ex(
        code, _ptr(h(q)), _ptr(k_packed), _ptr(h(k_scales)), _ptr(h(k_biases)),
        _ptr(v_packed), _ptr(h(v_scales)), _ptr(h(v_biases)), _ptr(sinks),
        _ptr(h(mask)), _ptr(mask_bool), int(mask_head_stride), stride,
        int(window_size), batch, nq, n_kv_heads, dim, kv_seq_len, cap, q_l, bits,
        group_size, float(scale), _ptr(sel), nsel, _ptr(out), _threads(nthreads))
    if rc != 0:
        raise OracleError("invalid quantized problem")
    return out
