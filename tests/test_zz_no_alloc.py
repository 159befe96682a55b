"""GPU checks of tree_attn_forward_noalloc: the forward plus merge with the
split partials in the library's static device buffer.

Its output must equal tree_attn_forward + tree_attn_reduce with the same
split count, bit for bit, on consecutive calls whose sizes shrink (the
buffer keeps the previous call's contents), on the null stream and on a
side stream, and up to the buffer's limit; the fp tolerances against the
oracle hold as for the forward itself.
"""

import numpy as np
import pytest

import oracle
from tree_masked_decode_amd import inputs

from helpers import assert_close, dev, host, note

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "f16": 2e-3}


@pytest.fixture(scope="module")
def ta():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import tree_masked_decode_amd as ta
    ta._api()
    return ta


def _case(seed, H, Hk, D, L, q_l, kvd, tree):
    c = inputs.fp_case(dict(n_heads=H, n_kv_heads=Hk, head_dim=D, kv_seq_len=L,
                            kv_capacity=L + 5, q_l=q_l, tree=tree, mask_stride=L,
                            kv_dtype=kvd, kv_std=1.0), seed=seed)
    mask = None if tree == "chain" else oracle.tree_mask(c["parents"], L)
    return c, mask


def _both(ta, c, mask, nwg, stream=None):
    """(no-alloc result, forward + reduce result) for one case."""
    import torch
    q, k, v = dev(c["q"]), dev(c["k"]), dev(c["v"])
    m = None if mask is None else dev(mask)
    H, q_l, D = c["q"].shape
    L = c["kv_seq_len"]
    ref = ta.verify(q, k, v, m, kv_seq_len=L, scale=c["scale"], nwg=nwg)
    out = torch.full((q_l, H, D), float("nan"), dtype=torch.float32, device="cuda")
    if stream is None:
        ta.tree_attn_forward_noalloc(q, k, v, m, kv_seq_len=L, scale=c["scale"],
                                     nwg=nwg, out=out)
    else:
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            ta.tree_attn_forward_noalloc(q, k, v, m, kv_seq_len=L, scale=c["scale"],
                                         nwg=nwg, out=out, stream=stream)
        torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    return host(out), host(ref)


def test_noalloc_two_calls_shrinking(ta):
    # first call: fp16 K/V, explicit tree mask, 6 splits (2.4 MB of partials)
    note("noalloc call 1: f16 D=256 H=16 Hk=2 L=3000 q_l=24 nwg=6")
    c1, m1 = _case(70, 16, 2, 256, 3000, 24, "f16", "dynamic")
    got, ref = _both(ta, c1, m1, 6)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert_close(got, oracle.attention(c1["q"], c1["k"], c1["v"], m1, n_kv_heads=2,
                                       kv_seq_len=3000, scale=c1["scale"]),
                 TOL["f16"], "noalloc call 1")
    # second, smaller call: fp32 K/V, implicit rule, 3 splits, reading a
    # buffer that still holds the first call's partials
    note("noalloc call 2: f32 D=128 H=4 Hk=2 L=333 q_l=5 nwg=3")
    c2, m2 = _case(71, 4, 2, 128, 333, 5, "f32", "chain")
    got, ref = _both(ta, c2, m2, 3)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert_close(got, oracle.attention(c2["q"], c2["k"], c2["v"], None, n_kv_heads=2,
                                       kv_seq_len=333, scale=c2["scale"]),
                 TOL["f32"], "noalloc call 2")


def test_noalloc_side_stream_single_split_and_limit(ta):
    import torch
    # a side stream (default priority): the buffer is found through the
    # stream's device
    note("noalloc side stream: f16 D=128 H=8 Hk=2 L=700 q_l=9 nwg=4")
    c, m = _case(72, 8, 2, 128, 700, 9, "f16", "binary")
    got, ref = _both(ta, c, m, 4, stream=torch.cuda.Stream())
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # one split: no scratch, the forward writes out itself
    note("noalloc nwg=1")
    got, ref = _both(ta, c, m, 1)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # partials that nearly fill the buffer: 15 splits of 32 heads x 64
    # nodes x (512 + 2) floats = 63.2 MB of 64 MiB
    H, q_l, D, nwg = 32, 64, 512, 15
    assert ta.partials_bytes(H, D, q_l, nwg) <= ta.NOALLOC_SCRATCH_BYTES
    assert ta.partials_bytes(H, D, q_l, nwg + 1) > ta.NOALLOC_SCRATCH_BYTES
    note("noalloc near the limit: f16 D=512 H=32 Hk=4 L=2048 q_l=64 nwg=15")
    c, m = _case(73, H, 4, D, 2048, q_l, "f16", "dynamic")
    got, ref = _both(ta, c, m, nwg)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # beyond the limit: rejected before anything is enqueued, out untouched
    note("noalloc beyond the limit (host-side rejection)")
    out = torch.full((q_l, H, D), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ta.TreeAttnError, match="static scratch"):
        ta.tree_attn_forward_noalloc(dev(c["q"]), dev(c["k"]), dev(c["v"]), dev(m),
                                     kv_seq_len=2048, scale=c["scale"], nwg=nwg + 1,
                                     out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
