"""Host-side checks of the C ABI (no GPU): exports, sizes, split planning and
argument validation.

Validation mirrors "ops/tree_attention.rs" (mlx-native 0.9.2),
validate_params / validate_buffers and their unit tests: every rule has a
failing case here, and each failing call must return its error code before
anything reaches the GPU.  The calls below pass fake device addresses, so
they are only run where no GPU is reachable.
"""

import ctypes
import os
import re

import pytest

from tree_masked_decode_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")

no_gpu_only = pytest.mark.skipif(
    os.path.exists("/dev/kfd"),
    reason="fake-pointer validation calls run only where no GPU is reachable")


@pytest.fixture(scope="module")
def lib():
    from tree_masked_decode_amd import build
    if not os.path.exists(L.LIB_PATH):
        build.build()
    return L.load()


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^TA_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M))
    assert declared == set(L.EXPORTS)
    out = os.popen("nm -D --defined-only %s" % L.LIB_PATH).read()
    exported = set(re.findall(r" T (\w+)$", out, re.M))
    assert exported == declared, exported ^ declared


def test_partials_bytes_golden(lib, golden_dir):
    # "ops/tree_attention.rs" tmp_buffer_bytes unit test value.
    for line in open(os.path.join(golden_dir, "partials_bytes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        H, D, q_l, nwg, expect = map(int, line.split())
        assert lib.tree_attn_partials_bytes(H, D, q_l, nwg) == expect


def test_partials_bytes_formula_and_saturation(lib):
    assert lib.tree_attn_partials_bytes(24, 256, 64, 16) == 24 * 64 * 16 * 258 * 4
    assert lib.tree_attn_partials_bytes(1, 128, 1, 1) == 130 * 4
    big = 0xFFFFFFFF
    assert lib.tree_attn_partials_bytes(big, big, big, big) == ctypes.c_size_t(-1).value


def test_pick_nwg_properties(lib):
    for args in [(4, 2, 128, 256, 4, 0), (24, 4, 256, 4096, 16, 1),
                 (24, 4, 256, 32768, 64, 1), (32, 8, 512, 131072, 8, 1),
                 (1, 1, 128, 1, 1, 1)]:
        n = lib.tree_attn_pick_nwg(*args, 0)
        assert n >= 1
        assert n == lib.tree_attn_pick_nwg(*args, 256)
    # a longer context never gets fewer splits
    a = lib.tree_attn_pick_nwg(32, 8, 512, 8192, 8, 1, 0)
    b = lib.tree_attn_pick_nwg(32, 8, 512, 131072, 8, 1, 0)
    assert b >= a
    assert lib.tree_attn_pick_nwg(0, 1, 128, 10, 1, 1, 0) == 1
    assert lib.tree_attn_quant_pick_nwg(4, 32, 8, 128, 16384, 1, 0) >= 1


@no_gpu_only
def test_quant_pick_nwg_ex_follows_the_variant_footprint(lib):
    # without a device: two wavefronts per SIMD at dim 128, and the LDS of the
    # variant: 4-bit stages fit eight workgroups a CU, 8-bit ones six
    f = lib.tree_attn_quant_pick_nwg_ex
    assert f(4, 32, 8, 128, 16384, 1, 4, 64, 1, 1, 0) == 64
    assert f(4, 32, 8, 128, 16384, 1, 8, 64, 1, 1, 0) == 48
    assert f(4, 32, 8, 128, 16384, 1, 4, 64, 2, 1, 0) == 64
    # a short sequence caps the splits at two tiles each
    assert f(4, 32, 8, 128, 4096, 1, 4, 64, 1, 1, 0) == 64
    assert f(4, 32, 8, 128, 512, 1, 4, 64, 1, 1, 0) == 8
    # fp32 elements: wider scale/bias slices, still within the 8-per-CU plan
    assert f(4, 32, 8, 128, 16384, 1, 4, 64, 1, 0, 0) >= 48
    # degenerate shapes and unsupported variants still give a usable count
    assert f(0, 32, 8, 128, 16384, 1, 4, 64, 1, 1, 0) == 1
    assert f(4, 32, 8, 96, 16384, 1, 4, 32, 1, 1, 0) >= 1


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(L.LibraryMissing):
        L.load()


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "tree_masked_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text and "oracle.c" not in text, f
                assert "orc_" not in text, f


# --------------------------------------------------------------------------
# argument validation (fake device pointers: never dereferenced)
# --------------------------------------------------------------------------
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced
BIG = 1 << 40


def fwd(lib, **kw):
    p = dict(q=FAKE, q_bytes=BIG, k=FAKE, v=FAKE, kv_dtype=1, kv_bytes=BIG,
             mask=FAKE, mask_bytes=BIG, partials=FAKE, partials_bytes=BIG,
             out=FAKE, out_bytes=BIG, n_heads=16, n_kv_heads=8, head_dim=256,
             kv_seq_len=100, kv_capacity=1024, q_l=1, mask_stride=100,
             scale=1.0, nwg=4)
    p.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_forward(
        vp(p["q"]), p["q_bytes"], vp(p["k"]), vp(p["v"]), p["kv_dtype"],
        p["kv_bytes"], vp(p["mask"]), p["mask_bytes"], vp(p["partials"]),
        p["partials_bytes"], vp(p["out"]), p["out_bytes"], p["n_heads"],
        p["n_kv_heads"], p["head_dim"], p["kv_seq_len"], p["kv_capacity"],
        p["q_l"], p["mask_stride"], p["scale"], p["nwg"], None)


def fwd_noalloc(lib, **kw):
    p = dict(q=FAKE, q_bytes=BIG, k=FAKE, v=FAKE, kv_dtype=1, kv_bytes=BIG,
             mask=FAKE, mask_bytes=BIG, out=FAKE, out_bytes=BIG, n_heads=32,
             n_kv_heads=4, head_dim=512, kv_seq_len=2048, kv_capacity=2048, q_l=64,
             mask_stride=2048, scale=1.0, nwg=15)
    p.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_forward_noalloc(
        vp(p["q"]), p["q_bytes"], vp(p["k"]), vp(p["v"]), p["kv_dtype"],
        p["kv_bytes"], vp(p["mask"]), p["mask_bytes"], vp(p["out"]), p["out_bytes"],
        p["n_heads"], p["n_kv_heads"], p["head_dim"], p["kv_seq_len"],
        p["kv_capacity"], p["q_l"], p["mask_stride"], p["scale"], p["nwg"], None)


@no_gpu_only
@pytest.mark.parametrize("kw,code,word", [
    # 16 splits of 32 x 64 rows x (512 + 2) floats: 67.4 MB > 64 MiB
    (dict(nwg=16), L.TA_ESIZE, "static scratch"),
    (dict(nwg=65537), L.TA_EINVAL, "nwg"),
    (dict(out=None), L.TA_EINVAL, "out"),
    (dict(nwg=1, out_bytes=64 * 32 * 512 * 4 - 1), L.TA_ESIZE, "output"),
    (dict(head_dim=64), L.TA_EUNSUPPORTED, "head_dim"),
    (dict(kv_capacity=100), L.TA_EINVAL, "kv_capacity"),
    (dict(mask_bytes=64 * 2048 * 4 - 1), L.TA_ESIZE, "mask"),
])
def test_noalloc_validation(lib, kw, code, word):
    # every rule is checked on the host, before the scratch is looked up
    assert fwd_noalloc(lib, **kw) == code
    assert word in L.last_error()


def test_noalloc_limit_matches_partials_bytes(lib):
    import tree_masked_decode_amd as T
    assert T.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert lib.tree_attn_partials_bytes(32, 512, 64, 15) <= T.NOALLOC_SCRATCH_BYTES
    assert lib.tree_attn_partials_bytes(32, 512, 64, 16) > T.NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert re.search(r"#define TA_NOALLOC_SCRATCH_BYTES \(64ull << 20\)", text)


FWD_CASES = [
    # reference unit tests
    (dict(mask_stride=50), L.TA_EINVAL, "mask_stride"),
    (dict(head_dim=64), L.TA_EUNSUPPORTED, "head_dim"),
    (dict(q_l=0), L.TA_EINVAL, "q_l"),
    # the rest of validate_params
    (dict(n_heads=0), L.TA_EINVAL, "n_heads"),
    (dict(n_kv_heads=0), L.TA_EINVAL, "n_kv_heads"),
    (dict(n_heads=12, n_kv_heads=8), L.TA_EINVAL, "multiple"),
    (dict(kv_seq_len=0), L.TA_EINVAL, "kv_seq_len"),
    (dict(kv_capacity=99), L.TA_EINVAL, "kv_capacity"),
    (dict(kv_dtype=7), L.TA_EUNSUPPORTED, "dtype"),
    (dict(nwg=0), L.TA_EINVAL, "nwg"),
    (dict(scale=float("nan")), L.TA_EINVAL, "scale"),
    # validate_buffers: sizes
    (dict(q_bytes=16 * 256 * 4 - 1), L.TA_ESIZE, "q buffer"),
    (dict(kv_bytes=8 * 1024 * 256 * 2 - 1), L.TA_ESIZE, "k/v buffer"),
    (dict(kv_dtype=0, kv_bytes=8 * 1024 * 256 * 4 - 1), L.TA_ESIZE, "k/v buffer"),
    (dict(mask_bytes=100 * 4 - 1), L.TA_ESIZE, "tree mask"),
    (dict(nwg=1, out_bytes=16 * 256 * 4 - 1), L.TA_ESIZE, "output"),
    (dict(partials_bytes=16 * 4 * 258 * 4 - 1), L.TA_ESIZE, "partials"),
    # checked multiplication
    (dict(n_kv_heads=0xFFFFFFFF, n_heads=0xFFFFFFFF, kv_capacity=0xFFFFFFFF),
     L.TA_EOVERFLOW, "overflow"),
    # pointers
    (dict(q=None), L.TA_EINVAL, "NULL"),
    (dict(nwg=1, out=None), L.TA_EINVAL, "out"),
    (dict(partials=None), L.TA_EINVAL, "partials"),
    (dict(k=FAKE + 4), L.TA_EINVAL, "aligned"),
]


@no_gpu_only
@pytest.mark.parametrize("kw,code,word", FWD_CASES)
def test_forward_validation(lib, kw, code, word):
    assert fwd(lib, **kw) == code
    assert word in L.last_error()


def red(lib, **kw):
    p = dict(partials=FAKE, partials_bytes=BIG, out=FAKE, out_dtype=0,
             out_bytes=BIG, nrows=16, head_dim=256, nwg=4)
    p.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_reduce(vp(p["partials"]), p["partials_bytes"], vp(p["out"]),
                                p["out_dtype"], p["out_bytes"], p["nrows"],
                                p["head_dim"], p["nwg"], None)


@no_gpu_only
@pytest.mark.parametrize("kw,code,word", [
    (dict(nrows=0), L.TA_EINVAL, "nrows"),
    (dict(head_dim=130), L.TA_EUNSUPPORTED, "head_dim"),
    (dict(head_dim=1024), L.TA_EUNSUPPORTED, "head_dim"),
    (dict(nwg=0), L.TA_EINVAL, "nwg"),
    (dict(out_dtype=5), L.TA_EUNSUPPORTED, "dtype"),
    (dict(partials_bytes=16 * 4 * 258 * 4 - 1), L.TA_ESIZE, "partials"),
    (dict(out_bytes=16 * 256 * 4 - 1), L.TA_ESIZE, "output"),
    (dict(out_dtype=1, out_bytes=16 * 256 * 2 - 1), L.TA_ESIZE, "output"),
    (dict(out=None), L.TA_EINVAL, "NULL"),
])
def test_reduce_validation(lib, kw, code, word):
    assert red(lib, **kw) == code
    assert word in L.last_error()


def qf(lib, **kw):
    p = dict(q=FAKE, q_dtype=1, q_bytes=BIG, kp=FAKE, ks=FAKE, kb=FAKE, vp=FAKE,
             vs=FAKE, vb=FAKE, kv_bytes=[BIG] * 6, sinks=FAKE, sinks_bytes=BIG,
             mask=FAKE, mask_bytes=BIG, mhs=16384, mask_stride=16384,
             partials=FAKE, partials_bytes=BIG, out=FAKE, out_bytes=BIG,
             batch=4, nq=32, nkv=8, dim=128, L=16384, cap=16384, q_l=1, bits=4,
             G=64, scale=0.088, nwg=8)
    p.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    kvb = (ctypes.c_size_t * 6)(*p["kv_bytes"])
    return lib.tree_attn_quant_forward(
        vp(p["q"]), p["q_dtype"], p["q_bytes"], vp(p["kp"]), vp(p["ks"]),
        vp(p["kb"]), vp(p["vp"]), vp(p["vs"]), vp(p["vb"]), kvb, vp(p["sinks"]),
        p["sinks_bytes"], vp(p["mask"]), p["mask_bytes"], p["mhs"],
        p["mask_stride"], vp(p["partials"]), p["partials_bytes"], vp(p["out"]),
        p["out_bytes"], p["batch"], p["nq"], p["nkv"], p["dim"], p["L"],
        p["cap"], p["q_l"], p["bits"], p["G"], p["scale"], p["nwg"], None)


@no_gpu_only
@pytest.mark.parametrize("kw,code,word", [
    (dict(q_dtype=3), L.TA_EUNSUPPORTED, "dtype"),
    (dict(q_dtype=0, q_bytes=128 * 128 * 4 - 1), L.TA_ESIZE, "q buffer"),   # fp32 elements
    (dict(q_dtype=2, kv_bytes=[BIG, 32 * 16384 * 2 * 2 - 1, BIG, BIG, BIG, BIG]),
     L.TA_ESIZE, "k_scales"),                                          # bf16 elements
    (dict(bits=3), L.TA_EUNSUPPORTED, "bits"),
    (dict(dim=80), L.TA_EUNSUPPORTED, "dim"),
    (dict(dim=96), L.TA_EINVAL, "divisible"),      # dim 96 needs group_size 32
    (dict(G=48), L.TA_EUNSUPPORTED, "group_size"),
    (dict(dim=64, G=128), L.TA_EINVAL, "divisible"),
    (dict(nq=30), L.TA_EINVAL, "divisible"),
    (dict(cap=100), L.TA_EINVAL, "kv_capacity"),
    (dict(q_l=0), L.TA_EINVAL, "q_l"),
    (dict(mask_stride=100), L.TA_EINVAL, "mask_stride"),
    (dict(kv_bytes=[BIG, BIG, BIG, 32 * 16384 * 16 * 4 - 1, BIG, BIG]), L.TA_ESIZE, "v_packed"),
    (dict(kv_bytes=[BIG, 32 * 16384 * 2 * 2 - 1, BIG, BIG, BIG, BIG]), L.TA_ESIZE, "k_scales"),
    (dict(sinks_bytes=32 * 4 - 1), L.TA_ESIZE, "sinks"),
    (dict(mask_bytes=(127 * 16384 + 16384) * 2 - 1), L.TA_ESIZE, "mask"),
    (dict(q_bytes=128 * 128 * 2 - 1), L.TA_ESIZE, "q buffer"),
    (dict(nwg=1, out_bytes=128 * 128 * 2 - 1), L.TA_ESIZE, "output"),
    (dict(vb=None), L.TA_EINVAL, "NULL"),
    (dict(mhs=1 << 62), L.TA_EOVERFLOW, "overflow"),
    (dict(dim=64, G=64, cap=16385), L.TA_EUNSUPPORTED, "even"),
    # three fp16 scales per token: an odd capacity misaligns every other head
    (dict(dim=96, G=32, cap=16385), L.TA_EUNSUPPORTED, "even"),
    (dict(dim=96, G=32, cap=16385, q_dtype=2), L.TA_EUNSUPPORTED, "even"),
])
def test_quant_validation(lib, kw, code, word):
    assert qf(lib, **kw) == code
    assert word in L.last_error()


def qfx(lib, mask_kind=1, window=0, **kw):
    p = dict(q=FAKE, q_dtype=1, q_bytes=BIG, kp=FAKE, ks=FAKE, kb=FAKE, vp=FAKE,
             vs=FAKE, vb=FAKE, kv_bytes=[BIG] * 6, sinks=FAKE, sinks_bytes=BIG,
             mask=FAKE, mask_bytes=BIG, mhs=16384, mask_stride=16384,
             partials=FAKE, partials_bytes=BIG, out=FAKE, out_bytes=BIG,
             batch=4, nq=32, nkv=8, dim=128, L=16384, cap=16384, q_l=1, bits=4,
             G=64, scale=0.088, nwg=8)
    p.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    kvb = (ctypes.c_size_t * 6)(*p["kv_bytes"])
    return lib.tree_attn_quant_forward_ex(
        vp(p["q"]), p["q_dtype"], p["q_bytes"], vp(p["kp"]), vp(p["ks"]),
        vp(p["kb"]), vp(p["vp"]), vp(p["vs"]), vp(p["vb"]), kvb, vp(p["sinks"]),
        p["sinks_bytes"], vp(p["mask"]), mask_kind, p["mask_bytes"], p["mhs"],
        p["mask_stride"], window, vp(p["partials"]), p["partials_bytes"],
        vp(p["out"]), p["out_bytes"], p["batch"], p["nq"], p["nkv"], p["dim"],
        p["L"], p["cap"], p["q_l"], p["bits"], p["G"], p["scale"], p["nwg"], None)


@no_gpu_only
@pytest.mark.parametrize("kw,code,word", [
    (dict(mask_kind=3), L.TA_EINVAL, "mask_kind"),
    (dict(mask_kind=-1), L.TA_EINVAL, "mask_kind"),
    (dict(mask_kind=2, mask=None), L.TA_EINVAL, "NULL exactly"),
    (dict(mask_kind=0), L.TA_EINVAL, "NULL exactly"),
    (dict(mask_kind=2, mask_bytes=(127 * 16384 + 16384) * 4 - 1), L.TA_ESIZE, "mask"),
    (dict(mask_kind=1, mask_bytes=(127 * 16384 + 16384) * 2 - 1), L.TA_ESIZE, "mask"),
    (dict(mask_kind=2, mask=FAKE + 2), L.TA_EINVAL, "aligned"),
    (dict(mask_kind=2, mask_stride=100), L.TA_EINVAL, "mask_stride"),
    (dict(mask_kind=2, window=5, bits=3), L.TA_EUNSUPPORTED, "bits"),
])
def test_quant_ex_validation(lib, kw, code, word):
    assert qfx(lib, **kw) == code
    assert word in L.last_error()


@no_gpu_only
@pytest.mark.parametrize("ws,L_,code,word", [
    (16384, 16384, L.TA_EINVAL, "window_start"),
    (20000, 16384, L.TA_EINVAL, "window_start"),
    (5, 16384, L.TA_EUNSUPPORTED, "head_dim"),
])
def test_decode_validation(lib, ws, L_, code, word):
    vp = ctypes.c_void_p
    hd = 96 if code == L.TA_EUNSUPPORTED else 128
    rc = lib.tree_attn_decode(vp(FAKE), BIG, vp(FAKE), vp(FAKE), 1, BIG, vp(FAKE), BIG,
                              vp(FAKE), BIG, 8, 2, hd, L_, L_, 4, ws, 0.1, 2, None)
    assert rc == code
    assert word in L.last_error()


def mk(lib, parents, q_l=None, L_=16, stride=16, mask=FAKE, nbytes=BIG):
    arr = (ctypes.c_int32 * max(1, len(parents)))(*parents)
    q_l = len(parents) if q_l is None else q_l
    return lib.build_tree_mask(ctypes.cast(arr, ctypes.c_void_p), q_l, L_, stride,
                               None if mask is None else ctypes.c_void_p(mask),
                               nbytes, None)


@no_gpu_only
@pytest.mark.parametrize("args,code,word", [
    (dict(parents=[0, 0, 1]), L.TA_EINVAL, "topology"),
    (dict(parents=[-1, 1, 0]), L.TA_EINVAL, "topology"),
    (dict(parents=[-1, 0, -1]), L.TA_EINVAL, "topology"),
    (dict(parents=[-1], q_l=0), L.TA_EINVAL, "q_l"),
    (dict(parents=[-1] + list(range(1024)), L_=2048, stride=2048), L.TA_EUNSUPPORTED, "1024"),
    (dict(parents=[-1, 0, 1], L_=2, stride=2), L.TA_EINVAL, "kv_seq_len"),
    (dict(parents=[-1, 0, 1], stride=15), L.TA_EINVAL, "mask_stride"),
    (dict(parents=[-1, 0, 1], nbytes=3 * 16 * 4 - 1), L.TA_ESIZE, "mask buffer"),
    (dict(parents=[-1, 0, 1], mask=None), L.TA_EINVAL, "NULL"),
])
def test_tree_mask_validation(lib, args, code, word):
    assert mk(lib, **args) == code
    assert word in L.last_error()


def test_last_error_is_per_call(lib):
    if os.path.exists("/dev/kfd"):
        pytest.skip("fake-pointer call")
    assert fwd(lib, head_dim=64) == L.TA_EUNSUPPORTED
    assert L.last_error() != ""
    assert lib.tree_attn_partials_bytes(1, 4, 1, 1) == 24
