"""Code-generation guard for the fp16 forward's tile loop (CPU only; it
compiles csrc/fwd_f16.hip to gfx950 assembly with the library's own flags).

The fast tiles run an inner loop that only the rare rescale of O leaves, and
O stays in the matrix-core accumulation registers inside it.  If the
compiler folds that inner loop into the outer one, the loop-carried O moves
to ordinary registers and every tile ends with a copy of all of O out of the
accumulation registers (132 v_accvgpr_read per tile at head dim 512): the
kernel is still correct, only slower, so no parity test notices.  This test
checks, for every kernel instantiation, that a loop nested two deep exists
and that its blocks read no more accumulation registers than the score
copies (8 per 16-row block)."""
import collections
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tree_masked_decode_amd")


def _build_module():
    spec = importlib.util.spec_from_file_location("ta_build_flags", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def f16_asm(tmp_path_factory):
    b = _build_module()
    if shutil.which(b.HIPCC) is None and not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "fwd_f16.s")
    flags = [f for f in b.CFLAGS if f not in ("-fPIC", "-fvisibility=hidden")]
    cmd = [b.HIPCC, *flags, *b.FILE_FLAGS.get("fwd_f16.hip", []), "-S", "--cuda-device-only",
           os.path.join(b.CSRC, "fwd_f16.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _kernels(asm):
    for m in re.finditer(r"^(_Z\w*fwd_f16_kernelILi(\d+)ELi(\d+)E\w*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        yield m.group(1), int(m.group(2)), int(m.group(3)), asm[m.end():end]


def test_fast_tile_loop_stays_nested_and_keeps_o_in_accumulators(f16_asm):
    seen = 0
    for name, head_dim, rb, body in _kernels(f16_asm):
        seen += 1
        depth, max_depth = 0, 0
        reads = collections.Counter()
        for line in body.split("\n"):
            label = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):", line)
            if label:
                d = re.search(r"Depth=(\d)", line)
                depth = int(d.group(1)) if d else 0
                max_depth = max(max_depth, depth)
                continue
            tok = line.strip().split()
            if tok and tok[0].startswith("v_accvgpr_read"):
                reads[depth] += 1
        assert max_depth >= 2, "%s: the fast-tile loop is not nested" % name
        assert reads[2] <= 8 * rb, "%s: %d accumulation-register reads in the inner loop" % (
            name, reads[2])
    assert seen >= 30, "expected every instantiation in the assembly, found %d" % seen
