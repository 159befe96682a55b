"""Build libtreeattn.so (HIP, gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object in _build/ and linked
into tree_masked_decode_amd/libtreeattn.so.  Objects are rebuilt when their
source or any header changed.  `python -m tree_masked_decode_amd.build`
builds from the command line.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtreeattn.so")
ARCH = os.environ.get("TREEATTN_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-fno-gpu-rdc", "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # No packed-fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-file flags.  The quantized kernel at head dims up to 128 keeps its
# matrix-instruction accumulators in ordinary VGPRs: its inline rescale of O
# otherwise makes the compiler copy every accumulator between AGPRs and
# VGPRs once per tile.  Wider heads need the AGPRs for O.
FILE_FLAGS = {
    "quant_d%d_%s.hip" % (d, t): ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    for d in (64, 96, 128) for t in ("f16", "bf16", "f32")
}
# The fp16 forward's inputs are finite by contract: without NaNs to honour,
# fmaxf on matrix-instruction results needs no canonicalizing instruction.
FILE_FLAGS["fwd_f16.hip"] = ["-fno-honor-nans"]
FILE_FLAGS["fwd_wide.hip"] = ["-fno-honor-nans"]


def _headers():
    return glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(
        os.path.join(ROOT, "include", "*.h"))


def _stale(target, deps):
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(src, obj, extra):
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is expected and harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    return msg


def build(force: bool = False, verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    hdrs = _headers()
    objs, jobs = [], []
    for s in srcs:
        o = os.path.join(BUILD, os.path.basename(s)[:-4] + ".o")
        objs.append(o)
        if force or _stale(o, [s, *hdrs]):
            jobs.append((s, o))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for msg in ex.map(lambda j: _compile(
                j[0], j[1], FILE_FLAGS.get(os.path.basename(j[0]), []) + list(extra)), jobs):
            if verbose and msg.strip():
                print(msg)
    if force or jobs or _stale(LIB, objs):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv, verbose=True))
