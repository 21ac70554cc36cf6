"""Builds libgrpo.so in-tree with hipcc for gfx950.

    python -m rl_post_loss_amd.build          # or rl_post_loss_amd.build.build_library()

The library is written next to this file so it travels with the source tree.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgrpo.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: the kernels spell out every fused multiply-add they want
# (fmaf), so the order of every rounding is fixed by the source.
# -packed-fp32-ops off: no v_pk_* fp32 forms anywhere.
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    "-Wno-unused-but-set-variable",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    return p.returncode, out


def build_library(verbose=False, jobs=None, extra_flags=(), lib_path=None, build_dir=None):
    """Compiles every csrc/*.hip for gfx950 and links libgrpo.so.  Always
    rebuilds.  Raises RuntimeError with the compiler output on failure.
    extra_flags (e.g. a -D tuning knob), lib_path and build_dir serve
    side-by-side builds of variants; the defaults build the library the
    package loads."""
    lib = lib_path or LIB
    bdir = build_dir or BUILD_DIR
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(bdir, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), 8)

    def compile_one(pair):
        src, obj = pair
        return src, _run([HIPCC, *FLAGS, *extra_flags, "-c", src, "-o", obj])

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(compile_one, zip(srcs, objs)))
    for src, (rc, out) in results:
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    tmp = lib + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, lib)
    return lib


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)
