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


# Host-side sanitizers for a CPU-only check of the host code (argument
# validation, workspace layout, CSR handling): every sanitizer flag applies
# to the host pass only; device code is compiled as usual.
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer "
                 "-Xarch_host -g").split()
HOST_SANITIZED_SOURCES = ("grpo_api.hip", "grpo_prep.hip")


def asan_runtime():
    """The clang AddressSanitizer runtime a process must preload to load a
    host-sanitized library."""
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return hits[-1]


def build_host_sanitized(lib_path, build_dir):
    """libgrpo with the host code of HOST_SANITIZED_SOURCES built under
    AddressSanitizer and UndefinedBehaviorSanitizer, the other objects as
    usual.  For CPU-only tests of host validation (load it in a process that
    preloads asan_runtime())."""
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in sources():
        name = os.path.basename(src)
        obj = os.path.join(build_dir, name + ".o")
        extra = HOST_SANITIZE if name in HOST_SANITIZED_SOURCES else []
        if not extra:
            # reuse the regular object when it is newer than every source
            reg = os.path.join(BUILD_DIR, name + ".o")
            newest = max(os.path.getmtime(f) for f in glob.glob(os.path.join(CSRC, "*")) +
                         [os.path.join(ROOT, "include", "grpo.h")])
            if os.path.exists(reg) and os.path.getmtime(reg) >= newest:
                obj = reg
        objs.append((src, obj, extra))
    todo = [(s, o, e) for s, o, e in objs if e or not o.startswith(BUILD_DIR)]

    def compile_one(item):
        src, obj, extra = item
        return src, _run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj])

    with ThreadPoolExecutor(max_workers=max(1, min(len(todo), 8))) as ex:
        results = list(ex.map(compile_one, todo))
    for src, (rc, out) in results:
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SANITIZE, "-o",
                    str(lib_path), *[o for _, o, _ in objs]])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    return str(lib_path)


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)
