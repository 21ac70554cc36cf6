"""The host code of libgrpo (argument validation, workspace layout, CSR
handling in grpo_api.hip and grpo_prep.hip) under AddressSanitizer and
UndefinedBehaviorSanitizer: a host-sanitized build of the library runs the
whole ABI test file (tests/test_abi.py: every entry point with invalid and
edge-case arguments through fake device pointers) in a child process that
preloads the sanitizer runtime.  Any report aborts that process.  CPU only:
the fake pointers must never reach a launch."""

import os
import subprocess
import sys

import pytest
import torch

from rl_post_loss_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-validation tests use fake device pointers")


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    lib = B.build_host_sanitized(tmp_path / "libgrpo_hostsan.so", tmp_path / "obj")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in syms and "__ubsan_handle" in syms, "host code not instrumented"
    env = dict(os.environ,
               LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               GRPO_TEST_LIB=lib)
    # the sanitized library is the one the tests load
    probe = ("import os, ctypes; from rl_post_loss_amd import _abi; "
             "lib = _abi.load_library(os.environ['GRPO_TEST_LIB']); "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); print(lib._name)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p",
                        "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout and " failed" not in r.stdout
