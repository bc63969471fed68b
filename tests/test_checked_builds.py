"""The host-AddressSanitizer build of the library on the CPU: the C ABI tests
run against libresa_asan.so with the sanitizer runtime preloaded, so every
argument check, size query and rejection path of the host layer runs under
AddressSanitizer (no call reaches the GPU)."""
import os
import subprocess
import sys

import pytest

from block_sparse_attention_quest_amd import build as Bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_asan():
    lib = Bld.lib_path("asan")
    rt = Bld.asan_runtime()
    if not os.path.exists(lib) or not rt:
        pytest.skip("libresa_asan.so or the AddressSanitizer runtime is missing")
    assert b"__asan_init" in open(lib, "rb").read(), "libresa_asan.so is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, RESA_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "AddressSanitizer" not in out, out[-3000:]
    assert " passed" in out
