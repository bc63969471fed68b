"""Build libresa in-tree with hipcc for gfx950.

Three builds of the same sources:
  libresa.so        the library (release).
  libresa_debug.so  checked build: RESA_DEBUG_CHECKS compiles the kernels'
                    device-side precondition checks in, and every call waits
                    for its stream to report a failed check as
                    RESA_ERR_INVALID (for tests; the RESA_LIB environment
                    variable makes the binding load it).
  libresa_asan.so   the host code built with AddressSanitizer (device code as
                    in the release build), for the C ABI tests on the CPU with
                    the sanitizer runtime preloaded.

Usage: python -m block_sparse_attention_quest_amd.build [release|debug_checks|asan|all] [-g]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libresa.so")
SOURCES = ["resa_api.hip", "k_descriptors.hip", "k_select.hip", "k_decode.hip", "k_rectify.hip"]

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result"]

# host code only: each sanitizer flag is preceded by -Xarch_host
ASAN_HOST_FLAGS = "-g -Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()

VARIANTS = {
    "release": ("libresa.so", []),
    "debug_checks": ("libresa_debug.so", ["-DRESA_DEBUG_CHECKS"]),
    "asan": ("libresa_asan.so", ASAN_HOST_FLAGS),
}


def lib_path(variant: str = "release") -> str:
    return os.path.join(PKG, VARIANTS[variant][0])


def asan_runtime() -> str:
    """The host AddressSanitizer runtime of the ROCm compiler (for LD_PRELOAD)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def _command(variant: str, debug: bool) -> list:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    out = lib_path(variant)
    cmd = [hipcc] + HIP_FLAGS + VARIANTS[variant][1] + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs
    if debug:
        cmd.insert(1, "-g")
    return cmd + ["-o", out + ".tmp"]


def build(variant: str = "release", debug: bool = False, verbose: bool = False) -> str:
    return build_many([variant], debug, verbose)[0]


def build_many(variants, debug: bool = False, verbose: bool = False) -> list:
    """Compile the given variants side by side; raise if any fails."""
    procs = []
    for v in variants:
        cmd = _command(v, debug)
        if verbose:
            print(" ".join(cmd))
        procs.append((v, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for v, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed.append(v)
    if failed:
        raise RuntimeError(f"hipcc failed building {', '.join(VARIANTS[v][0] for v in failed)}")
    for v in variants:
        os.replace(lib_path(v) + ".tmp", lib_path(v))
    return [lib_path(v) for v in variants]


def build_all(verbose: bool = False) -> list:
    return build_many(list(VARIANTS), verbose=verbose)


if __name__ == "__main__":
    which = [a for a in sys.argv[1:] if not a.startswith("-")] or ["release"]
    names = list(VARIANTS) if which == ["all"] else which
    for path in build_many(names, debug="-g" in sys.argv, verbose=True):
        print(path)
