"""Build libresa.so in-tree with hipcc for gfx950.

Usage: python -m block_sparse_attention_quest_amd.build [--debug]
"""
from __future__ import annotations

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


def build(debug: bool = False, verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs + ["-o", tmp]
    if debug:
        cmd.insert(1, "-g")
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libresa.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv, verbose=True))
