"""Builds libspecverify.so (HIP, gfx950) in-tree with hipcc.

    python -m speculative_decoding_verification_12_amd.build

Every kernel and the C-ABI host code are compiled in one hipcc invocation. Packed fp32 vector
instructions are disabled for the device code (`-target-feature -packed-fp32-ops`), and
automatic a*b+c contraction is off (`-ffp-contract=off`): reference exponents such as fl(m*c)
must be the same rounded product wherever they appear; explicit fmaf() calls stay fused.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = ["api.hip", "verify_sample.hip", "verify_greedy.hip", "predict.hip", "kv_cache.hip",
           "ngram.hip"]
ARCH = os.environ.get("SPEC_VERIFY_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def build_command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
