"""Builds the plain-C ABI test program (tests/c_abi/abi_worked_example) with gcc against the
in-tree libspecverify.so and the HIP runtime's C API.

    python tests/c_abi/build.py
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "speculative_decoding_verification_12_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCE = os.path.join(HERE, "abi_worked_example.c")
BINARY = os.path.join(HERE, "abi_worked_example")


def build(verbose: bool = True) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SOURCE, "-o", BINARY + ".tmp",
           "-L", PKG, "-lspecverify", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           # the library is found next to the package wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../speculative_decoding_verification_12_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
