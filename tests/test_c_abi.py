"""The C ABI used from plain C: a test program (tests/c_abi/abi_worked_example.c, built by
`__graft_entry__.build()`) that includes only spec_verify.h and the HIP runtime's C API, runs the
D3D page's worked greedy round and hand-worked two-token sampling cases, and checks every output
against the values stated in its header comment."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BINARY = os.path.join(HERE, "c_abi", "abi_worked_example")


def test_c_program_is_built():
    assert os.path.exists(BINARY), "run __graft_entry__.build() (it builds tests/c_abi)"


@pytest.mark.gpu
def test_c_program_worked_examples():
    print(f"[gpu] {BINARY}", flush=True)
    r = subprocess.run([BINARY], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().splitlines()[-1] == "ok", r.stdout
