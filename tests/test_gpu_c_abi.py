"""The C ABI from plain C: tests/c_abi/c_abi_parity.c (built with the
library) quantizes and rebuilds a small KV set through lynx.h on the GPU
and compares codes, metadata and both reconstructions with the oracle's C
library, and checks that bad arguments are refused."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "c_abi_parity")


def test_c_program_matches_oracle():
    assert os.path.exists(BIN), "build first: python -c 'import __graft_entry__ as g; g.build()'"
    print("[gpu-c-abi] tests/c_abi/c_abi_parity", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "c-abi parity ok" in r.stdout
