"""The library called from plain C (tests/c_abi_main.c, built by
__graft_entry__.build()): header compiled as C99, HIP runtime allocations, the
NULL stream, no PyTorch. The program checks the layer's integer special cases
element by element against the textbook integer products (see its header
comment) and prints "c abi ok"."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi_main")


@pytest.mark.gpu
def test_plain_c_caller_integer_cases():
    if not os.path.exists(BIN):          # normally built beforehand by build()
        from tests import c_abi_build
        c_abi_build.build()
    print("\n  running tests/c_abi_main", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=180)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout
