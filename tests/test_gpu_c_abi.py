"""The C ABI from plain C (tests/c_abi/abi_check.c): layout -> dispatch ->
combine on the program's own HIP stream, checked against the oracle inside
the program. Built by __graft_entry__.build()."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_check")


def test_c_program_on_the_gpu():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build()"
    print("[gpu-c-abi] running abi_check", flush=True)
    sys.stdout.flush()
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "abi_check ok" in r.stdout, r.stderr
