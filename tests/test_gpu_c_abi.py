"""The C ABI called from plain C (tests/host/abi_c_caller.c, built by __graft_entry__.build): device
buffers from the HIP runtime, no Python or torch on the calling side, results against the oracle's
C functions.  The program prints one PASS/FAIL line per check."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "host", "bin", "abi_c_caller")

pytestmark = pytest.mark.gpu


def test_plain_c_caller():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built; run __graft_entry__.build() first")
    print("case: tests/host/bin/abi_c_caller", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.strip().splitlines()
    assert lines[-1] == "ALL PASSED" and not any(l.startswith("FAIL") for l in lines)
    assert sum(l.startswith("PASS") for l in lines) == 13, lines
