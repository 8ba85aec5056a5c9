"""The library called from plain C (no Python, no torch) gives the oracle's bytes (GPU).

tests/c_abi/abi_check.c allocates device memory with the HIP runtime, calls the
rearrangement and inverse entry points on a stream of its own and compares the
results with the C oracle; it also checks the documented error returns. It is
compiled by __graft_entry__.build().
"""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECK = os.path.join(ROOT, "tests", "c_abi", "abi_check")


def test_plain_c_caller():
    assert os.path.exists(CHECK), "tests/c_abi/abi_check is missing: run __graft_entry__.build() first"
    print("case plain C caller", CHECK, flush=True)
    res = subprocess.run([CHECK], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("all ok")
