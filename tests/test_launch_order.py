"""Host check of the order in which the kernels deal work units to workgroup slots (no GPU).

tests/c_abi/order_check.cpp includes csrc/launch_order.h and runs, on the CPU, the very functions
the kernels and their launches use: for both orders (contiguous ranges per XCD, runs of units dealt
to the XCDs in turn) and many unit counts and run lengths (among them the forward kernels' runs of
11 K windows and of 4 row blocks), including a last run that is only partly filled, every unit gets
exactly one slot, and an interleaved run stays on one XCD.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_every_unit_gets_one_slot(tmp_path):
    from group_scale_factor_amd import _build

    exe = str(tmp_path / "order_check")
    res = subprocess.run([_build.hipcc(), "-x", "hip", "--offload-arch=" + _build.ARCH, "-std=c++17", "-O1", "-Wall",
                          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", _build.INCLUDE,
                          "-o", exe, os.path.join(ROOT, "tests", "c_abi", "order_check.cpp")],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout[-2000:] + run.stderr[-4000:]
