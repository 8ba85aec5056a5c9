"""Host check of the byte ranges the MXFP8 casts derive from their scanned group tables (no GPU).

tests/c_abi/ranges_check.cpp includes the casts' HIP source and runs, on the CPU, the functions
the kernels use to decode each work unit and to size the launch, with group tables built on the
host: with a correct table every byte of the blocked scale allocation and every code is written
exactly once and every access lies inside its buffer; with corrupted tables (every width negated,
random values) every access still lies inside its buffer. The clamping helpers of
csrc/write_ranges.h are checked on their own as well.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_cast_write_ranges_stay_in_bounds(tmp_path):
    from group_scale_factor_amd import _build

    exe = str(tmp_path / "ranges_check")
    res = subprocess.run([_build.hipcc(), "-x", "hip", "--offload-arch=" + _build.ARCH, "-std=c++17", "-O1", "-Wall",
                          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", _build.INCLUDE,
                          "-o", exe, os.path.join(ROOT, "tests", "c_abi", "ranges_check.cpp")],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout[-2000:] + run.stderr[-4000:]
