"""The CPU oracle built with sanitizers (no GPU).

tests/c_abi/oracle_sanitize.c links oracle/mx_rearrange_oracle.c directly and
runs every entry point on exactly-sized heap buffers (edge shapes, strided
rows, many and empty groups, short totals, non-finite inputs, error paths,
round trips through the inverses, the threaded rearrangement against the
single-threaded one). Under AddressSanitizer and UndefinedBehaviorSanitizer any
read or write outside a buffer, and any undefined behaviour, stops it with a
non-zero exit; under ThreadSanitizer so does any data race between the threads
of the threaded rearrangement.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SANITIZERS = {
    "address_ub": (["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
                   {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"}),
    "thread": (["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"}),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("kind", sorted(SANITIZERS))
def test_oracle_under_sanitizers(tmp_path, kind):
    flags, env_add = SANITIZERS[kind]
    exe = str(tmp_path / "oracle_sanitize")
    build = subprocess.run(
        ["gcc", "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror"] + flags + ["-o", exe,
         os.path.join(ROOT, "tests", "c_abi", "oracle_sanitize.c"),
         os.path.join(ROOT, "oracle", "mx_rearrange_oracle.c"), "-pthread", "-lm"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, **env_add)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout[-2000:] + run.stderr[-4000:]
