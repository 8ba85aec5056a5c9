"""Compiles the gfx950 HIP library in-tree with hipcc (no JIT cache, no torch extension)."""

import os
import re
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", name)
           for name in ("mx_rearrange.hip", "mx_unrearrange.hip", "mx_quantize.hip", "mx_pad.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libmxrearrange.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# DPP instructions whose DPP operand is the second operand of the operation
# (v_subrev_u32_dpp and the like). On gfx950 a v_subrev_u32_dpp has been
# measured to return the operands' difference the other way round, so the
# generated code must hold none of them.
REVERSED_DPP = re.compile(r"\bv_\w*rev\w*_dpp\b")


def device_assembly(source):
    """gfx950 assembly of one source, compiled with the library's flags."""
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "device.s")
        res = subprocess.run([hipcc()] + flags + ["--cuda-device-only", "-S", "-I", INCLUDE, "-o", out, source],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc -S failed for %s:\n%s" % (source, res.stderr))
        with open(out) as f:
            return f.read()


def check_device_code():
    """Raise if any source compiles to a reversed-operand DPP instruction."""
    for src in SOURCES:
        bad = sorted(set(m.group(0) for m in REVERSED_DPP.finditer(device_assembly(src))))
        if bad:
            raise RuntimeError("%s: generated code holds %s" % (os.path.basename(src), ", ".join(bad)))


def build(verbose=False):
    """Compile libmxrearrange.so next to this file. Always recompiles; the result replaces the library in
    one step from a file of this process's own, so concurrent builds neither collide nor expose a
    half-written library."""
    check_device_code()
    tmp = "%s.tmp%d" % (LIBRARY, os.getpid())
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
