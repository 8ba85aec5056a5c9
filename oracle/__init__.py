"""CPU oracle for the grouped MXFP8 scale-factor rearrangement (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The HIP library and its Python binding never do, and this package
imports nothing from them.

The arithmetic lives in ``mx_rearrange_oracle.c``: a plain C loop over groups and
over every position of each group's padded matrix. This module only compiles it
with gcc and calls it through ctypes with host numpy arrays.
"""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "mx_rearrange_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def compile_library(src, dst, verbose=False):
    """Compile one oracle source file into a shared library (plain gcc -O2, one thread)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-o", dst + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(dst + ".tmp", dst)


def build(verbose=False):
    """Compile the oracle into liboracle.so next to its source."""
    compile_library(SOURCE, LIBRARY, verbose)


class Oracle:
    """ctypes front end for one compiled copy of the oracle."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        for name in ("oracle_M_groups_out_bytes", "oracle_K_groups_out_bytes"):
            fn = getattr(lib, name)
            fn.argtypes = [i64, i64, i32]
            fn.restype = i64
        for name in ("oracle_M_groups", "oracle_K_groups"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, i32, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.oracle_3d_out_bytes.argtypes = [i64, i64, i64]
        lib.oracle_3d_out_bytes.restype = i64
        lib.oracle_3d.argtypes = [ctypes.c_void_p, i64, i64, i64, i64, i64, ctypes.c_void_p]
        lib.oracle_3d.restype = ctypes.c_int
        self.lib = lib

    def out_bytes(self, kind, rows, cols, num_groups):
        fn = self.lib.oracle_M_groups_out_bytes if kind == "M" else self.lib.oracle_K_groups_out_bytes
        return int(fn(rows, cols, num_groups))

    def rearrange(self, kind, scales, offs, out=None):
        """Run the oracle on a host (rows, cols) uint8 array with unit column stride.

        ``scales`` may have any row stride >= cols (a strided numpy view); ``offs``
        holds the cumulative int32 group end offsets. Returns the flat uint8
        output of out_bytes(...) bytes. Raises ValueError when the oracle rejects
        the input.
        """
        if scales.dtype != np.uint8 or scales.ndim != 2:
            raise ValueError("scales must be a 2-D uint8 array")
        rows, cols = scales.shape
        if cols > 1 and rows > 0 and scales.strides[1] != 1:
            raise ValueError("scales must have unit column stride")
        ld = scales.strides[0] if rows > 1 else cols
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        G = int(offs.shape[0])
        n = self.out_bytes(kind, rows, cols, G) if G > 0 else 0
        if out is None:
            out = np.empty(max(n, 0), dtype=np.uint8)
        elif out.dtype != np.uint8 or out.size < n or not out.flags.c_contiguous:
            raise ValueError("out must be a contiguous uint8 array of at least %d bytes" % n)
        fn = self.lib.oracle_M_groups if kind == "M" else self.lib.oracle_K_groups
        sp = scales.__array_interface__["data"][0] if rows * cols > 0 else None
        rc = fn(sp, rows, cols, ld, offs.ctypes.data if G > 0 else None, G,
                out.ctypes.data if out.size > 0 else None)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return out[:n]

    def out_bytes_3d(self, experts, rows, cols):
        return int(self.lib.oracle_3d_out_bytes(experts, rows, cols))

    def rearrange_3d(self, scales, out=None):
        """Run the oracle on a host (experts, rows, cols) uint8 array with unit column stride.

        Expert and row strides are taken from the array (any strided view).
        Returns the flat uint8 output of out_bytes_3d(...) bytes.
        """
        if scales.dtype != np.uint8 or scales.ndim != 3:
            raise ValueError("scales must be a 3-D uint8 array")
        E, rows, cols = scales.shape
        if E * rows * cols > 0 and cols > 1 and scales.strides[2] != 1:
            raise ValueError("scales must have unit column stride")
        ld = scales.strides[1] if rows > 1 else cols
        es = scales.strides[0] if E > 1 else rows * ld
        n = self.out_bytes_3d(E, rows, cols)
        if out is None:
            out = np.empty(max(n, 0), dtype=np.uint8)
        sp = scales.__array_interface__["data"][0] if E * rows * cols > 0 else None
        rc = self.lib.oracle_3d(sp, E, rows, cols, es, ld, out.ctypes.data if out.size > 0 else None)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return out[:n]


_default = None


def default():
    """The oracle built from this package's source (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def out_bytes(kind, rows, cols, num_groups):
    return default().out_bytes(kind, rows, cols, num_groups)


def rearrange(kind, scales, offs, out=None):
    return default().rearrange(kind, scales, offs, out)


def out_bytes_3d(experts, rows, cols):
    return default().out_bytes_3d(experts, rows, cols)


def rearrange_3d(scales, out=None):
    return default().rearrange_3d(scales, out)
