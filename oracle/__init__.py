"""CPU oracle (test infrastructure) for everything the HIP library computes: the grouped MXFP8
scale-factor rearrangement (M groups, K groups, per-expert 3-D) and its inverse, the MXFP8 casts
(dim0 with M-groups scales, dim1 with K-groups scales, dim1 of stacked expert weights) and the
per-group padding of data rows.

Only the tests (including the plain C caller in tests/c_abi, which links the
compiled oracle), the smoke check and the benchmark's CPU-baseline leg may
import, link or call it. The HIP library and its Python binding never do, and
this package imports nothing from them.

The arithmetic lives in ``mx_rearrange_oracle.c``: a plain C loop over groups and
over every position of each group's padded matrix, and a plain per-block loop for
the quantisation (nearest E4M3 code found by trying every code). This module only
compiles it with gcc and calls it through ctypes with host numpy arrays.
"""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "mx_rearrange_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def compile_library(src, dst, verbose=False):
    """Compile one oracle source file into a shared library (plain gcc -O2). The compiler writes a file of
    this process's own and it replaces `dst` in one step, so processes building at once (parallel test
    workers) neither collide nor load a half-written library."""
    tmp = "%s.tmp%d" % (dst, os.getpid())
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, dst)


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
        for name in ("oracle_M_groups_threads", "oracle_K_groups_threads"):
            fn = getattr(lib, name, None)
            if fn is not None:   # absent from the planted-mistake copies of older sources
                fn.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, i32, ctypes.c_void_p, ctypes.c_int]
                fn.restype = ctypes.c_int
        lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e8m0_of_amax.argtypes = [ctypes.c_double]
        lib.oracle_e8m0_of_amax.restype = ctypes.c_int
        lib.oracle_quantize_dim0.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_quantize_dim0.restype = ctypes.c_int
        lib.oracle_scales_dim0.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p]
        lib.oracle_scales_dim0.restype = ctypes.c_int
        lib.oracle_quantize_dim0_M_groups.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, i32,
                                                      ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_quantize_dim0_M_groups.restype = ctypes.c_int
        lib.oracle_quantize_dim1.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_quantize_dim1.restype = ctypes.c_int
        lib.oracle_quantize_dim1_K_groups.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, i32,
                                                      ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_quantize_dim1_K_groups.restype = ctypes.c_int
        lib.oracle_scales_dim1.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p]
        lib.oracle_scales_dim1.restype = ctypes.c_int
        lib.oracle_pad_M_groups_out_rows.argtypes = [i64, i32]
        lib.oracle_pad_M_groups_out_rows.restype = i64
        lib.oracle_pad_M_groups.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, i32, ctypes.c_void_p]
        lib.oracle_pad_M_groups.restype = ctypes.c_int
        lib.oracle_unpad_M_groups.argtypes = [ctypes.c_void_p, i64, i64, ctypes.c_void_p, i32, ctypes.c_void_p, i64]
        lib.oracle_unpad_M_groups.restype = ctypes.c_int
        for name in ("oracle_unrearrange_M_groups", "oracle_unrearrange_K_groups"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p, i64, i64, ctypes.c_void_p, i32, ctypes.c_void_p, i64]
            fn.restype = ctypes.c_int
        lib.oracle_3d_out_bytes.argtypes = [i64, i64, i64]
        lib.oracle_3d_out_bytes.restype = i64
        lib.oracle_3d.argtypes = [ctypes.c_void_p, i64, i64, i64, i64, i64, ctypes.c_void_p]
        lib.oracle_3d.restype = ctypes.c_int
        lib.oracle_quantize_dim1_3d.argtypes = [ctypes.c_void_p, i64, i64, i64, i64, i64, ctypes.c_void_p,
                                                ctypes.c_void_p]
        lib.oracle_quantize_dim1_3d.restype = ctypes.c_int
        self.lib = lib

    def out_bytes(self, kind, rows, cols, num_groups):
        fn = self.lib.oracle_M_groups_out_bytes if kind == "M" else self.lib.oracle_K_groups_out_bytes
        return int(fn(rows, cols, num_groups))

    def rearrange(self, kind, scales, offs, out=None, threads=None):
        """Run the oracle on a host (rows, cols) uint8 array with unit column stride.

        ``scales`` may have any row stride >= cols (a strided numpy view); ``offs``
        holds the cumulative int32 group end offsets. Returns the flat uint8
        output of out_bytes(...) bytes. Raises ValueError when the oracle rejects
        the input. ``threads`` (an int) shares the one call among that many host
        threads (the same bytes; a CPU baseline spread over cores); None runs the
        single-threaded definition.
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
        sp = scales.__array_interface__["data"][0] if rows * cols > 0 else None
        args = [sp, rows, cols, ld, offs.ctypes.data if G > 0 else None, G, out.ctypes.data if out.size > 0 else None]
        if threads is None:
            fn = self.lib.oracle_M_groups if kind == "M" else self.lib.oracle_K_groups
        else:
            fn = self.lib.oracle_M_groups_threads if kind == "M" else self.lib.oracle_K_groups_threads
            args.append(int(threads))
        rc = fn(*args)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return out[:n]

    def unrearrange(self, kind, blocked, rows, cols, offs):
        """Inverse rearrangement: the (rows, cols) row-major matrix from a blocked output of out_bytes(...) bytes."""
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        G = int(offs.shape[0])
        blocked = np.ascontiguousarray(blocked, dtype=np.uint8).reshape(-1)
        if G < 1 or blocked.size < self.out_bytes(kind, rows, cols, G):
            raise ValueError("blocked input too small")
        out = np.empty((rows, cols), np.uint8)
        fn = self.lib.oracle_unrearrange_M_groups if kind == "M" else self.lib.oracle_unrearrange_K_groups
        rc = fn(blocked.ctypes.data if blocked.size else None, rows, cols, offs.ctypes.data, G,
                out.ctypes.data if out.size else None, cols)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return out

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

    def quantize_dim0(self, x_bits):
        """MXFP8 dim0 cast of a host (rows, K) uint16 array of bf16 bit patterns (any row stride).

        Returns (q, scales): q (rows, K) uint8 E4M3 codes, scales (rows, K/32) uint8 E8M0 bytes.
        """
        rows, K, ld = self._bf16_shape(x_bits)
        q = np.empty((rows, K), np.uint8)
        scales = np.empty((rows, K // 32), np.uint8)
        rc = self.lib.oracle_quantize_dim0(self._ptr(x_bits), rows, K, ld, q.ctypes.data, scales.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return q, scales

    def scales_dim0(self, x_bits):
        """Only the (rows, K/32) E8M0 scale bytes of the dim0 cast."""
        rows, K, ld = self._bf16_shape(x_bits)
        scales = np.empty((rows, K // 32), np.uint8)
        rc = self.lib.oracle_scales_dim0(self._ptr(x_bits), rows, K, ld, scales.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return scales

    def quantize_dim0_M_groups(self, x_bits, offs):
        """dim0 cast whose scales go straight into the M-groups blocked layout.

        Returns (q, blocked): blocked holds out_bytes("M", rows, K/32, G) bytes.
        """
        rows, K, ld = self._bf16_shape(x_bits)
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        G = int(offs.shape[0])
        q = np.empty((rows, K), np.uint8)
        blocked = np.empty(max(self.out_bytes("M", rows, K // 32, G), 1) if G > 0 else 1, np.uint8)
        rc = self.lib.oracle_quantize_dim0_M_groups(self._ptr(x_bits), rows, K, ld,
                                                    offs.ctypes.data if G > 0 else None, G,
                                                    q.ctypes.data, blocked.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return q, blocked[: self.out_bytes("M", rows, K // 32, G)]

    def quantize_dim1(self, x_bits):
        """MXFP8 cast of a host (T, N) bf16 bit-pattern array along T (blocks of 32 tokens).

        Returns (qT, scales): qT (N, T) uint8 codes (transposed), scales (N, T/32) E8M0 bytes.
        """
        T, N, ld = self._bf16_shape(x_bits)
        qT = np.empty((N, T), np.uint8)
        scales = np.empty((N, T // 32), np.uint8)
        rc = self.lib.oracle_quantize_dim1(self._ptr(x_bits), T, N, ld, qT.ctypes.data, scales.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return qT, scales

    def quantize_dim1_3d(self, w_bits):
        """dim1 cast of stacked expert weights: a host (E, K, N) bf16 bit-pattern array (any expert and
        row strides, unit column stride), blocks of 32 along K.

        Returns (q, blocked): q (E, N, K) uint8 codes (each expert transposed), blocked the
        out_bytes_3d(E, N, K/32) bytes of per-expert blocked scales.
        """
        if w_bits.dtype != np.uint16 or w_bits.ndim != 3:
            raise ValueError("weights must be a 3-D uint16 (bf16 bit pattern) array")
        E, K, N = w_bits.shape
        if E * K * N > 0 and N > 1 and w_bits.strides[2] != 2:
            raise ValueError("weights must have unit column stride")
        ld = w_bits.strides[1] // 2 if K > 1 else N
        es = w_bits.strides[0] // 2 if E > 1 else K * ld
        q = np.empty((E, N, K), np.uint8)
        n = self.out_bytes_3d(E, N, K // 32)
        blocked = np.empty(max(n, 1), np.uint8)
        ptr = w_bits.__array_interface__["data"][0] if E * K * N > 0 else None
        rc = self.lib.oracle_quantize_dim1_3d(ptr, E, K, N, es, ld, q.ctypes.data if q.size else None,
                                              blocked.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return q, blocked[:n]

    def scales_dim1(self, x_bits):
        """Only the (N, T/32) E8M0 scale bytes of the dim1 cast of (T, N) bf16 bit patterns."""
        T, N, ld = self._bf16_shape(x_bits)
        scales = np.empty((N, T // 32), np.uint8)
        rc = self.lib.oracle_scales_dim1(self._ptr(x_bits), T, N, ld, scales.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return scales

    def quantize_dim1_K_groups(self, x_bits, offs):
        """dim1 cast whose scales go into the K-groups blocked layout; offs are token offsets (int32).

        Returns (qT, blocked): blocked holds out_bytes("K", N, T/32, G) bytes.
        """
        T, N, ld = self._bf16_shape(x_bits)
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        G = int(offs.shape[0])
        qT = np.empty((N, T), np.uint8)
        n = self.out_bytes("K", N, T // 32, G) if G > 0 else 0
        blocked = np.empty(max(n, 1), np.uint8)
        rc = self.lib.oracle_quantize_dim1_K_groups(self._ptr(x_bits), T, N, ld,
                                                    offs.ctypes.data if G > 0 else None, G,
                                                    qT.ctypes.data, blocked.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return qT, blocked[:n]

    def pad_M_groups(self, data, offs):
        """Per-group row padding of a host (rows, cols) uint8 matrix (any row stride).

        Returns the (rows + 128*G, cols) padded matrix (row stride cols)."""
        if data.dtype != np.uint8 or data.ndim != 2:
            raise ValueError("data must be a 2-D uint8 array")
        rows, cols = data.shape
        if rows > 0 and cols > 1 and data.strides[1] != 1:
            raise ValueError("data must have unit column stride")
        ld = data.strides[0] if rows > 1 else cols
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        G = int(offs.shape[0])
        out_rows = int(self.lib.oracle_pad_M_groups_out_rows(rows, G))
        padded = np.empty((max(out_rows, 0), cols), np.uint8)
        rc = self.lib.oracle_pad_M_groups(self._ptr(data), rows, cols, max(ld, cols), offs.ctypes.data if G else None,
                                          G, padded.ctypes.data if padded.size else None)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return padded

    def unpad_M_groups(self, padded, rows, offs):
        """Inverse of pad_M_groups: (rows, cols) from the (rows + 128*G, cols) padded matrix."""
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        G = int(offs.shape[0])
        cols = padded.shape[1]
        if padded.shape[0] != int(self.lib.oracle_pad_M_groups_out_rows(rows, G)) or not padded.flags.c_contiguous:
            raise ValueError("padded must be a contiguous (rows + 128*G, cols) array")
        data = np.empty((rows, cols), np.uint8)
        rc = self.lib.oracle_unpad_M_groups(self._ptr(padded), rows, cols, offs.ctypes.data if G else None, G,
                                            data.ctypes.data if data.size else None, cols)
        if rc != 0:
            raise ValueError("oracle rejected the input (status %d)" % rc)
        return data

    @staticmethod
    def _bf16_shape(x_bits):
        if x_bits.dtype != np.uint16 or x_bits.ndim != 2:
            raise ValueError("x must be a 2-D uint16 array of bf16 bit patterns")
        rows, K = x_bits.shape
        if rows > 0 and K > 1 and x_bits.strides[1] != 2:
            raise ValueError("x must have unit column stride")
        ld = x_bits.strides[0] // 2 if rows > 1 else K
        return rows, K, ld

    @staticmethod
    def _ptr(a):
        return a.__array_interface__["data"][0] if a.size > 0 else None


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


def rearrange(kind, scales, offs, out=None, threads=None):
    return default().rearrange(kind, scales, offs, out, threads)


def out_bytes_3d(experts, rows, cols):
    return default().out_bytes_3d(experts, rows, cols)


def rearrange_3d(scales, out=None):
    return default().rearrange_3d(scales, out)


def quantize_dim0(x_bits):
    return default().quantize_dim0(x_bits)


def quantize_dim0_M_groups(x_bits, offs):
    return default().quantize_dim0_M_groups(x_bits, offs)


def scales_dim0(x_bits):
    return default().scales_dim0(x_bits)


def quantize_dim1(x_bits):
    return default().quantize_dim1(x_bits)


def quantize_dim1_3d(w_bits):
    return default().quantize_dim1_3d(w_bits)


def quantize_dim1_K_groups(x_bits, offs):
    return default().quantize_dim1_K_groups(x_bits, offs)


def scales_dim1(x_bits):
    return default().scales_dim1(x_bits)


def pad_M_groups(data, offs):
    return default().pad_M_groups(data, offs)


def unpad_M_groups(padded, rows, offs):
    return default().unpad_M_groups(padded, rows, offs)


def unrearrange(kind, blocked, rows, cols, offs):
    return default().unrearrange(kind, blocked, rows, cols, offs)
