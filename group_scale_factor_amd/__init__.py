"""Grouped MXFP8 scale-factor rearrangement for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/mx_rearrange.h``. It only
marshals arguments: it checks dtypes and devices, reads sizes and strides,
allocates the output with torch when none is given, and calls the HIP library
on the current torch stream. Every byte of the result is produced by the HIP
kernels; there is no CPU or PyTorch fallback, and importing the binding
fails loudly when the library has not been built.

    out = mx_block_rearrange_M_groups(scales, group_end_offsets)
    out = mx_block_rearrange_K_groups(scales, group_end_offsets)
    out = mx_block_rearrange_3d(expert_scales)
    q, blocked_scales = mx_quantize_dim0_M_groups(x_bf16, group_end_offsets)
    qT, blocked_scales = mx_quantize_dim1_K_groups(x_bf16, token_group_end_offsets)
    q, blocked_scales = mx_quantize_dim1_3d(w_bf16)          # (E, K, N) expert weights, cast along K
    padded = mx_pad_M_groups(data, group_end_offsets)
    scales = mx_block_unrearrange_M_groups(blocked, rows, cols, group_end_offsets)   # and _K_groups
    data = mx_unpad_M_groups(padded, rows, group_end_offsets)

``scales`` is a (rows, cols) uint8 CUDA tensor with unit column stride (any
row stride >= cols, any base alignment); ``group_end_offsets`` an int32 CUDA
tensor of cumulative group ends (rows for M, scale columns for K). The result is
a flat uint8 tensor of ``*_out_bytes(rows, cols, G)`` bytes holding the blocked
128x4-tile layout of every group, padding zeroed. ``expert_scales`` is an
(E, rows, cols) uint8 CUDA tensor with unit column stride (per-expert weight
scales); every expert becomes its own blocked matrix. ``x_bf16`` is a
(rows, K) torch.bfloat16 CUDA tensor (K a multiple of 32, unit column stride);
the MXFP8 cast returns its E4M3 codes as a (rows, K) uint8 tensor and its E8M0
scales already in the M-groups blocked layout.
"""

import ctypes
import os

from . import _build

LIBRARY = _build.LIBRARY

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise ImportError(
            "HIP library %s is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)" % LIBRARY)
    lib = ctypes.CDLL(LIBRARY)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    for name in ("mx_block_rearrange_M_groups", "mx_block_rearrange_K_groups"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, i64, i64, i64, vp, i32, vp, vp]
        fn.restype = ctypes.c_int
    lib.mx_block_rearrange_3d.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp]
    lib.mx_block_rearrange_3d.restype = ctypes.c_int
    lib.mx_quantize_dim0_M_groups.argtypes = [vp, i64, i64, i64, vp, i32, vp, vp, vp]
    lib.mx_quantize_dim0_M_groups.restype = ctypes.c_int
    lib.mx_quantize_dim1_3d.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.mx_quantize_dim1_3d.restype = ctypes.c_int
    lib.mx_quantize_dim1_K_groups.argtypes = [vp, i64, i64, i64, vp, i32, vp, vp, vp]
    lib.mx_quantize_dim1_K_groups.restype = ctypes.c_int
    lib.mx_pad_M_groups.argtypes = [vp, i64, i64, i64, vp, i32, vp, vp]
    lib.mx_pad_M_groups.restype = ctypes.c_int
    lib.mx_unpad_M_groups.argtypes = [vp, i64, i64, vp, i32, vp, i64, vp]
    lib.mx_unpad_M_groups.restype = ctypes.c_int
    for name in ("mx_block_unrearrange_M_groups", "mx_block_unrearrange_K_groups"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, i64, i64, vp, i32, vp, i64, vp]
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def library():
    """The loaded ctypes handle of libmxrearrange.so."""
    return _load()


# Output sizes and status texts. The C headers define these as static inline functions (the library
# exports only the entry points); the same formulas are restated here to size the outputs torch allocates.
# A CPU test compiles the headers and checks every function below against them.

def _round_up(x, m):
    return (x + m - 1) // m * m


def mx_rearrange_M_groups_out_bytes(rows, cols, num_groups):
    """(rows + 128*G) * round_up(cols, 4); -1 for invalid sizes (include/mx_rearrange.h)."""
    if rows < 0 or cols < 0 or num_groups < 1:
        return -1
    return (rows + 128 * num_groups) * _round_up(cols, 4)


def mx_rearrange_K_groups_out_bytes(rows, cols, num_groups):
    """round_up(rows, 128) * (cols + 4*G); -1 for invalid sizes (include/mx_rearrange.h)."""
    if rows < 0 or cols < 0 or num_groups < 1:
        return -1
    return _round_up(rows, 128) * (cols + 4 * num_groups)


def mx_rearrange_3d_out_bytes(experts, rows, cols):
    """E * round_up(rows, 128) * round_up(cols, 4); -1 for invalid sizes (include/mx_rearrange.h)."""
    lim = (1 << 31) - 128
    if experts < 0 or rows < 0 or cols < 0 or rows >= lim or cols >= lim:
        return -1
    per_expert = _round_up(rows, 128) * _round_up(cols, 4)
    if per_expert > 0 and experts > ((1 << 63) - 1) // per_expert:
        return -1
    return experts * per_expert


def mx_quantize_dim0_M_groups_scale_bytes(rows, K, num_groups):
    """(rows + 128*G) * round_up(K/32, 4); -1 for invalid sizes (include/mx_quantize.h)."""
    if rows < 0 or K < 0 or K % 32 != 0 or num_groups < 1:
        return -1
    return (rows + 128 * num_groups) * _round_up(K // 32, 4)


def mx_quantize_dim1_K_groups_scale_bytes(T, N, num_groups):
    """round_up(N, 128) * (T/32 + 4*G); -1 for invalid sizes (include/mx_quantize.h)."""
    if T < 0 or N < 0 or T % 32 != 0 or num_groups < 1:
        return -1
    return _round_up(N, 128) * (T // 32 + 4 * num_groups)


def mx_quantize_dim1_3d_scale_bytes(experts, K, N):
    """E * round_up(N, 128) * round_up(K/32, 4); -1 for invalid sizes (include/mx_quantize.h)."""
    if experts < 0 or K < 0 or N < 0 or K % 32 != 0:
        return -1
    return experts * _round_up(N, 128) * _round_up(K // 32, 4)


def mx_pad_M_groups_out_rows(rows, num_groups):
    """rows + 128*G; -1 for invalid sizes (include/mx_pad.h)."""
    if rows < 0 or num_groups < 1:
        return -1
    return rows + 128 * num_groups


STATUS_TEXT = {
    0: "success",
    -1: "a required pointer is NULL",
    -2: "invalid shape or stride: negative, too large, or a row stride out of its range",
    -3: "num_groups out of range (at least 1; the casts and the inverse also cap it)",
    -4: "a buffer or row stride is not aligned as the entry point requires",
    -5: "HIP kernel launch failed",
}


def mx_rearrange_strerror(status):
    """Text of a status code (include/mx_rearrange.h)."""
    return STATUS_TEXT.get(status, "unknown status")


class RearrangeError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__("mx_block_rearrange failed (%d): %s" % (status, mx_rearrange_strerror(status)))


def _call(kind, scales, group_end_offsets, out, stream):
    import torch

    lib = _load()
    if scales.dtype != torch.uint8 or scales.dim() != 2:
        raise TypeError("scales must be a 2-D torch.uint8 tensor")
    if group_end_offsets.dtype != torch.int32 or group_end_offsets.dim() != 1:
        raise TypeError("group_end_offsets must be a 1-D torch.int32 tensor")
    if not (scales.is_cuda and group_end_offsets.is_cuda):
        raise ValueError("scales and group_end_offsets must be GPU tensors")
    if scales.device != group_end_offsets.device:
        raise ValueError("scales and group_end_offsets must be on the same device")
    if not group_end_offsets.is_contiguous():
        raise ValueError("group_end_offsets must be contiguous")
    rows, cols = scales.shape
    if rows > 1 and cols > 1 and scales.stride(1) != 1:
        raise ValueError("scales must have unit column stride (row-major rows)")
    row_stride = scales.stride(0) if rows > 1 else cols
    G = group_end_offsets.numel()
    size_fn = mx_rearrange_M_groups_out_bytes if kind == "M" else mx_rearrange_K_groups_out_bytes
    n = size_fn(rows, cols, G)
    if n < 0:
        raise ValueError("invalid sizes rows=%d cols=%d num_groups=%d" % (rows, cols, G))
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=scales.device)
    else:
        if out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() < n:
            raise ValueError("out must be a contiguous uint8 tensor of at least %d bytes" % n)
        if out.device != scales.device:
            raise ValueError("out must be on the scales' device")
    if stream is None:
        stream = torch.cuda.current_stream(scales.device).cuda_stream
    fn = lib.mx_block_rearrange_M_groups if kind == "M" else lib.mx_block_rearrange_K_groups
    rc = fn(scales.data_ptr() or None, rows, cols, row_stride, group_end_offsets.data_ptr() or None,
            G, out.data_ptr() or None, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return out


def mx_block_rearrange_M_groups(scales, group_end_offsets, out=None, stream=None):
    """Groups along M: each group's rows padded to 128, columns to 4, blocked 128x4 tiles.

    Returns the flat uint8 output (rows + 128*G) * round_up(cols, 4) bytes long.
    ``stream`` is a raw hipStream_t handle (int); default: torch's current stream.
    """
    return _call("M", scales, group_end_offsets, out, stream)


def mx_block_rearrange_K_groups(scales, group_end_offsets, out=None, stream=None):
    """Groups along K: each group's scale columns padded to 4, rows to 128, one blocked matrix per group.

    Returns the flat uint8 output round_up(rows, 128) * (cols + 4*G) bytes long.
    ``stream`` is a raw hipStream_t handle (int); default: torch's current stream.
    """
    return _call("K", scales, group_end_offsets, out, stream)


def mx_block_rearrange_3d(scales, out=None, stream=None):
    """Per-expert weight scales (E, rows, cols): one blocked matrix per expert.

    Expert e's rows are padded to a multiple of 128 and its columns to a
    multiple of 4; the experts follow one another. Returns the flat uint8 output
    of E * round_up(rows, 128) * round_up(cols, 4) bytes. Any expert and row
    strides (row stride >= cols) with unit column stride.
    ``stream`` is a raw hipStream_t handle (int); default: torch's current stream.
    """
    import torch

    lib = _load()
    if scales.dtype != torch.uint8 or scales.dim() != 3:
        raise TypeError("scales must be a 3-D torch.uint8 tensor")
    if not scales.is_cuda:
        raise ValueError("scales must be a GPU tensor")
    E, rows, cols = scales.shape
    if E * rows * cols > 0 and cols > 1 and scales.stride(2) != 1:
        raise ValueError("scales must have unit column stride")
    row_stride = scales.stride(1) if rows > 1 else cols
    expert_stride = scales.stride(0) if E > 1 else rows * row_stride
    n = mx_rearrange_3d_out_bytes(E, rows, cols)
    if n < 0:
        raise ValueError("invalid sizes experts=%d rows=%d cols=%d" % (E, rows, cols))
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=scales.device)
    else:
        if out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() < n:
            raise ValueError("out must be a contiguous uint8 tensor of at least %d bytes" % n)
        if out.device != scales.device:
            raise ValueError("out must be on the scales' device")
    if stream is None:
        stream = torch.cuda.current_stream(scales.device).cuda_stream
    rc = lib.mx_block_rearrange_3d(scales.data_ptr() or None, E, rows, cols, expert_stride, row_stride,
                                   out.data_ptr() or None, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return out


def _unrearrange(kind, blocked, rows, cols, group_end_offsets, out, stream):
    import torch

    lib = _load()
    if blocked.dtype != torch.uint8 or not blocked.is_cuda or not blocked.is_contiguous():
        raise TypeError("blocked must be a contiguous torch.uint8 GPU tensor")
    _check_offsets(group_end_offsets, blocked.device)
    G = group_end_offsets.numel()
    size_fn = mx_rearrange_M_groups_out_bytes if kind == "M" else mx_rearrange_K_groups_out_bytes
    n = size_fn(rows, cols, G)
    if n < 0 or blocked.numel() < n:
        raise ValueError("blocked must hold the %d bytes of the forward output" % max(n, 0))
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=blocked.device)
    elif out.dtype != torch.uint8 or out.shape != (rows, cols) or out.device != blocked.device or (
            rows > 0 and cols > 1 and out.stride(1) != 1):
        raise ValueError("out must be a (rows, cols) uint8 tensor with unit column stride on the same device")
    row_stride = out.stride(0) if rows > 1 else cols
    if stream is None:
        stream = torch.cuda.current_stream(blocked.device).cuda_stream
    fn = lib.mx_block_unrearrange_M_groups if kind == "M" else lib.mx_block_unrearrange_K_groups
    rc = fn(blocked.data_ptr() or None, rows, cols, group_end_offsets.data_ptr() or None, G,
            out.data_ptr() or None, row_stride, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return out


def mx_block_unrearrange_M_groups(blocked, rows, cols, group_end_offsets, out=None, stream=None):
    """Inverse of mx_block_rearrange_M_groups: the (rows, cols) uint8 scales (zeros past the last group)."""
    return _unrearrange("M", blocked, rows, cols, group_end_offsets, out, stream)


def mx_block_unrearrange_K_groups(blocked, rows, cols, group_end_offsets, out=None, stream=None):
    """Inverse of mx_block_rearrange_K_groups: the (rows, cols) uint8 scales (zeros past the last group)."""
    return _unrearrange("K", blocked, rows, cols, group_end_offsets, out, stream)


def mx_quantize_dim0_M_groups(x, group_end_offsets, q=None, scales=None, stream=None):
    """MXFP8 cast along rows (blocks of 32) with the scales placed in the M-groups blocked layout.

    ``x``: (rows, K) torch.bfloat16 CUDA tensor, unit column stride, 16-byte aligned rows.
    Returns (q, scales): q a (rows, K) uint8 tensor of E4M3 codes (``q.view(torch.float8_e4m3fn)``
    reads them as floats), scales the flat uint8 blocked E8M0 output of
    (rows + 128*G) * round_up(K/32, 4) bytes.
    """
    import torch

    lib = _load()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("x must be a 2-D torch.bfloat16 tensor")
    if group_end_offsets.dtype != torch.int32 or group_end_offsets.dim() != 1:
        raise TypeError("group_end_offsets must be a 1-D torch.int32 tensor")
    if not (x.is_cuda and group_end_offsets.is_cuda) or x.device != group_end_offsets.device:
        raise ValueError("x and group_end_offsets must be GPU tensors on one device")
    if not group_end_offsets.is_contiguous():
        raise ValueError("group_end_offsets must be contiguous")
    rows, K = x.shape
    if rows > 0 and K > 1 and x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    row_stride = x.stride(0) if rows > 1 else K
    G = group_end_offsets.numel()
    n = mx_quantize_dim0_M_groups_scale_bytes(rows, K, G)
    if n < 0:
        raise ValueError("invalid sizes rows=%d K=%d num_groups=%d" % (rows, K, G))
    if q is None:
        q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    elif q.dtype != torch.uint8 or q.shape != (rows, K) or not q.is_contiguous() or q.device != x.device:
        raise ValueError("q must be a contiguous (rows, K) uint8 tensor on x's device")
    if scales is None:
        scales = torch.empty(n, dtype=torch.uint8, device=x.device)
    elif scales.dtype != torch.uint8 or not scales.is_contiguous() or scales.numel() < n or scales.device != x.device:
        raise ValueError("scales must be a contiguous uint8 tensor of at least %d bytes on x's device" % n)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = lib.mx_quantize_dim0_M_groups(x.data_ptr() or None, rows, K, row_stride,
                                       group_end_offsets.data_ptr() or None, G, q.data_ptr() or None,
                                       scales.data_ptr() or None, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return q, scales


def mx_quantize_dim1_K_groups(x, token_group_end_offsets, qT=None, scales=None, stream=None):
    """MXFP8 cast along tokens (blocks of 32 tokens per feature) with scales in the K-groups blocked layout.

    ``x``: (T, N) torch.bfloat16 CUDA tensor (tokens x features), T a multiple of 32, unit column
    stride, 16-byte aligned rows; ``token_group_end_offsets``: int32 cumulative token ends.
    Returns (qT, scales): qT an (N, T) uint8 tensor of E4M3 codes (x transposed), scales the flat uint8
    blocked E8M0 output of round_up(N, 128) * (T/32 + 4*G) bytes.
    """
    import torch

    lib = _load()
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("x must be a 2-D torch.bfloat16 tensor")
    offs = token_group_end_offsets
    if offs.dtype != torch.int32 or offs.dim() != 1:
        raise TypeError("token_group_end_offsets must be a 1-D torch.int32 tensor")
    if not (x.is_cuda and offs.is_cuda) or x.device != offs.device:
        raise ValueError("x and token_group_end_offsets must be GPU tensors on one device")
    if not offs.is_contiguous():
        raise ValueError("token_group_end_offsets must be contiguous")
    T, N = x.shape
    if T > 0 and N > 1 and x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    row_stride = x.stride(0) if T > 1 else N
    G = offs.numel()
    n = mx_quantize_dim1_K_groups_scale_bytes(T, N, G)
    if n < 0:
        raise ValueError("invalid sizes T=%d N=%d num_groups=%d" % (T, N, G))
    if qT is None:
        qT = torch.empty((N, T), dtype=torch.uint8, device=x.device)
    elif qT.dtype != torch.uint8 or qT.shape != (N, T) or not qT.is_contiguous() or qT.device != x.device:
        raise ValueError("qT must be a contiguous (N, T) uint8 tensor on x's device")
    if scales is None:
        scales = torch.empty(n, dtype=torch.uint8, device=x.device)
    elif scales.dtype != torch.uint8 or not scales.is_contiguous() or scales.numel() < n or scales.device != x.device:
        raise ValueError("scales must be a contiguous uint8 tensor of at least %d bytes on x's device" % n)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = lib.mx_quantize_dim1_K_groups(x.data_ptr() or None, T, N, row_stride, offs.data_ptr() or None, G,
                                       qT.data_ptr() or None, scales.data_ptr() or None, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return qT, scales


def _bytes_view(t, name):
    import torch

    if t.element_size() != 1:
        raise TypeError("%s must have 1-byte elements (uint8 or a float8 dtype)" % name)
    return t if t.dtype == torch.uint8 else t.view(torch.uint8)


def _check_offsets(offs, device):
    import torch

    if offs.dtype != torch.int32 or offs.dim() != 1:
        raise TypeError("group_end_offsets must be a 1-D torch.int32 tensor")
    if not offs.is_cuda or offs.device != device:
        raise ValueError("group_end_offsets must be a GPU tensor on the data's device")
    if not offs.is_contiguous():
        raise ValueError("group_end_offsets must be contiguous")


def mx_quantize_dim1_3d(w, q=None, scales=None, stream=None):
    """MXFP8 cast of stacked expert weights along their first matrix dimension, written per expert.

    ``w``: (E, K, N) torch.bfloat16 CUDA tensor (any expert and row strides that are multiples of 8
    elements, unit column stride), K a multiple of 32. Returns (q, scales): q an (E, N, K) uint8
    tensor of E4M3 codes (each expert transposed), scales the flat uint8 per-expert blocked E8M0
    output of E * round_up(N, 128) * round_up(K/32, 4) bytes.
    """
    import torch

    lib = _load()
    if w.dtype != torch.bfloat16 or w.dim() != 3 or not w.is_cuda:
        raise TypeError("w must be a 3-D torch.bfloat16 GPU tensor")
    E, K, N = w.shape
    if E * K * N > 0 and N > 1 and w.stride(2) != 1:
        raise ValueError("w must have unit column stride")
    row_stride = w.stride(1) if K > 1 else N
    expert_stride = w.stride(0) if E > 1 else K * row_stride
    n = mx_quantize_dim1_3d_scale_bytes(E, K, N)
    if n < 0:
        raise ValueError("invalid sizes E=%d K=%d N=%d" % (E, K, N))
    if q is None:
        q = torch.empty((E, N, K), dtype=torch.uint8, device=w.device)
    elif q.dtype != torch.uint8 or q.shape != (E, N, K) or not q.is_contiguous() or q.device != w.device:
        raise ValueError("q must be a contiguous (E, N, K) uint8 tensor on w's device")
    if scales is None:
        scales = torch.empty(n, dtype=torch.uint8, device=w.device)
    elif scales.dtype != torch.uint8 or not scales.is_contiguous() or scales.numel() < n or scales.device != w.device:
        raise ValueError("scales must be a contiguous uint8 tensor of at least %d bytes on w's device" % n)
    if stream is None:
        stream = torch.cuda.current_stream(w.device).cuda_stream
    rc = lib.mx_quantize_dim1_3d(w.data_ptr() or None, E, K, N, expert_stride, row_stride, q.data_ptr() or None,
                                 scales.data_ptr() or None, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return q, scales


def mx_pad_M_groups(data, group_end_offsets, out=None, stream=None):
    """Pads each token group's rows to a multiple of 128 (zero rows), groups stacked as the M-groups scales.

    ``data``: (rows, cols) CUDA tensor of 1-byte elements, unit column stride. Returns the
    (rows + 128*G, cols) uint8 padded tensor (group g's rows start at the sum of the earlier groups'
    padded sizes; every other row is zero).
    """
    import torch

    lib = _load()
    if data.dim() != 2:
        raise TypeError("data must be a 2-D tensor")
    d = _bytes_view(data, "data")
    if not d.is_cuda:
        raise ValueError("data must be a GPU tensor")
    _check_offsets(group_end_offsets, d.device)
    rows, cols = d.shape
    if rows > 0 and cols > 1 and d.stride(1) != 1:
        raise ValueError("data must have unit column stride")
    row_stride = d.stride(0) if rows > 1 else cols
    G = group_end_offsets.numel()
    out_rows = mx_pad_M_groups_out_rows(rows, G)
    if out_rows < 0:
        raise ValueError("invalid sizes rows=%d num_groups=%d" % (rows, G))
    if out is None:
        out = torch.empty((out_rows, cols), dtype=torch.uint8, device=d.device)
    elif out.dtype != torch.uint8 or out.shape != (out_rows, cols) or not out.is_contiguous() or out.device != d.device:
        raise ValueError("out must be a contiguous (%d, %d) uint8 tensor on the data's device" % (out_rows, cols))
    if stream is None:
        stream = torch.cuda.current_stream(d.device).cuda_stream
    rc = lib.mx_pad_M_groups(d.data_ptr() or None, rows, cols, row_stride, group_end_offsets.data_ptr() or None, G,
                             out.data_ptr() or None, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return out


def mx_unpad_M_groups(padded, rows, group_end_offsets, out=None, stream=None):
    """Inverse of mx_pad_M_groups: the (rows, cols) uint8 tensor of each group's rows (zeros past the last end).

    ``padded``: contiguous (rows + 128*G, cols) CUDA tensor of 1-byte elements. ``out`` may be any
    (rows, cols) uint8 view with unit column stride (its row stride is kept).
    """
    import torch

    lib = _load()
    if padded.dim() != 2:
        raise TypeError("padded must be a 2-D tensor")
    src = _bytes_view(padded, "padded")
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("padded must be a contiguous GPU tensor")
    _check_offsets(group_end_offsets, src.device)
    G = group_end_offsets.numel()
    cols = src.shape[1]
    if src.shape[0] != mx_pad_M_groups_out_rows(rows, G):
        raise ValueError("padded must have rows + 128*G rows")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    elif out.dtype != torch.uint8 or out.shape != (rows, cols) or out.device != src.device or (
            rows > 0 and cols > 1 and out.stride(1) != 1):
        raise ValueError("out must be a (rows, cols) uint8 tensor with unit column stride on the same device")
    row_stride = out.stride(0) if rows > 1 else cols
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    rc = lib.mx_unpad_M_groups(src.data_ptr() or None, rows, cols, group_end_offsets.data_ptr() or None, G,
                               out.data_ptr() or None, row_stride, stream or None)
    if rc != 0:
        raise RearrangeError(rc)
    return out


__all__ = [
    "mx_quantize_dim1_3d",
    "mx_quantize_dim1_3d_scale_bytes",
    "mx_block_unrearrange_M_groups",
    "mx_block_unrearrange_K_groups",
    "mx_pad_M_groups",
    "mx_unpad_M_groups",
    "mx_quantize_dim1_K_groups",
    "mx_quantize_dim1_K_groups_scale_bytes",
    "mx_quantize_dim0_M_groups",
    "mx_quantize_dim0_M_groups_scale_bytes",
    "mx_block_rearrange_3d",
    "mx_rearrange_3d_out_bytes",
    "mx_block_rearrange_M_groups",
    "mx_block_rearrange_K_groups",
    "mx_rearrange_M_groups_out_bytes",
    "mx_rearrange_K_groups_out_bytes",
    "mx_pad_M_groups_out_rows",
    "mx_rearrange_strerror",
    "RearrangeError",
    "library",
]
