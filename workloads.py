"""Seeded synthetic inputs for the grouped MXFP8 scale rearrangement.

This module only draws inputs: E8M0 scale bytes and cumulative int32 group end
offsets. It holds none of the rearrangement's arithmetic (no padding, no prefix
sums of padded sizes, no layout), so both the CPU oracle and the HIP library can
be fed from it without sharing any of the method.

The named workloads stand in for the shapes the pages benchmark:

* "[mxfp8 moe training] fallback cuda kernel for when input doesn't meet 2d TMA
  constraints", Benchmarks table: M-groups scales of shape (131072, 44), the
  DeepSeek-V3-16B expert shape with 44-byte rows.
* "[mxfp8 moe training] use dim1 cast cuda kernel for 3d weights by reshaping to
  2d", Benchmarks tables: activations A of shape (16640, 5120), whose block-32
  scales are (16640, 160).
* The same page's B operand of shape (E, 8192, 5120) for E = 16 and 64: per-expert
  weight scales of shape (E, 8192, 160), one blocked matrix per expert.
* The same page's activations A of shape (16640, 5120) in bf16, as the input of the
  MXFP8 dim0 cast whose scales go straight into the M-groups blocked layout.
* The dim1 cast of bf16 activations of shape (131072, 7168) (tokens x features), whose
  scales are the (7168, 4096) K-groups shape below.
* "Add CuTeDSL MXFP8 K-groups scale rearrange kernel", realistic-shapes table:
  M x TotalK = 7168 x 131072 and 28672 x 262144 with 8 groups, group widths drawn
  with a granularity of one scale column (the bench's multiple-of-1 option).

No dataset is involved; every value is drawn from numpy's PCG64 generator with
the workload's number as seed, offsets first, then values.
"""

from dataclasses import dataclass

import numpy as np


@dataclass
class Workload:
    name: str            # short identifier
    kind: str            # "M" (groups of rows) or "K" (groups of scale columns)
    rows: int
    cols: int
    offs: np.ndarray     # int32[G], cumulative group end offsets (rows for M, scale cols for K)
    scales: np.ndarray   # uint8[rows, cols], C-contiguous (row stride == cols)
    description: str

    @property
    def num_groups(self) -> int:
        return int(self.offs.shape[0])


def _sorted_cuts(rng, total, n_cuts):
    """n_cuts distinct interior cut points in [1, total), sorted."""
    return np.sort(rng.choice(np.arange(1, total), n_cuts, replace=False))


def _offsets_from_cuts(cuts, total):
    return np.concatenate([cuts, [total]]).astype(np.int32)


def _values(rng, rows, cols, lo, hi):
    return rng.integers(lo, hi + 1, size=(rows, cols), dtype=np.uint8)


def m_groups_tiny(seed=1):
    """(1024, 16) scales, 4 groups whose sizes are not multiples of 128, values in [110, 140]."""
    rng = np.random.default_rng(seed)
    rows, cols = 1024, 16
    while True:
        offs = _offsets_from_cuts(_sorted_cuts(rng, rows, 3), rows)
        sizes = np.diff(np.concatenate([[0], offs]))
        if np.all(sizes % 128 != 0):
            break
    return Workload("m_groups_tiny", "M", rows, cols, offs, _values(rng, rows, cols, 110, 140),
                    "M-groups tiny: uint8 scales (1024, 16), 4 groups")


def m_groups_skinny(seed=2):
    """(131072, 44) scales (44-byte rows), 8 multinomial groups, values in [100, 150]."""
    rng = np.random.default_rng(seed)
    rows, cols, G = 131072, 44, 8
    sizes = rng.multinomial(rows, [1.0 / G] * G)
    offs = np.cumsum(sizes).astype(np.int32)
    return Workload("m_groups_skinny", "M", rows, cols, offs, _values(rng, rows, cols, 100, 150),
                    "M-groups skinny: uint8 scales (131072, 44), 8 groups")


def m_groups_experts(seed=3):
    """(16640, 160) scales, 16 expert groups of which 3 are forced empty, values in [100, 150]."""
    rng = np.random.default_rng(seed)
    rows, cols, G = 16640, 160, 16
    empty = rng.choice(G, 3, replace=False)
    p = np.full(G, 1.0 / (G - 3))
    p[empty] = 0.0
    sizes = rng.multinomial(rows, p)
    offs = np.cumsum(sizes).astype(np.int32)
    return Workload("m_groups_experts", "M", rows, cols, offs, _values(rng, rows, cols, 100, 150),
                    "M-groups: uint8 scales (16640, 160), 16 groups, some empty")


def k_groups(seed=4):
    """M = 7168, TotalK = 131072: (7168, 4096) scales, 8 groups of arbitrary scale-column width."""
    rng = np.random.default_rng(seed)
    rows, cols, G = 7168, 4096, 8
    offs = _offsets_from_cuts(_sorted_cuts(rng, cols, G - 1), cols)
    return Workload("k_groups", "K", rows, cols, offs, _values(rng, rows, cols, 100, 150),
                    "K-groups: uint8 scales (7168, 4096), 8 groups")


def k_groups_large(seed=5):
    """M = 28672, TotalK = 262144: (28672, 8192) scales, 8 groups of arbitrary scale-column width."""
    rng = np.random.default_rng(seed)
    rows, cols, G = 28672, 8192, 8
    offs = _offsets_from_cuts(_sorted_cuts(rng, cols, G - 1), cols)
    return Workload("k_groups_large", "K", rows, cols, offs, _values(rng, rows, cols, 100, 150),
                    "K-groups large: uint8 scales (28672, 8192), 8 groups")


@dataclass
class ExpertWorkload:
    """Per-expert weight scales: E matrices of (rows, cols) scale bytes, no offsets."""
    name: str
    experts: int
    rows: int
    cols: int
    scales: np.ndarray   # uint8[experts, rows, cols]; unit column stride, strides as drawn
    description: str
    kind: str = "3d"


def _expert_values(rng, experts, rows, cols, expert_pad, lo, hi):
    """(experts, rows, cols) bytes in [lo, hi]; expert_pad spare bytes between experts."""
    es = rows * cols + expert_pad
    base = rng.integers(lo, hi + 1, size=max(experts * es, 1), dtype=np.uint8)
    return np.lib.stride_tricks.as_strided(base, shape=(experts, rows, cols), strides=(es, cols, 1))


def experts_3d_small(seed=6):
    """3 experts of (300, 45) scales, 64 spare bytes between experts, values in [1, 255]."""
    rng = np.random.default_rng(seed)
    return ExpertWorkload("experts_3d_small", 3, 300, 45, _expert_values(rng, 3, 300, 45, 64, 1, 255),
                          "3-D expert scales: 3 x (300, 45), experts 64 bytes apart beyond their size")


def experts_3d_e16(seed=7):
    """Weights (16, 8192, 5120): block-32 scales (16, 8192, 160), values in [100, 150]."""
    rng = np.random.default_rng(seed)
    return ExpertWorkload("experts_3d_e16", 16, 8192, 160, _expert_values(rng, 16, 8192, 160, 0, 100, 150),
                          "3-D expert scales: uint8 (16, 8192, 160)")


def experts_3d_e64(seed=8):
    """Weights (64, 8192, 5120): block-32 scales (64, 8192, 160), values in [100, 150]."""
    rng = np.random.default_rng(seed)
    return ExpertWorkload("experts_3d_e64", 64, 8192, 160, _expert_values(rng, 64, 8192, 160, 0, 100, 150),
                          "3-D expert scales: uint8 (64, 8192, 160)")


@dataclass
class QuantWorkload:
    """bf16 activations (as uint16 bit patterns) and group offsets for an MXFP8 cast.

    kind "quant": dim0 cast, rows x K, offsets in rows (M groups). kind "quant_k": dim1 cast,
    rows = T tokens x K = N features, offsets in tokens (K groups of the transposed scales)."""
    name: str
    rows: int
    K: int
    offs: np.ndarray     # int32[G], cumulative group end offsets in rows
    x: np.ndarray        # uint16[rows, K], bf16 bit patterns, C-contiguous
    description: str
    kind: str = "quant"

    @property
    def num_groups(self) -> int:
        return int(self.offs.shape[0])


def _bf16_activations(rng, rows, K, row_exp, zero_block_p):
    """Standard normal values times 2^U{-row_exp..row_exp} per row, a fraction of all-zero
    32-element blocks, truncated to bf16 (the upper 16 bits of each binary32)."""
    v = rng.standard_normal((rows, K), dtype=np.float32)
    v *= (2.0 ** rng.integers(-row_exp, row_exp + 1, size=(rows, 1))).astype(np.float32)
    if zero_block_p > 0:
        zb = rng.random((rows, K // 32)) < zero_block_p
        v.reshape(rows, K // 32, 32)[zb] = 0.0
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def quant_m_groups_small(seed=9):
    """(1000, 640) bf16 activations, 5 groups (one empty, sizes not multiples of 128)."""
    rng = np.random.default_rng(seed)
    rows, K = 1000, 640
    offs = np.array([130, 130, 383, 700, 1000], np.int32)
    return QuantWorkload("quant_m_groups_small", rows, K, offs, _bf16_activations(rng, rows, K, 20, 0.02),
                         "MXFP8 dim0 cast: bf16 (1000, 640), 5 groups")


def quant_m_groups(seed=10):
    """(16640, 5120) bf16 activations, 16 expert groups of which 3 are forced empty."""
    rng = np.random.default_rng(seed)
    rows, K, G = 16640, 5120, 16
    empty = rng.choice(G, 3, replace=False)
    p = np.full(G, 1.0 / (G - 3))
    p[empty] = 0.0
    offs = np.cumsum(rng.multinomial(rows, p)).astype(np.int32)
    return QuantWorkload("quant_m_groups", rows, K, offs, _bf16_activations(rng, rows, K, 8, 0.0),
                         "MXFP8 dim0 cast: bf16 (16640, 5120), 16 groups, some empty")


def quant_m_groups_skinny(seed=19):
    """(131072, 1408) bf16 activations with the 8 groups of m_groups_skinny: the data whose block-32 scales
    are the (131072, 44) M-groups skinny shape (44 scale columns, padded to 48 in the blocked layout)."""
    rng = np.random.default_rng(seed)
    f = m_groups_skinny()
    return QuantWorkload("quant_m_groups_skinny", f.rows, 44 * 32, f.offs,
                         _bf16_activations_chunked(rng, f.rows, 44 * 32, 8),
                         "MXFP8 dim0 cast: bf16 (131072, 1408), the 8 groups of the skinny M-groups shape")


def _bf16_activations_chunked(rng, rows, K, row_exp, chunk_rows=8192):
    """As _bf16_activations without zero blocks, drawn in row chunks to bound host memory."""
    out = np.empty((rows, K), np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = _bf16_activations(rng, r1 - r0, K, row_exp, 0.0)
    return out


def quant_k_groups_small(seed=11):
    """(2048, 312) bf16 tokens x features, 5 token groups (ends multiples of 32, one empty)."""
    rng = np.random.default_rng(seed)
    T, N = 2048, 312
    offs = np.array([320, 320, 1056, 1984, 2048], np.int32)
    return QuantWorkload("quant_k_groups_small", T, N, offs, _bf16_activations(rng, T, N, 20, 0.0),
                         "MXFP8 dim1 cast: bf16 (2048, 312) tokens x features, 5 token groups", kind="quant_k")


def quant_k_groups(seed=12):
    """(131072, 7168) bf16 tokens x features, 8 token groups whose ends are multiples of 32:
    the dim1 cast whose scales are the (7168, 4096) K-groups shape."""
    rng = np.random.default_rng(seed)
    T, N, G = 131072, 7168, 8
    offs = (32 * _offsets_from_cuts(_sorted_cuts(rng, T // 32, G - 1), T // 32)).astype(np.int32)
    return QuantWorkload("quant_k_groups", T, N, offs, _bf16_activations_chunked(rng, T, N, 8),
                         "MXFP8 dim1 cast: bf16 (131072, 7168) tokens x features, 8 token groups", kind="quant_k")


@dataclass
class ExpertQuantWorkload:
    """Stacked expert weights for the dim1 cast written per expert: E matrices of K x N bf16 bit
    patterns (blocks of 32 along K), possibly a strided view (expert and row strides multiples of 8)."""
    name: str
    experts: int
    K: int
    N: int
    w: np.ndarray        # uint16[E, K, N] view, unit column stride
    description: str
    kind: str = "quant_3d"


def quant_3d_small(seed=17):
    """3 experts of (320, 300) bf16, experts 4000 elements apart beyond their size, rows 320 apart."""
    rng = np.random.default_rng(seed)
    E, K, N, ld = 3, 320, 300, 320
    es = K * ld + 4000
    flat = _bf16_activations(rng, (E * es) // ld + 1, ld, 20, 0.02).reshape(-1)
    w = np.lib.stride_tricks.as_strided(flat, shape=(E, K, N), strides=(2 * es, 2 * ld, 2))
    return ExpertQuantWorkload("quant_3d_small", E, K, N, w,
                               "dim1 cast of 3 experts of (320, 300) bf16, strided experts and rows")


def quant_3d_e16(seed=18):
    """16 experts of (5120, 8192) bf16: the weights B (16, 8192, 5120) of the MoE benchmarks, cast along
    the 5120-long reduction dimension; scales (16, 8192, 160)."""
    rng = np.random.default_rng(seed)
    E, K, N = 16, 5120, 8192
    w = _bf16_activations_chunked(rng, E * K, N, 8, chunk_rows=2048).reshape(E, K, N)
    return ExpertQuantWorkload("quant_3d_e16", E, K, N, w,
                               "dim1 cast of expert weights (16, 5120, 8192) bf16, written per expert")


@dataclass
class PadWorkload:
    """MXFP8 data rows (E4M3 code bytes) and M-group offsets for per-group row padding."""
    name: str
    rows: int
    cols: int
    offs: np.ndarray     # int32[G], cumulative group end offsets in rows
    data: np.ndarray     # uint8[rows, cols], C-contiguous
    description: str
    kind: str = "pad"

    @property
    def num_groups(self) -> int:
        return int(self.offs.shape[0])


def pad_m_groups_small(seed=13):
    """(1000, 208) data bytes, 5 groups (one empty, sizes not multiples of 128)."""
    rng = np.random.default_rng(seed)
    rows, cols = 1000, 208
    offs = np.array([130, 130, 383, 700, 1000], np.int32)
    return PadWorkload("pad_m_groups_small", rows, cols, offs, _values(rng, rows, cols, 0, 255),
                       "per-group row padding: uint8 (1000, 208), 5 groups")


def pad_m_groups(seed=14):
    """(16640, 5120) E4M3 data bytes of the activations A, 16 expert groups of which 3 are forced empty."""
    rng = np.random.default_rng(seed)
    rows, cols, G = 16640, 5120, 16
    empty = rng.choice(G, 3, replace=False)
    p = np.full(G, 1.0 / (G - 3))
    p[empty] = 0.0
    offs = np.cumsum(rng.multinomial(rows, p)).astype(np.int32)
    return PadWorkload("pad_m_groups", rows, cols, offs, _values(rng, rows, cols, 0, 255),
                       "per-group row padding: uint8 (16640, 5120), 16 groups, some empty")


@dataclass
class InverseWorkload:
    """Input of the inverse rearrangement: a blocked scale buffer and the group offsets it was laid out with.

    The blocked bytes are drawn at random (every byte, padding included); their
    count is the forward layout's size, supplied by the caller.
    """
    name: str
    kind: str            # "inv_M" or "inv_K"
    rows: int
    cols: int
    offs: np.ndarray     # int32 cumulative group ends (rows for M, scale columns for K)
    seed: int
    description: str

    @property
    def num_groups(self) -> int:
        return int(self.offs.shape[0])

    def blocked(self, n_bytes):
        return np.random.default_rng(self.seed).integers(0, 256, size=n_bytes, dtype=np.uint8)


def inverse_m_groups_skinny(seed=15):
    """The (131072, 44) M-groups scales of m_groups_skinny, read back from a blocked buffer."""
    f = m_groups_skinny()
    return InverseWorkload("inverse_m_groups_skinny", "inv_M", f.rows, f.cols, f.offs, seed,
                           "inverse M-groups: blocked -> (131072, 44) scales, 8 groups")


def inverse_k_groups_large(seed=16):
    """The (28672, 8192) K-groups scales of k_groups_large, read back from a blocked buffer."""
    f = k_groups_large()
    return InverseWorkload("inverse_k_groups_large", "inv_K", f.rows, f.cols, f.offs, seed,
                           "inverse K-groups: blocked -> (28672, 8192) scales, 8 groups")


WORKLOADS = {
    "m_groups_tiny": m_groups_tiny,
    "m_groups_skinny": m_groups_skinny,
    "m_groups_experts": m_groups_experts,
    "k_groups": k_groups,
    "k_groups_large": k_groups_large,
}

WORKLOADS_3D = {
    "experts_3d_small": experts_3d_small,
    "experts_3d_e16": experts_3d_e16,
    "experts_3d_e64": experts_3d_e64,
}


WORKLOADS_QUANT = {
    "quant_m_groups_small": quant_m_groups_small,
    "quant_m_groups": quant_m_groups,
    "quant_m_groups_skinny": quant_m_groups_skinny,
    "quant_k_groups_small": quant_k_groups_small,
    "quant_k_groups": quant_k_groups,
}


WORKLOADS_QUANT_3D = {
    "quant_3d_small": quant_3d_small,
    "quant_3d_e16": quant_3d_e16,
}


WORKLOADS_PAD = {
    "pad_m_groups_small": pad_m_groups_small,
    "pad_m_groups": pad_m_groups,
}


WORKLOADS_INVERSE = {
    "inverse_m_groups_skinny": inverse_m_groups_skinny,
    "inverse_k_groups_large": inverse_k_groups_large,
}


def make(name: str):
    if name in WORKLOADS_INVERSE:
        return WORKLOADS_INVERSE[name]()
    if name in WORKLOADS_QUANT_3D:
        return WORKLOADS_QUANT_3D[name]()
    if name in WORKLOADS_3D:
        return WORKLOADS_3D[name]()
    if name in WORKLOADS_QUANT:
        return WORKLOADS_QUANT[name]()
    if name in WORKLOADS_PAD:
        return WORKLOADS_PAD[name]()
    return WORKLOADS[name]()


def random_offsets(rng, total, num_groups, p_empty=0.25, short_total=False):
    """Cumulative end offsets for num_groups groups over [0, total].

    Groups are made empty with probability p_empty; with short_total the last
    end offset may stop before total (trailing rows or columns in no group).
    """
    end = total
    if short_total and total > 0:
        end = int(rng.integers(0, total + 1))
    cuts = np.sort(rng.integers(0, end + 1, size=num_groups - 1)) if num_groups > 1 else np.zeros(0, np.int64)
    offs = np.concatenate([cuts, [end]]).astype(np.int64)
    # collapse some groups to empty by repeating the previous end
    for g in range(num_groups):
        if rng.random() < p_empty:
            offs[g] = offs[g - 1] if g > 0 else 0
    offs = np.maximum.accumulate(offs)
    return offs.astype(np.int32)


def random_scales(rng, rows, cols, ld=None, lo=1, hi=255):
    """A (rows, cols) uint8 array with row stride ld >= cols (a strided view of a larger buffer)."""
    ld = cols if ld is None else ld
    base = rng.integers(lo, hi + 1, size=max(rows * ld, 1), dtype=np.uint8)
    return np.lib.stride_tricks.as_strided(base[: rows * ld] if rows * ld else base[:0],
                                           shape=(rows, cols), strides=(ld, 1))
