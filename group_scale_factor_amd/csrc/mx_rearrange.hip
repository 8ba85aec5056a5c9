// Grouped MXFP8 scale-factor rearrangement for gfx950 (MI355X).
//
// Moves E8M0 scale bytes from a row-major (rows x cols) matrix into the
// blocked, swizzled layout of 128x4 tiles, one group at a time, with groups
// along M (rows) or K (scale columns). Pages this follows (pytorch/ao pull
// requests): "[mxfp8 moe training] compute prefix sum of group sizes inside
// kernel intead of precomputing" (Context, Changes: padded group starts as an
// in-kernel prefix sum); "[mxfp8 moe training] fallback cuda kernel for when
// input doesn't meet 2d TMA constraints" (Context: any row width, no 16-byte
// stride rule); "[mxfp8 moe training] add bench script for scale conversion to
// blocked format kernels for groups along K" (128x4 tiles per group along K);
// "Add CuTeDSL MXFP8 K-groups scale rearrange kernel" (review: widths padded to
// 4 columns, empty groups, zero padding, 128-bit loads with a byte-exact
// fallback).
//
// The work is pure data movement, bound by HBM bandwidth; there is no
// arithmetic on the scale values. Design:
//   * One workgroup (4 wave64s) handles one work unit: 128 rows x up to 256
//     padded scale columns of one group, i.e. up to 64 output tiles, which are
//     contiguous in the output (up to 32 KiB written with 16-byte stores).
//   * Group lookup: every wave loads the end offsets, one group per lane,
//     clamps them into a non-decreasing sequence, and forms the padded sizes
//     and their prefix sums with wave shuffles; a ballot over the cumulative
//     unit counts names the group of the unit. G > 64 is handled in 64-lane
//     slices with a carry.
//   * Load: the unit's source bytes are fetched as 16-byte aligned pieces
//     (global_load_dwordx4) covering each row segment (or, for contiguous
//     skinny rows, the whole strip as one range) and staged in LDS. A 16-byte
//     aligned piece that contains at least one byte of the matrix lies inside
//     the same memory page as that byte, so the cover never touches a page
//     the matrix does not; the extra bytes are never emitted.
//   * Interleave: after one barrier each lane assembles one 16-byte output
//     unit — the same 4-byte column word of rows i, i+32, i+64, i+96 of the
//     tile — from LDS. When the source is not 4-byte aligned each word is
//     assembled from two aligned LDS words with v_alignbyte_b32. Bytes past
//     the group's rows or columns are masked to zero.
//   * Store: consecutive lanes write consecutive 16 bytes (global_store_dwordx4).
//   * The whole output allocation is written exactly once by the same launch:
//     work units past the last group's data zero-fill the tail, so the output
//     needs no memset.
//   * Work units are spread over the 8 XCDs so that units that are neighbours
//     in the output run on the same XCD (workgroups are dealt to XCDs
//     round-robin), keeping shared boundary cache lines in one L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "mx_rearrange.h"

namespace {

constexpr int kThreads = 256;                 // 4 wave64s
constexpr int kWave = 64;
constexpr int kTileRows = 128;
constexpr int kUnitCols = 256;                // padded scale columns per work unit
constexpr int kMaxPieces = (kUnitCols + 30) / 16;            // 16-byte pieces covering one row segment
constexpr int kMaxPitch = 16 * kMaxPieces + 4;               // LDS row pitch: 4*pieces+1 words, odd
constexpr int kLdsSlack = 16;                 // room for the second word of an unaligned read
constexpr int kMaxLdsBytes = kTileRows * kMaxPitch + kLdsSlack;
constexpr int kMaxLoadIters = (kTileRows * kMaxPieces + kThreads - 1) / kThreads;
constexpr int64_t kMaxGrid = int64_t(1) << 20;
constexpr int64_t kMaxRowStride = int64_t(1) << 24;   // keeps a unit's byte span inside 32-bit buffer offsets
constexpr uint32_t kOutOfRange = 0xfffffff0u;          // buffer offset past any range: the load returns 0
constexpr int kRawBufferFlags = 0x00020000;            // buffer descriptor word 3: 32-bit raw data

static_assert(kUnitCols % 16 == 0, "unit width must be a multiple of 16 columns");
static_assert(kMaxLdsBytes <= 64 * 1024, "LDS per workgroup");

struct Params {
  const uint8_t *src;
  const int32_t *offs;
  uint8_t *out;
  int64_t ld;          // row stride in bytes
  int64_t out_bytes;   // whole output allocation
  int64_t units;       // work units
  int64_t vunits;      // units rounded up to a multiple of 8
  int rows;
  int cols;
  int groups;
  int padded_cols;     // M: round_up(cols, 4)
  int unit_cols;       // M: columns per unit in a row block; K: kUnitCols
  int per_row;         // M: units per output row block; K: units per 128-row block
  int pitch;           // LDS row pitch (bytes) in per-row staging
  int pieces;          // 16-byte pieces per LDS row in per-row staging
  int flat;            // M only: stage each 128-row strip as one contiguous range
};

// ---------------------------------------------------------------------------
// wave64 helpers
// ---------------------------------------------------------------------------

__device__ inline int wave_inclusive_sum(int x, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ inline int wave_inclusive_max(int x, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x = max(x, y);
  }
  return x;
}

__device__ inline int lane_value(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// ---------------------------------------------------------------------------
// group scan and lookup
// ---------------------------------------------------------------------------

// Where a work unit sits among the groups. Group sizes are counted in rows (M)
// or scale columns (K); "units" are 128-row blocks (M) or kUnitCols-column
// chunks of one 128-row block (K).
struct GroupHit {
  int group;        // index of the group holding the unit; == groups for the tail
  int start;        // first input row (M) / column (K) of the group
  int size;         // rows (M) / columns (K) of the group
  int first_unit;   // units of all earlier groups
  int padded_start; // K: padded columns of all earlier groups
  int total_units;  // tail only: units of all groups
  int total_padded; // tail only (K): padded columns of all groups
};

// Scans the cumulative end offsets in 64-lane slices and finds the group that
// holds unit `target`. limit = rows (M) or cols (K): each end offset is clamped
// into [previous end, limit], which leaves valid offsets unchanged and keeps
// every access in bounds for invalid ones.
template <bool KGROUPS>
__device__ GroupHit find_group(const int32_t *__restrict__ offs, int groups, int limit,
                               int target, int lane) {
  int carry_end = 0, carry_units = 0, carry_padded = 0;
  for (int base = 0; base < groups; base += kWave) {
    const int g = base + lane;
    const bool active = g < groups;
    int end = active ? offs[g] : 0;
    end = min(max(end, 0), limit);
    end = max(wave_inclusive_max(end, lane), carry_end);
    int prev = __shfl_up(end, 1, kWave);
    if (lane == 0) prev = carry_end;
    const int size = end - prev;                       // 0 for lanes past the last group
    const int padded = KGROUPS ? (size + 3) & ~3 : 0;  // K: width padded to 4 columns
    const int units = KGROUPS ? (padded + kUnitCols - 1) / kUnitCols : (size + kTileRows - 1) / kTileRows;
    const int cum_units = wave_inclusive_sum(units, lane) + carry_units;
    const int cum_padded = KGROUPS ? wave_inclusive_sum(padded, lane) + carry_padded : 0;
    const unsigned long long before = __ballot(active && cum_units <= target);
    const int n = __popcll(before);
    const int in_slice = min(kWave, groups - base);
    if (n < in_slice) {
      GroupHit h;
      h.group = base + n;
      h.start = lane_value(prev, n);
      h.size = lane_value(size, n);
      h.first_unit = lane_value(cum_units, n) - lane_value(units, n);
      h.padded_start = KGROUPS ? lane_value(cum_padded, n) - lane_value(padded, n) : 0;
      h.total_units = 0;
      h.total_padded = 0;
      return h;
    }
    carry_end = lane_value(end, kWave - 1);
    carry_units = lane_value(cum_units, kWave - 1);
    carry_padded = KGROUPS ? lane_value(cum_padded, kWave - 1) : 0;
  }
  GroupHit h;
  h.group = groups;
  h.start = carry_end;
  h.size = 0;
  h.first_unit = carry_units;
  h.padded_start = carry_padded;
  h.total_units = carry_units;
  h.total_padded = carry_padded;
  return h;
}

// ---------------------------------------------------------------------------
// zero-fill of a byte range [lo, hi) split into `parts` parts; lo is 16-byte
// aligned and hi a multiple of 4
// ---------------------------------------------------------------------------

__device__ inline void zero_part(uint8_t *__restrict__ out, int64_t lo, int64_t hi, int64_t part,
                                 int64_t parts) {
  const int64_t len16 = (hi - lo + 15) >> 4;
  const int64_t per = (len16 + parts - 1) / parts;
  const int64_t b = lo + 16 * min(per * part, len16);
  const int64_t e = min(lo + 16 * min(per * (part + 1), len16), hi);
  const int64_t full = b + ((e - b) & ~int64_t(15));
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int64_t p = b + 16 * threadIdx.x; p < full; p += 16 * kThreads)
    *reinterpret_cast<uint4 *>(out + p) = z;
  for (int64_t p = full + 4 * threadIdx.x; p < e; p += 4 * kThreads)
    *reinterpret_cast<uint32_t *>(out + p) = 0u;
}

// ---------------------------------------------------------------------------
// staging a 128-row strip in LDS
// ---------------------------------------------------------------------------

// Buffer resource over [base, base + bytes) for raw (unswizzled) buffer loads.
// A load whose offset lies past `bytes` returns zeros and touches no memory,
// which lets every lane issue its loads unconditionally.
__device__ inline __amdgpu_buffer_rsrc_t byte_buffer(const uint8_t *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, int(bytes), kRawBufferFlags);
}

__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t offset) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(offset), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Per-row staging: row r's segment [a, a + seg) with a = row_base + r*ld is
// fetched as the 16-byte pieces covering it and stored at LDS r*pitch; its
// first byte then sits at r*pitch + (a mod 16).
__device__ inline void stage_rows(uint8_t *__restrict__ lds, const uint8_t *row_base, int64_t ld,
                                  int nrows, int seg, int pitch, int pieces) {
  const uint32_t lead = uint32_t(reinterpret_cast<uintptr_t>(row_base) & 15);
  const uint8_t *base = row_base - lead;  // 16-byte aligned
  const uint32_t span = uint32_t((lead + int64_t(nrows - 1) * ld + seg + 15) & ~int64_t(15));
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(base, span);
  const int step_r = kThreads / pieces, step_k = kThreads % pieces;
  int r = threadIdx.x / pieces, k = threadIdx.x % pieces;
  uint4 v[kMaxLoadIters];
  uint32_t lds_off[kMaxLoadIters];
#pragma unroll
  for (int it = 0; it < kMaxLoadIters; ++it) {
    const uint32_t row_off = lead + uint32_t(r) * uint32_t(ld);  // in range whenever r < nrows
    const int need = int(((row_off & 15) + seg + 15) >> 4);
    const bool valid = r < nrows && k < need;
    v[it] = load16(rsrc, valid ? (row_off & ~15u) + 16 * k : kOutOfRange);
    lds_off[it] = valid ? uint32_t(r * pitch + 16 * k) : kOutOfRange;
    r += step_r;
    k += step_k;
    if (k >= pieces) { k -= pieces; ++r; }
  }
#pragma unroll
  for (int it = 0; it < kMaxLoadIters; ++it) {
    if (lds_off[it] != kOutOfRange) {
      uint32_t *d = reinterpret_cast<uint32_t *>(lds + lds_off[it]);
      d[0] = v[it].x;
      d[1] = v[it].y;
      d[2] = v[it].z;
      d[3] = v[it].w;
    }
  }
}

// Flat staging: the strip is one contiguous range [a, a + len); its 16-byte
// cover is copied to LDS from offset 0, so byte a sits at LDS (a mod 16).
__device__ inline void stage_flat(uint8_t *__restrict__ lds, const uint8_t *start, int len) {
  const uint32_t lead = uint32_t(reinterpret_cast<uintptr_t>(start) & 15);
  const int n = int((lead + len + 15) >> 4);
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(start - lead, uint32_t(16 * n));
  uint4 v[kMaxLoadIters];
#pragma unroll
  for (int it = 0; it < kMaxLoadIters; ++it) {
    const int k = threadIdx.x + it * kThreads;
    v[it] = load16(rsrc, k < n ? uint32_t(16 * k) : kOutOfRange);
  }
#pragma unroll
  for (int it = 0; it < kMaxLoadIters; ++it) {
    const int k = threadIdx.x + it * kThreads;
    if (k < n) *reinterpret_cast<uint4 *>(lds + 16 * k) = v[it];
  }
}

// ---------------------------------------------------------------------------
// emitting tiles from LDS
// ---------------------------------------------------------------------------

// Writes `tile_cols` tiles (128 rows x 4 columns each) contiguously at dst.
// Row r, column c of the unit is LDS byte row_off(r) + c with
// row_off(r) = first + r*row_step + (per_row_shift ? (addr + r*ld) mod 16 : 0).
// Rows >= nrows and columns >= ncols are written as zero.
template <bool ALIGNED>
__device__ inline void emit_tiles(const uint8_t *__restrict__ lds, uint8_t *__restrict__ dst, int tile_cols,
                                  int nrows, int ncols, int first, int row_step, bool per_row_shift,
                                  uintptr_t addr, int64_t ld) {
  const uint32_t *w32 = reinterpret_cast<const uint32_t *>(lds);
  const int n16 = tile_cols * 32;
  for (int v = threadIdx.x; v < n16; v += kThreads) {
    const int tc = v >> 5;
    const int i = v & 31;
    const int nvalid = ncols - 4 * tc;
    const uint32_t mask = nvalid >= 4 ? 0xffffffffu : (nvalid <= 0 ? 0u : (1u << (8 * nvalid)) - 1u);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = i + 32 * q;
      uint32_t x = 0;
      if (r < nrows) {
        int b = first + r * row_step + 4 * tc;
        if (per_row_shift) b += int((addr + uintptr_t(int64_t(r) * ld)) & 15);
        if (ALIGNED) {
          x = w32[b >> 2];
        } else {
          x = __builtin_amdgcn_alignbyte(w32[(b >> 2) + 1], w32[b >> 2], b & 3);
        }
        x &= mask;
      }
      w[q] = x;
    }
    *reinterpret_cast<uint4 *>(dst + 16 * int64_t(v)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Stages one unit of `nrows` rows x `ncols` source columns starting at
// row_base (row stride ld) and writes its tile_cols tiles at dst.
__device__ inline void copy_unit(uint8_t *__restrict__ lds, const Params &p, const uint8_t *row_base,
                                 int nrows, int ncols, int tile_cols, uint8_t *dst, bool flat) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(row_base);
  bool aligned;
  if (flat) {
    stage_flat(lds, row_base, nrows * ncols);
    aligned = ((a & 3) == 0) && ((ncols & 3) == 0);
  } else {
    stage_rows(lds, row_base, p.ld, nrows, ncols, p.pitch, p.pieces);
    aligned = ((a & 3) == 0) && ((p.ld & 3) == 0);
  }
  __syncthreads();
  const int first = flat ? int(a & 15) : 0;
  const int step = flat ? ncols : p.pitch;
  if (aligned)
    emit_tiles<true>(lds, dst, tile_cols, nrows, ncols, first, step, !flat, a, p.ld);
  else
    emit_tiles<false>(lds, dst, tile_cols, nrows, ncols, first, step, !flat, a, p.ld);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <bool KGROUPS>
__global__ __launch_bounds__(kThreads) void rearrange_kernel(Params p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & (kWave - 1);
  bool first_iter = true;
  for (int64_t vb = blockIdx.x; vb < p.vunits; vb += gridDim.x) {
    // consecutive units on one XCD: workgroup b runs on XCD b mod 8
    const int64_t unit = (vb & 7) * (p.vunits >> 3) + (vb >> 3);
    if (unit >= p.units) continue;
    if (!first_iter) __syncthreads();  // LDS of the previous unit is no longer read
    first_iter = false;

    const int64_t block = unit / p.per_row;             // output row block (M) / 128-row block (K)
    const int slot = int(unit - block * p.per_row);     // column chunk (M) / unit within the row block (K)

    if (!KGROUPS) {
      const GroupHit h = find_group<false>(p.offs, p.groups, p.rows, int(block), lane);
      const int64_t row_block_bytes = int64_t(kTileRows) * p.padded_cols;
      if (h.group < p.groups) {
        const int k = int(block) - h.first_unit;
        const int row0 = h.start + kTileRows * k;
        const int nrows = min(kTileRows, h.size - kTileRows * k);
        const int c0 = slot * p.unit_cols;
        const int ncols = min(p.unit_cols, p.cols - c0);
        const int tile_cols = min(p.unit_cols, p.padded_cols - c0) >> 2;
        uint8_t *dst = p.out + block * row_block_bytes + int64_t(c0) * kTileRows;
        copy_unit(lds, p, p.src + int64_t(row0) * p.ld + c0, nrows, ncols, tile_cols, dst, p.flat != 0);
      } else {
        const int64_t tail_units = (int64_t(p.per_row) * ((p.units / p.per_row) - h.total_units));
        const int64_t tail_index = (block - h.total_units) * p.per_row + slot;
        zero_part(p.out, int64_t(h.total_units) * row_block_bytes, p.out_bytes, tail_index, tail_units);
      }
    } else {
      const GroupHit h = find_group<true>(p.offs, p.groups, p.cols, slot, lane);
      const int64_t padded_rows = int64_t(((p.rows + kTileRows - 1) / kTileRows)) * kTileRows;
      if (h.group < p.groups) {
        const int chunk = slot - h.first_unit;
        const int padded_width = (h.size + 3) & ~3;
        const int c0 = h.start + chunk * kUnitCols;
        const int nrows = min(kTileRows, p.rows - kTileRows * int(block));
        const int ncols = min(kUnitCols, h.size - chunk * kUnitCols);
        const int tile_cols = min(kUnitCols, padded_width - chunk * kUnitCols) >> 2;
        uint8_t *dst = p.out + padded_rows * h.padded_start + block * kTileRows * padded_width +
                       int64_t(chunk) * kUnitCols * kTileRows;
        copy_unit(lds, p, p.src + block * kTileRows * p.ld + c0, nrows, ncols, tile_cols, dst, false);
      } else {
        // tail: round_up(rows,128) * (cols + 4G - padded total) zero bytes, a
        // 128 * (cols + 4G - padded total) slice per 128-row block
        const int64_t tail_cols = int64_t(p.cols) + 4 * int64_t(p.groups) - h.total_padded;
        const int64_t lo = padded_rows * h.total_padded + block * kTileRows * tail_cols;
        zero_part(p.out, lo, lo + kTileRows * tail_cols, slot - h.total_units, p.per_row - h.total_units);
      }
    }
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

bool sizes_ok(int64_t rows, int64_t cols, int64_t ld, int32_t groups) {
  if (rows < 0 || cols < 0 || ld < cols || ld > kMaxRowStride) return false;
  if (groups < 1) return true;  // reported separately
  const int64_t lim = (int64_t(1) << 31) - 1;
  return rows <= lim - 128 * int64_t(groups) && cols <= lim - 4 * int64_t(groups);
}

int launch(bool kgroups, const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld,
           const int32_t *offs, int32_t groups, uint8_t *out, hipStream_t stream) {
  if (!sizes_ok(rows, cols, ld, groups)) return MX_REARRANGE_ESHAPE;
  if (groups < 1) return MX_REARRANGE_EGROUPS;
  const int64_t out_bytes = kgroups ? mx_rearrange_K_groups_out_bytes(rows, cols, groups)
                                    : mx_rearrange_M_groups_out_bytes(rows, cols, groups);
  if (offs == nullptr) return MX_REARRANGE_ENULL;
  if (rows * cols > 0 && scales == nullptr) return MX_REARRANGE_ENULL;
  if (out_bytes > 0 && out == nullptr) return MX_REARRANGE_ENULL;
  if (reinterpret_cast<uintptr_t>(out) & 15) return MX_REARRANGE_EALIGN;
  if (out_bytes == 0) return MX_REARRANGE_OK;

  Params p;
  p.src = scales;
  p.offs = offs;
  p.out = out;
  p.ld = ld;
  p.out_bytes = out_bytes;
  p.rows = int(rows);
  p.cols = int(cols);
  p.groups = groups;
  p.padded_cols = int(round_up(cols, 4));
  const int64_t seg = std::min<int64_t>(cols, kUnitCols);   // widest row segment of a unit
  p.pieces = int((seg + 30) / 16);
  if (p.pieces < 1) p.pieces = 1;
  p.pitch = 16 * p.pieces + 4;
  int64_t units;
  if (!kgroups) {
    p.unit_cols = kUnitCols;
    p.per_row = int((p.padded_cols + kUnitCols - 1) / kUnitCols);
    // row blocks: every group's data plus at least one block of tail
    units = ((rows + kTileRows - 1) / kTileRows + groups) * p.per_row;
    // one contiguous range per strip when rows are packed, narrow and not 16-byte multiples
    p.flat = (ld == cols && p.per_row == 1 && (cols % 16) != 0) ? 1 : 0;
  } else {
    p.unit_cols = kUnitCols;
    // units per 128-row block: every group's chunks plus at least one of tail
    p.per_row = int((cols + 4 * int64_t(groups) + kUnitCols - 1) / kUnitCols + groups);
    units = ((rows + kTileRows - 1) / kTileRows) * p.per_row;
    p.flat = 0;
  }
  p.units = units;
  p.vunits = round_up(units, 8);
  const int64_t grid = std::min<int64_t>(p.vunits, kMaxGrid);
  size_t lds_bytes = p.flat ? size_t(kTileRows) * size_t(cols) + 32 + kLdsSlack
                            : size_t(kTileRows) * size_t(p.pitch) + kLdsSlack;
  lds_bytes = (lds_bytes + 15) & ~size_t(15);

  void *args[] = {&p};
  const void *fn = kgroups ? reinterpret_cast<const void *>(&rearrange_kernel<true>)
                           : reinterpret_cast<const void *>(&rearrange_kernel<false>);
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(kThreads), args, lds_bytes, stream);
  return e == hipSuccess ? MX_REARRANGE_OK : MX_REARRANGE_ELAUNCH;
}

}  // namespace

extern "C" {

int64_t mx_rearrange_M_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups) {
  if (rows < 0 || cols < 0 || num_groups < 1) return -1;
  return (rows + 128 * int64_t(num_groups)) * round_up(cols, 4);
}

int64_t mx_rearrange_K_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups) {
  if (rows < 0 || cols < 0 || num_groups < 1) return -1;
  return round_up(rows, 128) * (cols + 4 * int64_t(num_groups));
}

int mx_block_rearrange_M_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t row_stride,
                                const int32_t *group_end_offsets, int32_t num_groups, uint8_t *out,
                                hipStream_t stream) {
  return launch(false, scales, rows, cols, row_stride, group_end_offsets, num_groups, out, stream);
}

int mx_block_rearrange_K_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t row_stride,
                                const int32_t *group_end_offsets, int32_t num_groups, uint8_t *out,
                                hipStream_t stream) {
  return launch(true, scales, rows, cols, row_stride, group_end_offsets, num_groups, out, stream);
}

const char *mx_rearrange_strerror(int status) {
  switch (status) {
    case MX_REARRANGE_OK: return "success";
    case MX_REARRANGE_ENULL: return "a required pointer is NULL";
    case MX_REARRANGE_ESHAPE: return "invalid shape: rows/cols negative or too large, or row_stride < cols";
    case MX_REARRANGE_EGROUPS: return "num_groups must be >= 1";
    case MX_REARRANGE_EALIGN: return "out must be 16-byte aligned";
    case MX_REARRANGE_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
