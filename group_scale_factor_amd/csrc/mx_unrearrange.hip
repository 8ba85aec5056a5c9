// The inverse rearrangement for gfx950 (MI355X): blocked, swizzled 128x4-tile
// scales back to the row-major scale matrix, for groups along M and along K.
//
// The layout read is the one the forward kernels write (pages: "[mxfp8 moe
// training] compute prefix sum of group sizes inside kernel intead of
// precomputing", Context and Changes; "[mxfp8 moe training] add bench script
// for scale conversion to blocked format kernels for groups along K",
// description; "Add CuTeDSL MXFP8 K-groups scale rearrange kernel", review
// notes): element (r, c) of a tile at byte (r mod 32)*16 + (r div 32)*4 + c,
// tiles row-major, M groups stacked with rows padded to 128, K groups each its
// own blocked matrix with the width padded to 4. The pages describe no inverse
// kernel; this one reads every byte the forward map placed and writes zeros
// where no group holds data (rows past the last end for M, columns past the
// last end for K).
//
// A unit is the forward kernel's unit read backwards: 128 rows x up to 112
// columns of one group, whose tiles are contiguous in the blocked input. Lanes
// load 16-byte tile rows (the column word of rows i, i+32, i+64, i+96), scatter
// the four words into a row-major LDS strip (odd dword pitch), and after one
// barrier write the row segments out with 16-byte, 4-byte or 1-byte stores,
// whichever the segment's alignment allows. Spare units of the same launch
// write the zeros.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "group_table.h"
#include "mx_rearrange.h"

namespace {

constexpr int kUThreads = 256;
constexpr int kUMaxCols = 112;                     // columns per unit: 28 tiles, multiple of 16
constexpr int kUMaxTiles = kUMaxCols / 4;
constexpr int kUPitch = kUMaxTiles + 1;            // LDS dwords per row (odd)
constexpr int kULoads = (kUMaxTiles * 32 + kUThreads - 1) / kUThreads;
constexpr int kUMaxGroups = 4096;
constexpr int64_t kUMaxRowStride = int64_t(1) << 30;

struct UParams {
  const uint8_t *blocked;
  const int32_t *offs;
  uint8_t *out;
  int64_t ld;            // row stride of the row-major output
  int64_t units;
  int rows;
  int cols;
  int groups;
  int padded_cols;       // M: round_up(cols, 4)
  int unit_cols;         // columns per unit (multiple of 4)
  int per_row;           // M: units per output row block; K: units per 128-row block
};

// K groups: clamped cumulative ends e (scale columns), cumulative chunk counts
// cch (chunks of unit_cols padded columns) and cumulative padded widths cw.
__device__ __forceinline__ void scan_slice_k(const int32_t *__restrict__ offs, int groups, int cols, int unit_cols,
                                             int base, int carry_e, int carry_ch, int carry_w, int &e, int &cch,
                                             int &cw) {
  const int g = base + int(threadIdx.x & (kWave - 1));
  e = g < groups ? offs[g] : 0;
  e = min(max(e, 0), cols);
  e = max(wave_inclusive_max(e), carry_e);
  const int prev = wave_shift_up(e, carry_e);
  const int W = g < groups ? (e - prev + 3) & ~3 : 0;
  cch = wave_inclusive_sum((W + unit_cols - 1) / unit_cols) + carry_ch;
  cw = wave_inclusive_sum(W) + carry_w;
}

template <bool SMALL>
struct KGroups;

template <>
struct KGroups<true> {
  int groups, e, cch, cw;
  __device__ __forceinline__ void init(const UParams &p, int *) {
    groups = p.groups;
    scan_slice_k(p.offs, p.groups, p.cols, p.unit_cols, 0, 0, 0, 0, e, cch, cw);
  }
  __device__ __forceinline__ int count_cch_le(int64_t key) const {
    return __popcll(__ballot(int(threadIdx.x & (kWave - 1)) < groups && int64_t(cch) <= key));
  }
  __device__ __forceinline__ int end(int g) const { return __builtin_amdgcn_readlane(e, g); }
  __device__ __forceinline__ int chunks_through(int g) const { return __builtin_amdgcn_readlane(cch, g); }
  __device__ __forceinline__ int width_through(int g) const { return __builtin_amdgcn_readlane(cw, g); }
};

template <>
struct KGroups<false> {
  int groups;
  const int *es, *cchs, *cws;
  __device__ __forceinline__ void init(const UParams &p, int *lds) {
    groups = p.groups;
    int *e_out = lds, *ch_out = lds + p.groups, *w_out = lds + 2 * p.groups;
    if (threadIdx.x < kWave) {
      int ce = 0, cc = 0, cwd = 0;
      for (int base = 0; base < p.groups; base += kWave) {
        int e, cch, cw;
        scan_slice_k(p.offs, p.groups, p.cols, p.unit_cols, base, ce, cc, cwd, e, cch, cw);
        const int g = base + int(threadIdx.x);
        if (g < p.groups) {
          e_out[g] = e;
          ch_out[g] = cch;
          w_out[g] = cw;
        }
        ce = __builtin_amdgcn_readlane(e, kWave - 1);
        cc = __builtin_amdgcn_readlane(cch, kWave - 1);
        cwd = __builtin_amdgcn_readlane(cw, kWave - 1);
      }
    }
    __syncthreads();
    es = e_out;
    cchs = ch_out;
    cws = w_out;
  }
  __device__ __forceinline__ int count_cch_le(int64_t key) const {
    const int lane = threadIdx.x & (kWave - 1);
    int n = 0;
    for (int base = 0; base < groups; base += kWave) {
      const int c = __popcll(__ballot(base + lane < groups && int64_t(cchs[base + lane]) <= key));
      n += c;
      if (c < kWave) break;
    }
    return n;
  }
  __device__ __forceinline__ int end(int g) const { return es[g]; }
  __device__ __forceinline__ int chunks_through(int g) const { return cchs[g]; }
  __device__ __forceinline__ int width_through(int g) const { return cws[g]; }
};

// Reads tile_cols contiguous tiles at src (tile_cols*512 bytes, 16-byte
// aligned) and writes rows [0, nrows) x columns [0, ncols) of them to dst
// (row r at dst + r*ld). Called by the whole workgroup.
__device__ __forceinline__ void unit_out(uint32_t *lds, const uint8_t *src, int tile_cols, int nrows, int ncols,
                                         uint8_t *dst, int64_t ld) {
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(src, uint32_t(tile_cols) * 512u);
  uint4 v[kULoads];
#pragma unroll
  for (int it = 0; it < kULoads; ++it) {
    const int s = int(threadIdx.x) + it * kUThreads;
    const uint32_t off = s < tile_cols * 32 ? uint32_t(16 * s) : kOutOfRange;
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(off), 0, 2);
    v[it] = make_uint4(t[0], t[1], t[2], t[3]);
  }
  // piece s = 32*tile + i holds the words of rows i, i+32, i+64, i+96 in column word `tile`
#pragma unroll
  for (int it = 0; it < kULoads; ++it) {
    const int s = int(threadIdx.x) + it * kUThreads;
    const int tc = s < tile_cols * 32 ? s >> 5 : kUMaxTiles;   // column kUMaxTiles is spare
    const int i = s & 31;
    lds[(i + 0) * kUPitch + tc] = v[it].x;
    lds[(i + 32) * kUPitch + tc] = v[it].y;
    lds[(i + 64) * kUPitch + tc] = v[it].z;
    lds[(i + 96) * kUPitch + tc] = v[it].w;
  }
  __syncthreads();
  const uintptr_t a = reinterpret_cast<uintptr_t>(dst);
  if (((a | uint64_t(ld)) & 15) == 0) {
    // 16-byte aligned rows: one 16-byte piece per thread, a tail piece in dwords and bytes
    const int pieces = (ncols + 15) >> 4;
    for (int s = threadIdx.x; s < nrows * pieces; s += kUThreads) {
      const int r = s / pieces, k = s - r * pieces;
      const uint32_t *w = lds + r * kUPitch + 4 * k;
      uint8_t *d = dst + r * ld + 16 * k;
      const int n = min(16, ncols - 16 * k);
      if (n == 16) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4 *>(d));
      } else {
        for (int b = 0; b < n; ++b) d[b] = uint8_t(w[b >> 2] >> (8 * (b & 3)));
      }
    }
  } else if (((a | uint64_t(ld)) & 3) == 0) {
    const int words = (ncols + 3) >> 2;
    for (int s = threadIdx.x; s < nrows * words; s += kUThreads) {
      const int r = s / words, k = s - r * words;
      const uint32_t w = lds[r * kUPitch + k];
      uint8_t *d = dst + r * ld + 4 * k;
      const int n = min(4, ncols - 4 * k);
      if (n == 4)
        *reinterpret_cast<uint32_t *>(d) = w;
      else
        for (int b = 0; b < n; ++b) d[b] = uint8_t(w >> (8 * b));
    }
  } else {
    for (int s = threadIdx.x; s < nrows * ncols; s += kUThreads) {
      const int r = s / ncols, c = s - r * ncols;
      dst[r * ld + c] = uint8_t(lds[r * kUPitch + (c >> 2)] >> (8 * (c & 3)));
    }
  }
}

// Zero bytes of rows [r0, r1) x columns [c0, c1) of the output, share `part` of `parts`.
__device__ __forceinline__ void zero_region(uint8_t *out, int64_t ld, int64_t r0, int64_t r1, int64_t c0, int64_t c1,
                                            int64_t part, int64_t parts) {
  const int64_t w = c1 - c0;
  const int64_t total = (r1 - r0) * w;
  if (total <= 0 || parts <= 0) return;
  const int64_t per = (total + parts - 1) / parts;
  const int64_t b = min(per * part, total), e = min(per * (part + 1), total);
  for (int64_t s = b + threadIdx.x; s < e; s += kUThreads) {
    const int64_t r = s / w;
    out[(r0 + r) * ld + c0 + (s - r * w)] = 0;
  }
}

template <bool KGROUPS, bool SMALL>
__global__ __launch_bounds__(kUThreads) void unrearrange_kernel(UParams p) {
  extern __shared__ __align__(16) int ulds[];
  uint32_t *strip = reinterpret_cast<uint32_t *>(ulds);
  int *group_lds = ulds + kTileRows * kUPitch;
  const int64_t n8 = int64_t(gridDim.x) / 8 * 8;
  const int64_t u = int64_t(blockIdx.x) < n8 ? (int64_t(blockIdx.x) & 7) * (n8 >> 3) + (int64_t(blockIdx.x) >> 3)
                                             : int64_t(blockIdx.x);
  if (!KGROUPS) {
    MGroups<SMALL> grp;
    grp.init(p.offs, p.groups, p.rows, group_lds);
    if (u >= p.units) return;
    const int64_t ob = u / p.per_row;                  // output row block of the blocked layout
    const int cc = int(u - ob * p.per_row);
    const int g = grp.count_pends_le(ob * kTileRows);
    if (g < p.groups) {
      const int start = g ? grp.end(g - 1) : 0;
      const int pstart = g ? grp.pend_at(g - 1) : 0;
      const int64_t k = ob - pstart / kTileRows;
      const int row0 = start + int(k) * kTileRows;
      const int nrows = int(min(int64_t(kTileRows), int64_t(grp.end(g) - start) - k * kTileRows));
      const int c0 = cc * p.unit_cols;
      const int ncols = min(p.unit_cols, p.cols - c0);
      if (nrows <= 0 || ncols <= 0) return;
      const uint8_t *src = p.blocked + ob * kTileRows * int64_t(p.padded_cols) + int64_t(c0) * kTileRows;
      unit_out(strip, src, (ncols + 3) >> 2, nrows, ncols, p.out + int64_t(row0) * p.ld + c0, p.ld);
    } else {
      // spare units: zero the rows after the last group
      const int64_t first_spare = grp.pend_at(p.groups - 1) / kTileRows;
      const int64_t parts = p.units - first_spare * p.per_row;
      zero_region(p.out, p.ld, grp.end(p.groups - 1), p.rows, 0, p.cols, u - first_spare * p.per_row, parts);
    }
  } else {
    KGroups<SMALL> grp;
    grp.init(p, group_lds);
    if (u >= p.units) return;
    const int64_t rb = u / p.per_row;                  // 128-row block
    const int slot = int(u - rb * p.per_row);
    const int total_chunks = grp.chunks_through(p.groups - 1);
    const int nrows = min(kTileRows, p.rows - int(rb) * kTileRows);
    const int64_t padded_rows = int64_t((p.rows + kTileRows - 1) / kTileRows) * kTileRows;
    if (slot < total_chunks) {
      const int g = grp.count_cch_le(slot);
      const int first = g ? grp.chunks_through(g - 1) : 0;
      const int k = slot - first;
      const int start = g ? grp.end(g - 1) : 0;
      const int w = grp.end(g) - start;
      const int W = (w + 3) & ~3;
      const int C = g ? grp.width_through(g - 1) : 0;
      const int c0 = k * p.unit_cols;
      const int ncols = min(p.unit_cols, w - c0);       // real columns (the chunk may hold only padding)
      if (nrows <= 0 || ncols <= 0) return;
      const uint8_t *src = p.blocked + padded_rows * C + rb * kTileRows * int64_t(W) + int64_t(c0) * kTileRows;
      unit_out(strip, src, (ncols + 3) >> 2, nrows, ncols, p.out + rb * kTileRows * p.ld + start + c0, p.ld);
    } else {
      // spare slots of this row block: zero its rows' columns after the last group
      zero_region(p.out, p.ld, rb * kTileRows, rb * kTileRows + nrows, grp.end(p.groups - 1), p.cols,
                  slot - total_chunks, p.per_row - total_chunks);
    }
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int launch_unrearrange(bool kgroups, const uint8_t *blocked, int64_t rows, int64_t cols, const int32_t *offs,
                       int32_t groups, uint8_t *out, int64_t ld, hipStream_t stream) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (rows < 0 || cols < 0 || ld < cols || ld > kUMaxRowStride) return MX_REARRANGE_ESHAPE;
  if (groups < 1 || groups > kUMaxGroups) return MX_REARRANGE_EGROUPS;
  if (rows > lim - 128 * int64_t(groups) || cols > lim - 4 * int64_t(groups)) return MX_REARRANGE_ESHAPE;
  if (offs == nullptr) return MX_REARRANGE_ENULL;
  if (rows * cols == 0) return MX_REARRANGE_OK;   // nothing to write
  if (blocked == nullptr || out == nullptr) return MX_REARRANGE_ENULL;
  if (reinterpret_cast<uintptr_t>(blocked) & 15) return MX_REARRANGE_EALIGN;

  UParams p = {};
  p.blocked = blocked;
  p.offs = offs;
  p.out = out;
  p.ld = ld;
  p.rows = int(rows);
  p.cols = int(cols);
  p.groups = groups;
  p.padded_cols = int(round_up(cols, 4));
  p.unit_cols = kUMaxCols;
  if (!kgroups) {
    p.per_row = (p.padded_cols + p.unit_cols - 1) / p.unit_cols;
    p.units = ((rows + kTileRows - 1) / kTileRows + groups) * p.per_row;
  } else {
    p.per_row = int((cols + 4 * int64_t(groups) + p.unit_cols - 1) / p.unit_cols + groups);
    p.units = ((rows + kTileRows - 1) / kTileRows) * p.per_row;
  }
  if (p.units > lim) return MX_REARRANGE_ESHAPE;
  const bool small = groups <= kWave;
  const size_t lds = size_t(kTileRows) * kUPitch * 4 + (small ? 0 : size_t(kgroups ? 3 : 2) * groups * sizeof(int));
  const void *fn = kgroups ? (small ? reinterpret_cast<const void *>(&unrearrange_kernel<true, true>)
                                    : reinterpret_cast<const void *>(&unrearrange_kernel<true, false>))
                           : (small ? reinterpret_cast<const void *>(&unrearrange_kernel<false, true>)
                                    : reinterpret_cast<const void *>(&unrearrange_kernel<false, false>));
  void *args[] = {&p};
  const hipError_t e = hipLaunchKernel(fn, dim3(unsigned(p.units)), dim3(kUThreads), args, lds, stream);
  return e == hipSuccess ? MX_REARRANGE_OK : MX_REARRANGE_ELAUNCH;
}

}  // namespace

extern "C" {

int mx_block_unrearrange_M_groups(const uint8_t *blocked, int64_t rows, int64_t cols,
                                  const int32_t *group_end_offsets, int32_t num_groups, uint8_t *scales,
                                  int64_t row_stride, hipStream_t stream) {
  return launch_unrearrange(false, blocked, rows, cols, group_end_offsets, num_groups, scales, row_stride, stream);
}

int mx_block_unrearrange_K_groups(const uint8_t *blocked, int64_t rows, int64_t cols,
                                  const int32_t *group_end_offsets, int32_t num_groups, uint8_t *scales,
                                  int64_t row_stride, hipStream_t stream) {
  return launch_unrearrange(true, blocked, rows, cols, group_end_offsets, num_groups, scales, row_stride, stream);
}

}  // extern "C"
