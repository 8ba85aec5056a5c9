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
// M groups: a unit is 128 rows of one group within one 128-column window of
// the output row (one 128-byte line of each row when the rows are so aligned);
// its tiles are contiguous in the blocked input. K groups: a unit is 128 rows
// x one 256-column window of the output (128 columns above 64 groups, whose
// table takes LDS), holding the tiles of every group that
// has columns in the window (read one group after another), so no two units
// write the same output line. Lanes load 16-byte tile rows (the column word of
// rows i, i+32, i+64, i+96) and place the four words in a row-major LDS strip
// (odd dword pitch) — as words, or byte by byte where a K group's columns are
// not word-aligned in the window — and after one barrier write the row
// segments out: 16-byte stores of words realigned with v_alignbyte for every
// aligned 16-byte chunk inside a segment, at most three dwords and three bytes
// at either end. When an M unit's output rows are contiguous (row stride ==
// width, whole words) the strip is packed and the unit's rows are stored as one
// segment. Rows (M) past the last group are zeroed by spare units of the same
// launch; K windows zero their own columns past the last group.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "group_table.h"
#include "launch_order.h"
#include "mx_rearrange.h"
#include "write_ranges.h"

namespace {

// Unit geometry (threads, output columns). M units: 128 columns (one
// 128-byte line of each row), 128 threads. K windows with at most 64 groups:
// 256 columns (two lines of each row), 512 threads, measured faster on the
// large K shapes (256-column M units were slower on the skinny M shape). K
// windows of more than 64 groups, whose table takes LDS: 128 columns, 256
// threads.
template <int THREADS, int COLS>
struct UGeom {
  static constexpr int threads = THREADS;
  static constexpr int cols = COLS;
  static constexpr int max_tiles = cols / 4 + 1;   // a K window may start up to 3 columns into a tile
  static constexpr int pitch = max_tiles + 2;      // LDS dwords per strip row (odd)
  static constexpr int loads = (max_tiles * 32 + threads - 1) / threads;
};
using GM = UGeom<128, 128>;
using GKWide = UGeom<512, 256>;
using GKNarrow = UGeom<256, 128>;
template <bool KGROUPS, bool SMALL>
using UnitGeom = typename std::conditional<KGROUPS, typename std::conditional<SMALL, GKWide, GKNarrow>::type, GM>::type;
constexpr int kUMaxGroups = 4096;
constexpr int kUKDealWindows = 11;   // K windows per run of the interleaved XCD order
constexpr int64_t kUMaxRowStride = int64_t(1) << 30;
static_assert(kTileRows * GKWide::pitch * 4 <= 64 * 1024 &&
                  kTileRows * GKNarrow::pitch * 4 + 2 * kUMaxGroups * 4 <= 64 * 1024 &&
                  kTileRows * GM::pitch * 4 + 2 * kUMaxGroups * 4 <= 64 * 1024,
              "LDS per workgroup: the strip, and the group table of more than 64 groups");

struct UParams {
  const uint8_t *blocked;
  const int32_t *offs;
  uint8_t *out;
  int64_t ld;            // row stride of the row-major output
  int64_t units;
  int64_t blocked_bytes; // size of the blocked input (the forward output allocation)
  int rows;
  int cols;
  int groups;
  int padded_cols;       // M: round_up(cols, 4)
  int per_row;           // M: units per output row block; K: units per 128-row block
  int64_t deal;          // interleaved order: consecutive units dealt to one XCD at a time
};

// K groups: clamped cumulative ends e (scale columns) and cumulative padded
// widths cw.
__device__ __forceinline__ void scan_slice_k(const int32_t *__restrict__ offs, int groups, int cols, int base,
                                             int carry_e, int carry_w, int &e, int &cw) {
  const int g = base + int(threadIdx.x & (kWave - 1));
  e = g < groups ? offs[g] : 0;
  e = min(max(e, 0), cols);
  e = max(wave_inclusive_max(e), carry_e);
  const int prev = wave_shift_up(e, carry_e);
  const int W = g < groups ? (e - prev + 3) & ~3 : 0;
  cw = wave_inclusive_sum(W) + carry_w;
}

template <bool SMALL>
struct KGroups;

template <>
struct KGroups<true> {
  int groups, e, cw;
  __device__ __forceinline__ void init(const UParams &p, int *) {
    groups = p.groups;
    scan_slice_k(p.offs, p.groups, p.cols, 0, 0, 0, e, cw);
  }
  __device__ __forceinline__ int count_ends_le(int64_t key) const {
    return __popcll(__ballot(int(threadIdx.x & (kWave - 1)) < groups && int64_t(e) <= key));
  }
  __device__ __forceinline__ int end(int g) const { return __builtin_amdgcn_readlane(e, g); }
  __device__ __forceinline__ int width_through(int g) const { return __builtin_amdgcn_readlane(cw, g); }
};

template <>
struct KGroups<false> {
  int groups;
  const int *es, *cws;
  __device__ __forceinline__ void init(const UParams &p, int *lds) {
    groups = p.groups;
    int *e_out = lds, *w_out = lds + p.groups;
    if (threadIdx.x < kWave) {
      int ce = 0, cwd = 0;
      for (int base = 0; base < p.groups; base += kWave) {
        int e, cw;
        scan_slice_k(p.offs, p.groups, p.cols, base, ce, cwd, e, cw);
        const int g = base + int(threadIdx.x);
        if (g < p.groups) {
          e_out[g] = e;
          w_out[g] = cw;
        }
        ce = __builtin_amdgcn_readlane(e, kWave - 1);
        cwd = __builtin_amdgcn_readlane(cw, kWave - 1);
      }
    }
    __syncthreads();
    es = e_out;
    cws = w_out;
  }
  __device__ __forceinline__ int count_ends_le(int64_t key) const {
    const int lane = threadIdx.x & (kWave - 1);
    int n = 0;
    for (int base = 0; base < groups; base += kWave) {
      const int c = __popcll(__ballot(base + lane < groups && int64_t(es[base + lane]) <= key));
      n += c;
      if (c < kWave) break;
    }
    return n;
  }
  __device__ __forceinline__ int end(int g) const { return es[g]; }
  __device__ __forceinline__ int width_through(int g) const { return cws[g]; }
};

// End offset of group `lane` for the first 64 groups (0 past the last one),
// loaded through a buffer resource: the range check, not a branch, keeps the
// load unconditional, so it can be issued ahead of the tile loads and waited
// for alone.
__device__ __forceinline__ int first_ends(const int32_t *offs, int groups) {
  const __amdgpu_buffer_rsrc_t r = byte_buffer(offs, 4 * uint32_t(min(groups, kWave)));
  return __builtin_amdgcn_raw_buffer_load_b32(r, 4 * int(threadIdx.x & (kWave - 1)), 0, 0);
}

// The M-groups table of at most 64 groups from end offsets already loaded
// (raw: lane g's end offset): clamped non-decreasing ends and padded
// cumulative ends, as MGroups<true>::init forms them.
__device__ __forceinline__ void init_loaded(MGroups<true> &grp, int raw, int groups, int rows) {
  const int g = int(threadIdx.x & (kWave - 1));
  grp.groups = groups;
  int e = g < groups ? min(max(raw, 0), rows) : 0;
  e = wave_inclusive_max(e);
  const int prev = wave_shift_up(e, 0);
  const int padded = g < groups ? (e - prev + kTileRows - 1) / kTileRows * kTileRows : 0;
  grp.e = e;
  grp.pend = wave_inclusive_sum(padded);
}

// A row segment of ncols bytes at p split by alignment: head_bytes single bytes,
// head_dwords 4-byte aligned dwords, `chunks` 16-byte aligned chunks from
// chunk0, tail_dwords dwords, then single bytes from tail_bytes0 to ncols.
struct RowSplit {
  int head_bytes, head_dwords, chunk0, chunks, tail_dwords, tail_bytes0;
  __device__ __forceinline__ RowSplit(const uint8_t *p, int ncols) {
    const int m = int(reinterpret_cast<uintptr_t>(p) & 15);
    head_bytes = min((4 - (m & 3)) & 3, ncols);
    const int dwords = (ncols - head_bytes) >> 2;       // whole aligned dwords of the segment
    chunk0 = (16 - m) & 15;                             // first 16-byte aligned byte (>= head_bytes)
    head_dwords = min((chunk0 - head_bytes) >> 2, dwords);
    chunks = (dwords - head_dwords) >> 2;
    tail_dwords = dwords - head_dwords - 4 * chunks;
    tail_bytes0 = head_bytes + 4 * dwords;
    if (chunks == 0) chunk0 = head_bytes + 4 * head_dwords;   // tail dwords follow the head ones
  }
};

// Issues the loads of tile_cols contiguous tiles at src (16-byte aligned); at
// most `bytes` of them are read, pieces past that load as zeros.
template <class G>
__device__ __forceinline__ void issue_loads(uint4 (&v)[G::loads], const uint8_t *src, int tile_cols, uint32_t bytes) {
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(src, bytes);
#pragma unroll
  for (int it = 0; it < G::loads; ++it) {
    const int s = int(threadIdx.x) + it * G::threads;
    const uint32_t off = s < tile_cols * 32 ? uint32_t(16 * s) : kOutOfRange;
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(off), 0, 2);
    v[it] = make_uint4(t[0], t[1], t[2], t[3]);
  }
}

// Scatters the loaded tiles into the LDS strip, row r's column word c at
// lds[r*pitch + c]. Called by the whole workgroup; ends with a barrier.
__device__ __forceinline__ void scatter_strip(uint32_t *lds, int pitch, const uint4 (&v)[GM::loads], int tile_cols) {
  // piece s = 32*tile + i holds the words of rows i, i+32, i+64, i+96 in column word `tile`
#pragma unroll
  for (int it = 0; it < GM::loads; ++it) {
    const int s = int(threadIdx.x) + it * GM::threads;
    if (s < tile_cols * 32) {
      const int tc = s >> 5, i = s & 31;
      lds[(i + 0) * pitch + tc] = v[it].x;
      lds[(i + 32) * pitch + tc] = v[it].y;
      lds[(i + 64) * pitch + tc] = v[it].z;
      lds[(i + 96) * pitch + tc] = v[it].w;
    }
  }
  __syncthreads();
}

// K windows: places ntiles loaded tiles of one group in the window's LDS strip
// (row r at lds + r*G::pitch words). The first byte of tile tc's words belongs
// at window column col0 + 4*tc; only bytes at window columns [lo, hi), the
// group's part of the window, are written. Word-aligned tiles inside the range
// are written as words, the others byte by byte. Groups place disjoint column
// ranges, so no barrier is needed between them.
template <class G>
__device__ __forceinline__ void scatter_window(uint32_t *lds, const uint4 (&v)[G::loads], int ntiles, int col0,
                                               int lo, int hi) {
  uint8_t *lb = reinterpret_cast<uint8_t *>(lds);
#pragma unroll
  for (int it = 0; it < G::loads; ++it) {
    const int s = int(threadIdx.x) + it * G::threads;
    if (s < ntiles * 32) {
      const int i = s & 31;
      const int col = col0 + 4 * (s >> 5);
      const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
      if ((col & 3) == 0 && col >= lo && col + 4 <= hi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) lds[(i + 32 * q) * G::pitch + (col >> 2)] = w[q];
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int c = col + b;
          if (c >= lo && c < hi) {
#pragma unroll
            for (int q = 0; q < 4; ++q) lb[(i + 32 * q) * G::pitch * 4 + c] = uint8_t(w[q] >> (8 * b));
          }
        }
      }
    }
  }
}

// Writes rows [0, nrows) x bytes [skip, skip + ncols) of the LDS strip (row r
// from lds + r*pitch words) to dst, row r at dst + r*ld (ld unused when nrows
// is 1). Called by the whole workgroup. NT: the 16-byte chunk stores are
// non-temporal (measured faster for M units, slower for K units).
template <bool NT, int THREADS>
__device__ __forceinline__ void store_rows(const uint32_t *lds, int pitch, int skip, int nrows, int ncols,
                                           uint8_t *dst, int64_t ld) {
  // Store. Split each row segment by its alignment: up to 3 single bytes, up
  // to 3 dwords, whole 16-byte chunks, up to 3 dwords, up to 3 bytes. Three
  // passes (chunks, end dwords, end bytes) keep every store instruction's lanes
  // busy; a pass that the alignment rules out is skipped. Addresses stay derived
  // from dst, so the stores are global (flat ones would also count against the
  // LDS reads' wait counter).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uintptr_t dst_bits = reinterpret_cast<uintptr_t>(dst) | uintptr_t(nrows > 1 ? ld : 0);
  const int max_chunks = ncols >> 4;
  for (int s = threadIdx.x; s < nrows * max_chunks; s += THREADS) {
    const int r = s / max_chunks, q = s - r * max_chunks;
    uint8_t *row_ptr = dst + int64_t(r) * ld;
    const RowSplit sp(row_ptr, ncols);
    if (q >= sp.chunks) continue;
    const int lo = sp.chunk0 + 16 * q;
    const uint32_t *w = lds + r * pitch + ((skip + lo) >> 2);
    const int sh = (skip + lo) & 3;
    u32x4 v;
    if (sh) {
      const uint32_t x0 = w[0], x1 = w[1], x2 = w[2], x3 = w[3], x4 = w[4];   // w[4] still below lo + 16
      v = u32x4{__builtin_amdgcn_alignbyte(x1, x0, sh), __builtin_amdgcn_alignbyte(x2, x1, sh),
                __builtin_amdgcn_alignbyte(x3, x2, sh), __builtin_amdgcn_alignbyte(x4, x3, sh)};
    } else {
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
    if (NT)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(row_ptr + lo));
    else
      *reinterpret_cast<u32x4 *>(row_ptr + lo) = v;
  }
  if ((dst_bits & 15) != 0 || (ncols & 15) != 0) {
    for (int s = threadIdx.x; s < nrows * 6; s += THREADS) {
      const int r = s / 6, k = s - r * 6;
      uint8_t *row_ptr = dst + int64_t(r) * ld;
      const RowSplit sp(row_ptr, ncols);
      const int d0 = k < 3 ? (k < sp.head_dwords ? sp.head_bytes + 4 * k : -1)
                           : (k - 3 < sp.tail_dwords ? sp.chunk0 + 16 * sp.chunks + 4 * (k - 3) : -1);
      if (d0 < 0) continue;
      const uint32_t *w = lds + r * pitch + ((skip + d0) >> 2);
      const int sh = (skip + d0) & 3;
      *reinterpret_cast<uint32_t *>(row_ptr + d0) = sh ? __builtin_amdgcn_alignbyte(w[1], w[0], sh) : w[0];
    }
  }
  if ((dst_bits & 3) != 0 || (ncols & 3) != 0) {
    for (int s = threadIdx.x; s < nrows * 6; s += THREADS) {
      const int r = s / 6, k = s - r * 6;
      uint8_t *row_ptr = dst + int64_t(r) * ld;
      const RowSplit sp(row_ptr, ncols);
      const int j = k < 3 ? (k < sp.head_bytes ? k : -1) : (sp.tail_bytes0 + (k - 3) < ncols ? sp.tail_bytes0 + k - 3 : -1);
      if (j < 0) continue;
      row_ptr[j] = uint8_t(lds[r * pitch + ((skip + j) >> 2)] >> (8 * ((skip + j) & 3)));
    }
  }
}

// One unit, its tiles loaded into v: rows [0, nrows) x columns [skip, skip +
// ncols) to dst, row r at dst + r*ld. When the rows are contiguous (ld ==
// ncols) and whole words, the strip is packed with pitch ncols/4 and the unit's
// output is stored as one segment of nrows*ncols bytes.
template <bool NT>
__device__ __forceinline__ void unit_out(uint32_t *lds, const uint4 (&v)[GM::loads], int skip, int tile_cols, int nrows,
                                         int ncols, uint8_t *dst, int64_t ld) {
  if (skip == 0 && ld == ncols && (ncols & 3) == 0) {
    scatter_strip(lds, ncols >> 2, v, tile_cols);
    store_rows<NT, GM::threads>(lds, 0, 0, 1, nrows * ncols, dst, 0);
  } else {
    scatter_strip(lds, GM::pitch, v, tile_cols);
    store_rows<NT, GM::threads>(lds, GM::pitch, skip, nrows, ncols, dst, ld);
  }
}

// Zero bytes of rows [r0, r1) x columns [c0, c1) of the output, share `part` of `parts`.
__device__ __forceinline__ void zero_region(uint8_t *out, int64_t ld, int64_t r0, int64_t r1, int64_t c0, int64_t c1,
                                            int64_t part, int64_t parts) {
  const int64_t w = c1 - c0;
  const int64_t total = (r1 - r0) * w;
  if (total <= 0 || parts <= 0 || part < 0) return;
  const int64_t per = (total + parts - 1) / parts;
  const int64_t b = min(per * part, total), e = min(per * (part + 1), total);
  for (int64_t s = b + threadIdx.x; s < e; s += GM::threads) {
    const int64_t r = s / w;
    out[(r0 + r) * ld + c0 + (s - r * w)] = 0;
  }
}

template <bool KGROUPS, bool SMALL, bool IL>
__global__ __launch_bounds__((UnitGeom<KGROUPS, SMALL>::threads)) void unrearrange_kernel(UParams p) {
  using GK = typename std::conditional<SMALL, GKWide, GKNarrow>::type;   // K window geometry
  extern __shared__ __align__(16) int ulds[];
  uint32_t *strip = reinterpret_cast<uint32_t *>(ulds);
  int *group_lds = ulds + kTileRows * UnitGeom<KGROUPS, SMALL>::pitch;
  // the order of units over the XCDs (launch_order.h); slots past the last
  // unit map to units >= p.units, which do nothing
  const int64_t u = unit_of_slot<IL>(blockIdx.x, gridDim.x, p.deal);
  if (!KGROUPS) {
    const int64_t ob = u / p.per_row;                  // output row block of the blocked layout
    const int cc = int(u - ob * p.per_row);
    const int c0 = cc * GM::cols;
    const int ncols = min(GM::cols, p.cols - c0);
    const int tile_cols = (ncols + 3) >> 2;
    // The unit's tiles sit at a place fixed by its row block and column
    // window, whatever the groups are: their loads go out first and the group
    // table is scanned while they are in flight. (Units that turn out to lie
    // past the last group load tiles of the zero tail they never use; nothing
    // past the blocked input is read.)
    const int64_t src_off = ob * kTileRows * int64_t(p.padded_cols) + int64_t(c0) * kTileRows;
    const int64_t avail = u < p.units ? clamp64(p.blocked_bytes - src_off, 0, int64_t(tile_cols) * 512) : 0;
    uint4 v[GM::loads];
    MGroups<SMALL> grp;
    if constexpr (SMALL) {
      // the end offsets go out before the tiles, so the scan waits for them alone
      const int raw = first_ends(p.offs, p.groups);
      issue_loads<GM>(v, p.blocked + (avail > 0 ? src_off : 0), tile_cols, uint32_t(avail));
      __builtin_amdgcn_sched_barrier(0);
      init_loaded(grp, raw, p.groups, p.rows);
    } else {
      // (more than 64 groups: the table is scanned into LDS first)
      grp.init(p.offs, p.groups, p.rows, group_lds);
      issue_loads<GM>(v, p.blocked + (avail > 0 ? src_off : 0), tile_cols, uint32_t(avail));
    }
    if (u >= p.units) return;
    const int g = grp.count_pends_le(ob * kTileRows);
    if (g < p.groups) {
      const int start = g ? grp.end(g - 1) : 0;
      const int pstart = g ? grp.pend_at(g - 1) : 0;
      const int64_t k = ob - pstart / kTileRows;
      const int64_t row0 = start + k * kTileRows;
      const int nrows = int(min(int64_t(kTileRows), int64_t(grp.end(g) - start) - k * kTileRows));
      // (a correct table always passes the second test: the rows lie inside the output)
      if (nrows <= 0 || ncols <= 0 || !fits(row0, nrows, p.rows)) return;
      unit_out<true>(strip, v, 0, tile_cols, nrows, ncols, p.out + int64_t(row0) * p.ld + c0, p.ld);
    } else {
      // spare units: zero the rows after the last group
      const int64_t first_spare = grp.pend_at(p.groups - 1) / kTileRows;
      const int64_t parts = p.units - first_spare * p.per_row;
      zero_region(p.out, p.ld, clamp64(grp.end(p.groups - 1), 0, p.rows), p.rows, 0, p.cols,
                  u - first_spare * p.per_row, parts);
    }
  } else {
    KGroups<SMALL> grp;
    grp.init(p, group_lds);
    if (u >= p.units) return;
    const int64_t rb = u / p.per_row;                  // 128-row block
    const int c_lo = int(u - rb * p.per_row) * GK::cols; // output window [c_lo, c_hi)
    const int c_hi = min(c_lo + GK::cols, p.cols);
    const int nrows = min(kTileRows, p.rows - int(rb) * kTileRows);
    const int64_t padded_rows = int64_t((p.rows + kTileRows - 1) / kTileRows) * kTileRows;
    // the groups cover [0, last end) without gaps: a window reaching past it starts from zeros
    if (c_hi > grp.end(p.groups - 1)) {
      for (int d = threadIdx.x; d < kTileRows * GK::pitch; d += GK::threads) strip[d] = 0u;
      __syncthreads();
    }
    // every group with columns in the window, from the first whose end lies past c_lo
    for (int g = grp.count_ends_le(c_lo); g < p.groups; ++g) {
      const int start = g ? grp.end(g - 1) : 0;
      if (start >= c_hi) break;
      const int end = grp.end(g);
      if (end <= start) continue;
      const int lo = max(c_lo, start), hi = min(c_hi, end);   // the group's columns in the window
      const int t0 = (lo - start) >> 2;                        // its first tile there
      const int ntiles = ((hi - 1 - start) >> 2) - t0 + 1;
      const int W = (end - start + 3) & ~3;
      const int C = g ? grp.width_through(g - 1) : 0;
      const int64_t src_off = padded_rows * C + rb * kTileRows * int64_t(W) + int64_t(t0) * 512;
      // (a correct table always passes: the tiles read lie inside the blocked input)
      if (ntiles <= 0 || !fits(src_off, int64_t(ntiles) * 512, p.blocked_bytes)) continue;
      uint4 v[GK::loads];
      issue_loads<GK>(v, p.blocked + src_off, ntiles, uint32_t(ntiles) * 512u);
      scatter_window<GK>(strip, v, ntiles, start + 4 * t0 - c_lo, lo - c_lo, hi - c_lo);
    }
    __syncthreads();
    // no other unit writes these lines: stream them when every row starts on a 128-byte line
    uint8_t *dst = p.out + rb * kTileRows * p.ld + c_lo;
    if (((reinterpret_cast<uintptr_t>(p.out) | uintptr_t(p.ld)) & 127) == 0)
      store_rows<true, GK::threads>(strip, GK::pitch, 0, nrows, c_hi - c_lo, dst, p.ld);
    else
      store_rows<false, GK::threads>(strip, GK::pitch, 0, nrows, c_hi - c_lo, dst, p.ld);
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

template <bool KGROUPS, bool SMALL>
const void *kernel_of(bool il) {
  return il ? reinterpret_cast<const void *>(&unrearrange_kernel<KGROUPS, SMALL, true>)
            : reinterpret_cast<const void *>(&unrearrange_kernel<KGROUPS, SMALL, false>);
}

const void *kernel_for(bool kgroups, bool small, bool il) {
  return kgroups ? (small ? kernel_of<true, true>(il) : kernel_of<true, false>(il))
                 : (small ? kernel_of<false, true>(il) : kernel_of<false, false>(il));
}

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
  const bool small = groups <= kWave;   // group table in registers, else in LDS
  const bool wide = kgroups && small;   // 256-column K windows
  const int unit_cols = wide ? GKWide::cols : kgroups ? GKNarrow::cols : GM::cols;
  if (!kgroups) {
    p.per_row = (p.padded_cols + unit_cols - 1) / unit_cols;
    p.units = ((rows + kTileRows - 1) / kTileRows + groups) * p.per_row;
  } else {
    // one unit per (128-row block, output window)
    p.per_row = int((cols + unit_cols - 1) / unit_cols);
    p.units = ((rows + kTileRows - 1) / kTileRows) * p.per_row;
  }
  const int pitch = wide ? GKWide::pitch : kgroups ? GKNarrow::pitch : GM::pitch;
  const int threads = wide ? GKWide::threads : kgroups ? GKNarrow::threads : GM::threads;
  // The interleaved order deals runs of consecutive units to the XCDs in
  // turn: whole row blocks, or for K windows runs of kUKDealWindows when a
  // row block holds at least twice that many (its windows share no output
  // line): (28672, 8192) K inverse 79.3-79.9 against 80.6-81.1 us; runs of 8
  // or 16 windows took 81.5-82.1 us.
  p.deal = kgroups && p.per_row >= 2 * kUKDealWindows ? kUKDealWindows : p.per_row;
  if (slots_for(true, p.units, p.deal) > max_grid(threads)) return MX_REARRANGE_ESHAPE;
  p.blocked_bytes = kgroups ? mx_rearrange_K_groups_out_bytes(rows, cols, groups)
                            : mx_rearrange_M_groups_out_bytes(rows, cols, groups);
  const size_t lds = size_t(kTileRows) * pitch * 4 + (small ? 0 : size_t(2) * groups * sizeof(int));
  // A grid of more than one pass over the GPU deals runs of units (p.deal) to
  // the XCDs in turn (launch_order.h): with whole row blocks, measured on
  // (28672, 8192) K groups 80.7 against 85.0 us. A grid of one pass keeps contiguous ranges (interleaved,
  // the (131072, 44) M inverse took 4.89 against 4.58 us).
  const bool il = [&] {
    const void *plain = kernel_for(kgroups, small, false);
    const int64_t resident = resident_workgroups(plain, threads, lds);
    return resident > 0 && p.units > resident;
  }();
  const void *fn = kernel_for(kgroups, small, il);
  const int64_t grid = slots_for(il, p.units, p.deal);
  void *args[] = {&p};
  const hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(threads), args, lds, stream);
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
