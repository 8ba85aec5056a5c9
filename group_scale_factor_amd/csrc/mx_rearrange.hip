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
// fallback); "[mxfp8 moe training] use dim1 cast cuda kernel for 3d weights by
// reshaping to 2d" (Benchmarks tables: per-expert weights (E, N, K), whose
// scales become one blocked matrix per expert).
//
// The work is pure data movement, bound by HBM bandwidth; there is no
// arithmetic on the scale values. Design:
//   * One workgroup handles one work unit. M groups and per-expert matrices:
//     128 rows x a column chunk of one group, i.e. a run of whole output tiles
//     that are contiguous in the output. K groups: 128 rows x a 256-column
//     window of the input (two 128-byte lines per row when rows are so
//     aligned; 512 columns where that makes the grid fit the workgroups the
//     GPU holds at once), writing the tiles of every group whose tiles start
//     in the window — one contiguous output run per such group. A K unit's input
//     thus does not depend on the offsets: its loads are issued before the
//     offsets are scanned, and the scan runs while they are in flight.
//   * Group lookup: every wave loads the end offsets, one group per lane,
//     clamps them into a non-decreasing sequence, and forms the padded sizes
//     and their prefix sums with DPP scans; a ballot over the cumulative unit
//     counts (M) or over the groups' column ranges (K) names the group(s) of
//     the unit. G > 64 is handled in 64-lane slices with a carry.
//   * Load: the unit's source bytes are fetched as 16-byte aligned pieces
//     (buffer_load_dwordx4) covering each row segment (or, for packed narrow
//     rows, the whole strip as one range, loaded straight into LDS) and staged
//     in LDS. A 16-byte aligned piece that contains at least one byte of the
//     matrix lies inside the same memory page as that byte, so the cover never
//     touches a page the matrix does not; the extra bytes are never emitted.
//   * Interleave: after one barrier each lane assembles one 16-byte output
//     unit — the same 4-byte column word of rows i, i+32, i+64, i+96 of the
//     tile — from LDS. When the source is not 4-byte aligned each word is
//     assembled from two aligned LDS words with v_alignbyte_b32. Bytes past
//     the group's rows or columns are masked to zero.
//   * Store: consecutive lanes write consecutive 16 bytes, non-temporal
//     (global_store_dwordx4 nt; buffer stores with sc1 as well for M and K
//     launches that move more bytes than the MALL holds).
//   * The whole output allocation is written exactly once by the same launch:
//     work units past the last group's data zero-fill the tail, so the output
//     needs no memset.
//   * Work units are spread over the 8 XCDs (workgroups are dealt to XCDs
//     round-robin) so that units sharing boundary cache lines run on the same
//     XCD, keeping those lines in one L2. Grids of more than one pass over
//     the chip deal runs of units to the XCDs in turn (four row blocks for M
//     and per-expert units; for K windows, 11 windows of a row block), so
//     that the chip as a whole reads neighbouring rows; one-pass grids give
//     each XCD a contiguous range of units.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "group_table.h"
#include "launch_order.h"
#include "mx_rearrange.h"
#include "write_ranges.h"

namespace {

// Widest column chunk of an M unit: 112 columns are covered by at most 8
// aligned 16-byte pieces per row at any alignment, so a 128-row unit is at most
// 1024 pieces, 4 per lane of a 256-thread workgroup. Narrow units keep
// registers and LDS small (7 workgroups per CU), which measured faster than
// wider ones.
constexpr int kMaxUnitCols = 112;
constexpr int kMinUnitCols = 32;              // narrowest chunk the host splits M row blocks into
// K groups: input windows of 256 columns (two 128-byte lines per row when rows
// are line aligned), or 512 where that grid would need a small second pass
// over the chip (see launch()). A group's tile starts 4*k columns after the
// group's first column and belongs to the window holding that start, so a
// window's tiles read up to 3 columns past it.
constexpr int kWinCols = 256;
constexpr int kWinColsWide = 512;
constexpr int kWinColsAny = 128;              // windows of rows that do not start on 128-byte lines
constexpr int kTailColsPerUnit = 128;         // K: tail units per row block = ceil(4G / this)
constexpr int kTargetUnits = 1024;            // M: split row blocks into chunks until this many units
constexpr int kFlatMaxCols = 60;              // M: widest packed row staged as one flat range
constexpr int kMaxPieces = (kMaxUnitCols + 30) / 16;   // 16-byte pieces covering one row segment
constexpr int kMaxPitch = 16 * kMaxPieces + 4;         // LDS row pitch: 4*pieces+1 words, odd
constexpr int kMaxFlatPieces = (kTileRows * kFlatMaxCols + 30) / 16;
constexpr int kLdsSlack = 16;                 // room for the second word of an unaligned read
constexpr int64_t kMaxGrid = int64_t(1) << 20;
constexpr int64_t kMaxRowStride = int64_t(1) << 24;   // keeps a unit's byte span inside 32-bit buffer offsets
// Cache policy of the staging loads (buffer instruction bit 1: non-temporal).
// M strips share at most one line with their neighbour, so they stream. A K
// window's own lines are read by no other unit when rows are 128-byte aligned
// and stream too; the piece past the window (and every piece of rows not so
// aligned, whose lines straddle windows) is shared and keeps the default
// policy, so the neighbour finds it in L2.
constexpr int kFlatLoadPolicy = 2;
constexpr int kMRowsLoadPolicy = 2;
constexpr int kWindowLoadPolicy = 2;
constexpr int kSharedLoadPolicy = 0;
constexpr int k3dLoadPolicy = 2;
// Output stores are non-temporal. An M- or K-groups launch that moves more
// bytes than the 256 MB MALL holds also sets sc1 on them (buffer instruction
// cache policy: bit 1 nt, bit 4 sc1), in kernels built for it: measured 9%
// faster on M groups of 336 MB, 0.5-2.5% on K shapes of 336 to 941 MB;
// within 1% at 168-235 MB and 4-11% slower on smaller launches.
constexpr int64_t kWriteThroughBytes = int64_t(256) << 20;
// Runs of the interleaved XCD order (dispatch()): K windows per run, M and
// per-expert row blocks per run.
constexpr int kKDealWindows = 11;
constexpr int kMDealBlocks = 4;
constexpr int kStoreNtSc1 = 2 | 16;

// Staging modes; each is its own kernel instantiation (two for the modes that
// also have the sc1-store variant, kernel_for()).
enum Mode : int {
  kModeMFlat = 0,   // M groups, packed rows of <= 60 bytes, one contiguous range per 128-row strip
  kModeMRows = 1,   // M groups, one row segment at a time
  kModeMRowsNarrow = 3,  // M groups, one row segment of at most kNarrowUnitCols at a time
  kModeKWindows = 2,  // K groups, column windows of rows that start 128-byte aligned
  kModeKWindowsWide = 7,  // the same with windows of kWinColsWide columns
  kModeKWindowsAny = 6,  // K groups, column windows of rows at any alignment
  kMode3d = 4,      // per-expert matrices, one row segment at a time, no group lookup
  kMode3dWide = 5,  // the same with twice the threads, for grids of several units per CU slot
};

constexpr bool is_3d(int mode) { return mode == kMode3d || mode == kMode3dWide; }
constexpr bool is_k(int mode) { return mode == kModeKWindows || mode == kModeKWindowsWide || mode == kModeKWindowsAny; }
constexpr bool is_line_window(int mode) { return mode == kModeKWindows || mode == kModeKWindowsWide; }
constexpr int win_cols_for(int mode) {
  return mode == kModeKWindows ? kWinCols : mode == kModeKWindowsWide ? kWinColsWide : kWinColsAny;
}
constexpr int win_span_for(int mode) { return win_cols_for(mode) + 3; }
// 16-byte pieces covering a window row (and the 3 columns past it) at any alignment
constexpr int win_pieces_for(int mode) { return (win_span_for(mode) + 30) / 16; }

// Narrow M units (small problems split into many column chunks) get their own
// instantiation sized for them: fewer loads per lane, fewer registers.
constexpr int kNarrowUnitCols = 48;
// Per-expert units span a whole 128-row block of up to 160 columns (the
// block-32 scales of K = 5120): one contiguous output run per row block.
constexpr int k3dMaxUnitCols = 160;
// Threads per workgroup, measured per mode: 128 for the small per-unit work of
// flat strips and narrow chunks, 256 elsewhere; K windows of line-aligned rows
// and per-expert grids of more than k3dWideUnits units run 512 threads (fewer
// loads per lane, more units in flight).
constexpr int threads_for(int mode) {
  return mode == kModeMFlat || mode == kModeMRowsNarrow       ? 128
         : mode == kMode3dWide || is_line_window(mode) ? 512
                                                        : 256;
}
constexpr int64_t k3dWideUnits = 2048;
constexpr int max_unit_cols_for(int mode) {
  return mode == kModeMRowsNarrow ? kNarrowUnitCols
         : is_3d(mode)            ? k3dMaxUnitCols
         : is_k(mode)             ? win_span_for(mode)
                                  : kMaxUnitCols;
}
constexpr int max_pieces_for(int mode) { return (max_unit_cols_for(mode) + 30) / 16; }
constexpr int load_policy_for(int mode) {
  return mode == kModeMFlat    ? kFlatLoadPolicy
         : is_k(mode)            ? kSharedLoadPolicy
         : is_3d(mode)           ? k3dLoadPolicy
                                 : kMRowsLoadPolicy;
}
constexpr int load_iters_for(int mode) {
  return ((mode == kModeMFlat ? kMaxFlatPieces : kTileRows * max_pieces_for(mode)) + threads_for(mode) - 1) /
         threads_for(mode);
}

// Register budget hint (waves per SIMD); 1 leaves it to the compiler, which
// needs about 72 VGPRs, i.e. 7 waves per SIMD.
constexpr int kMinWavesPerEu = 1;

static_assert(kMaxUnitCols % 4 == 0 && kMinUnitCols % 4 == 0, "units are whole tile columns");
static_assert(kTileRows * kMaxPitch + kLdsSlack <= 64 * 1024, "LDS per workgroup");
static_assert(kTileRows * (16 * max_pieces_for(kMode3d) + 4) + kLdsSlack <= 64 * 1024, "LDS per workgroup");
static_assert(load_iters_for(kModeKWindowsAny) <= 8 && load_iters_for(kModeMFlat) <= 8 &&
                  load_iters_for(kMode3d) <= 8 && load_iters_for(kModeMRowsNarrow) <= 8 &&
                  load_iters_for(kModeMRows) <= 8,
              "staging unrolled to 8");
static_assert(k3dMaxUnitCols % 4 == 0, "units are whole tile columns");
static_assert(kNarrowUnitCols % 4 == 0 && kNarrowUnitCols >= kMinUnitCols, "narrow units");
static_assert(kTileRows * (16 * win_pieces_for(kModeKWindows) + 4) + kLdsSlack <= 64 * 1024 &&
                  kTileRows * (16 * win_pieces_for(kModeKWindowsAny) + 4) + kLdsSlack <= 64 * 1024,
              "LDS per workgroup");
// wide windows take more than 64 KB of LDS (gfx950: up to 160 KB per workgroup, raised per kernel)
constexpr int kWideLdsBytes = kTileRows * (16 * win_pieces_for(kModeKWindowsWide) + 4) + kLdsSlack + 32;
static_assert(kWideLdsBytes <= 160 * 1024, "LDS per workgroup");
static_assert(win_pieces_for(kModeKWindows) * 16 >= kWinCols + 16 &&
                  win_pieces_for(kModeKWindowsWide) * 16 >= kWinColsWide + 16,
              "a window row and the piece past it fit one LDS row");

struct Params {
  const uint8_t *src;
  const int32_t *offs;
  uint8_t *out;
  int64_t ld;          // row stride in bytes
  int64_t out_bytes;   // whole output allocation
  int64_t units;       // work units
  int64_t vunits;      // workgroup slots: a multiple of 8 covering every unit
  int64_t deal;        // interleaved order: consecutive units dealt to one XCD at a time
  int rows;
  int cols;
  int groups;
  int padded_cols;     // M and per-expert: round_up(cols, 4)
  int unit_cols;       // columns per unit chunk (multiple of 4)
  int per_row;         // M: units per output row block; K: units per 128-row block
  int pitch;           // LDS row pitch (bytes) in per-row staging
  int pieces;          // 16-byte pieces per LDS row in per-row staging
  int trash;           // LDS offset of 16 bytes that staging pieces without data are written to
  int64_t expert_stride;  // per-expert matrices: bytes between experts
  int64_t row_blocks;     // per-expert matrices: 128-row blocks per expert
  int windows;            // K: column windows per row block (the first units of each)
  int tail_units;         // K: units per row block that zero-fill its slice of the tail
  int write_through;      // M and K launches of more than kWriteThroughBytes: stores also carry sc1
};

__device__ __forceinline__ int lane_value(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// ---------------------------------------------------------------------------
// group scan and lookup
// ---------------------------------------------------------------------------

// Where an M output row block sits among the groups: group sizes in rows,
// units are 128-row blocks.
struct GroupHit {
  int group;        // index of the group holding the block; == groups for the tail
  int start;        // first input row of the group
  int size;         // rows of the group
  int first_unit;   // row blocks of all earlier groups (all groups, for the tail)
};

// Scans the cumulative end offsets in 64-lane slices and finds the group that
// holds output row block `target`. Each end offset is clamped into
// [previous end, rows], which leaves valid offsets unchanged and keeps every
// access in bounds for invalid ones. Every lane of the wave must call it.
__device__ __forceinline__ GroupHit find_group(const int32_t *__restrict__ offs, int groups, int rows, int target) {
  const int lane = threadIdx.x & (kWave - 1);
  int carry_end = 0, carry_units = 0;
  for (int base = 0; base < groups; base += kWave) {
    const int g = base + lane;
    const bool active = g < groups;
    int end = active ? offs[g] : 0;
    end = min(max(end, 0), rows);
    end = max(wave_inclusive_max(end), carry_end);
    const int prev = wave_shift_up(end, carry_end);
    const int size = end - prev;                       // 0 for lanes past the last group
    const int units = (size + kTileRows - 1) / kTileRows;
    const int cum_units = wave_inclusive_sum(units) + carry_units;
    const unsigned long long before = __ballot(active && cum_units <= target);
    const int n = __popcll(before);
    if (n < min(kWave, groups - base)) {
      GroupHit h;
      h.group = base + n;
      h.start = lane_value(prev, n);
      h.size = lane_value(size, n);
      h.first_unit = lane_value(cum_units, n) - lane_value(units, n);
      return h;
    }
    carry_end = lane_value(end, kWave - 1);
    carry_units = lane_value(cum_units, kWave - 1);
  }
  GroupHit h;
  h.group = groups;
  h.start = carry_end;
  h.size = 0;
  h.first_unit = carry_units;
  return h;
}

// K groups: one 64-group slice of the group table, per lane (group base +
// lane): first column, end column, width padded to 4, and the padded widths of
// all earlier groups. end_raw is the lane's end offset (any value past the last
// group); the ends are clamped into a non-decreasing sequence in [0, cols].
struct KSlice {
  int start, end, width, before;
};

__device__ __forceinline__ KSlice k_slice(int end_raw, int base, int groups, int cols, int carry_end,
                                          int carry_width) {
  const bool active = base + int(threadIdx.x & (kWave - 1)) < groups;
  int e = active ? min(max(end_raw, 0), cols) : 0;
  e = max(wave_inclusive_max(e), carry_end);
  KSlice s;
  s.start = wave_shift_up(e, carry_end);
  s.end = e;
  s.width = active ? (e - s.start + 3) & ~3 : 0;
  s.before = wave_inclusive_sum(s.width) + carry_width - s.width;
  return s;
}

// End offset g through a buffer resource over the G offsets: 0 past the last
// group, by the buffer's range check rather than a branch (a load under a
// branch is waited for where the branch ends, not where it is used).
__device__ __forceinline__ int end_offset(__amdgpu_buffer_rsrc_t offs, int g) {
  return __builtin_amdgcn_raw_buffer_load_b32(offs, 4 * g, 0, 0);
}

// ---------------------------------------------------------------------------
// stores
// ---------------------------------------------------------------------------

// 16-byte store, streamed past the caches: the output is never read back here.
__device__ __forceinline__ void store16(uint8_t *dst, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = {a, b, c, d};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(dst));
}

// Zero-fill of part `part` of `parts` of the byte range [lo, hi) of an output
// of `limit` bytes; lo is 16-byte aligned and hi a multiple of 4 (both clamped
// into the output, write_ranges.h).
template <int NT>
__device__ __forceinline__ void zero_part(uint8_t *__restrict__ out, int64_t lo, int64_t hi, int64_t limit,
                                          int64_t part, int64_t parts) {
  const ZeroSpan z = zero_share(lo, hi, limit, part, parts);
  for (int64_t q = z.begin + 16 * threadIdx.x; q < z.full; q += 16 * NT) store16(out + q, 0, 0, 0, 0);
  for (int64_t q = z.full + 4 * threadIdx.x; q < z.end; q += 4 * NT) *reinterpret_cast<uint32_t *>(out + q) = 0u;
}

// ---------------------------------------------------------------------------
// staging a 128-row strip in LDS
// ---------------------------------------------------------------------------

template <int POLICY>
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t offset) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(offset), 0, POLICY);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Per-row staging: row r's segment [a, a + seg) with a = row_base + r*ld is
// fetched as the 16-byte pieces covering it into LDS row r (pitch bytes); its
// first byte then sits at r*pitch + (a mod 16). Piece slot s = r*pieces + k
// goes to lane s mod NT; each lane issues exactly N loads back to back (N =
// slots per lane of this unit) before it waits for any of them. `between`
// runs once they are issued, before the first wait.
struct Nothing {
  __device__ __forceinline__ void operator()() const {}
};

template <int NT, int N, int POLICY, typename F>
__device__ __forceinline__ void stage_rows_n(uint8_t *__restrict__ lds, int trash, __amdgpu_buffer_rsrc_t rsrc,
                                             uint32_t lead, int64_t ld, int nrows, int seg, int pitch, int pieces,
                                             F &between) {
  const int step_r = NT / pieces, step_k = NT % pieces;
  const int r0 = threadIdx.x / pieces, k0 = threadIdx.x % pieces;
  uint4 v[N];
  int r = r0, k = k0;
#pragma unroll
  for (int it = 0; it < N; ++it) {
    const uint32_t row_off = lead + uint32_t(r) * uint32_t(ld);  // in range whenever r < nrows
    const int need = int(((row_off & 15) + seg + 15) >> 4);
    const bool valid = r < nrows && k < need;
    v[it] = load16<POLICY>(rsrc, valid ? (row_off & ~15u) + 16 * k : kOutOfRange);
    r += step_r;
    k += step_k;
    if (k >= pieces) { k -= pieces; ++r; }
  }
  if constexpr (!std::is_same<F, Nothing>::value) {
    __builtin_amdgcn_sched_barrier(0);  // every load issued before `between` starts
    between();
  }
  // The same walk again (cheaper than keeping N offsets live across the
  // loads). Every piece is written, slots without data to the trash bytes at
  // the end of LDS: a write under a condition would let the compiler move its
  // load under that condition too, one load after another.
  r = r0;
  k = k0;
#pragma unroll
  for (int it = 0; it < N; ++it) {
    const uint32_t row_off = lead + uint32_t(r) * uint32_t(ld);
    const int need = int(((row_off & 15) + seg + 15) >> 4);
    const int off = (r < nrows && k < need) ? r * pitch + 16 * k : trash;
    uint32_t *d = reinterpret_cast<uint32_t *>(lds + off);  // 4-byte aligned rows
    d[0] = v[it].x;
    d[1] = v[it].y;
    d[2] = v[it].z;
    d[3] = v[it].w;
    r += step_r;
    k += step_k;
    if (k >= pieces) { k -= pieces; ++r; }
  }
}

// Runs stage_rows_n with the smallest N >= n (n uniform, 1 <= n <= N).
template <int NT, int N, int POLICY, typename F>
__device__ __forceinline__ void stage_rows_upto(int n, uint8_t *__restrict__ lds, int trash,
                                                __amdgpu_buffer_rsrc_t rsrc, uint32_t lead, int64_t ld, int nrows,
                                                int seg, int pitch, int pieces, F &between) {
  if constexpr (N > 1) {
    if (n < N) {
      stage_rows_upto<NT, N - 1, POLICY>(n, lds, trash, rsrc, lead, ld, nrows, seg, pitch, pieces, between);
      return;
    }
  }
  stage_rows_n<NT, N, POLICY>(lds, trash, rsrc, lead, ld, nrows, seg, pitch, pieces, between);
}

template <int NT, int ITERS, int POLICY, typename F = Nothing>
__device__ __forceinline__ void stage_rows(uint8_t *__restrict__ lds, int trash, const uint8_t *row_base, int64_t ld,
                                           int nrows, int seg, int pitch, int pieces, F &&between = F()) {
  const uint32_t lead = uint32_t(reinterpret_cast<uintptr_t>(row_base) & 15);
  const uint8_t *base = row_base - lead;  // 16-byte aligned
  const uint32_t span = uint32_t((lead + int64_t(nrows - 1) * ld + seg + 15) & ~int64_t(15));
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(base, span);
  stage_rows_upto<NT, ITERS, POLICY>((nrows * pieces + NT - 1) / NT, lds, trash, rsrc, lead, ld, nrows, seg, pitch,
                                     pieces, between);
}

// Flat staging: the strip is one contiguous range [a, a + len); its 16-byte
// cover goes to LDS from offset 0, so byte a sits at LDS (a mod 16). The
// pieces go straight into LDS: a buffer load with the LDS flag writes lane l's
// 16 bytes at the wave's LDS base (m0) + 16*l, which with the wave's base at
// its first piece is LDS offset 16*(piece index). Lanes past the cover load
// nothing.
typedef __attribute__((address_space(3))) void LdsVoid;   // an LDS address, as the LDS-load builtin takes it

template <int NT, int N, int POLICY>
__device__ __forceinline__ void stage_flat_n(uint8_t *__restrict__ lds, __amdgpu_buffer_rsrc_t rsrc, int n) {
  const int t = threadIdx.x;
  const int wave_first = t & ~(kWave - 1);   // piece of the wave's lane 0 in the first round
#pragma unroll
  for (int it = 0; it < N; ++it) {
    if (t + it * NT < n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LdsVoid *)(lds + 16 * (wave_first + it * NT)), 16,
                                               16 * (t + it * NT), 0, 0, POLICY);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): every piece has landed in LDS
}

// Runs stage_flat_n with the smallest N >= m (m uniform, 1 <= m <= N).
template <int NT, int N, int POLICY>
__device__ __forceinline__ void stage_flat_upto(int m, uint8_t *__restrict__ lds, __amdgpu_buffer_rsrc_t rsrc, int n) {
  if constexpr (N > 1) {
    if (m < N) {
      stage_flat_upto<NT, N - 1, POLICY>(m, lds, rsrc, n);
      return;
    }
  }
  stage_flat_n<NT, N, POLICY>(lds, rsrc, n);
}

template <int NT, int ITERS, int POLICY>
__device__ __forceinline__ void stage_flat(uint8_t *__restrict__ lds, const uint8_t *start, int len) {
  const uint32_t lead = uint32_t(reinterpret_cast<uintptr_t>(start) & 15);
  const int n = int((lead + len + 15) >> 4);
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(start - lead, uint32_t(16 * n));
  stage_flat_upto<NT, ITERS, POLICY>((n + NT - 1) / NT, lds, rsrc, n);
}

// Window staging for rows that start 128-byte aligned: LDS row r gets bytes
// [0, W) of the window row, lines no other unit reads, loaded with
// POLICY, and, when `extra`, bytes [W, W + 16), the first
// columns of the next window, loaded first and with the shared policy. Rows
// past nrows load zeros. `between` runs once every load is issued and before
// any is waited for.
template <int NT, int W, int POLICY, typename F>
__device__ __forceinline__ void stage_window(uint8_t *__restrict__ lds, int trash, __amdgpu_buffer_rsrc_t rsrc,
                                             int64_t ld, int nrows, bool extra, int pitch, F &&between) {
  constexpr int kPieces = W / 16;
  constexpr int kMain = kTileRows * kPieces / NT;
  static_assert(kTileRows * kPieces % NT == 0 && NT >= kTileRows, "window staging covers 128 rows");
  const int re = int(threadIdx.x);
  const uint4 x = load16<kSharedLoadPolicy>(
      rsrc, extra && re < nrows ? uint32_t(re) * uint32_t(ld) + W : kOutOfRange);
  uint4 v[kMain];
#pragma unroll
  for (int it = 0; it < kMain; ++it) {
    const int q = int(threadIdx.x) + NT * it;
    const int r = q / kPieces, k = q % kPieces;
    v[it] = load16<POLICY>(rsrc, r < nrows ? uint32_t(r) * uint32_t(ld) + 16 * k : kOutOfRange);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load issued before `between` starts
  between();
  // every piece is written (the piece past the window, when there is none, to
  // the trash bytes), see stage_rows_n; LDS rows are 4-byte aligned
  uint32_t *d = reinterpret_cast<uint32_t *>(lds + (extra && re < kTileRows ? re * pitch + W : trash));
  d[0] = x.x;
  d[1] = x.y;
  d[2] = x.z;
  d[3] = x.w;
#pragma unroll
  for (int it = 0; it < kMain; ++it) {
    const int q = int(threadIdx.x) + NT * it;
    d = reinterpret_cast<uint32_t *>(lds + (q / kPieces) * pitch + 16 * (q % kPieces));
    d[0] = v[it].x;
    d[1] = v[it].y;
    d[2] = v[it].z;
    d[3] = v[it].w;
  }
}

// ---------------------------------------------------------------------------
// emitting tiles from LDS
// ---------------------------------------------------------------------------

// Writes `tile_cols` tiles (128 rows x 4 columns each) contiguously at dst.
// Row r, column c of the unit is LDS byte row_off(r) + c with
// row_off(r) = first + r*row_step (FLAT) or first + r*row_step + (addr + r*ld)
// mod 16 (per-row staging, where `first` is the unit's column in the staged
// segment).
// Rows >= nrows and columns >= ncols are written as zero. With WT the stores
// go through a buffer resource over the run and carry sc1 as well.
template <int NT, bool FLAT, bool ALIGNED, bool WT>
__device__ __forceinline__ void emit_tiles(const uint8_t *__restrict__ lds, uint8_t *__restrict__ dst,
                                           int tile_cols, int nrows, int ncols, int first, int row_step,
                                           uintptr_t addr, int64_t ld) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t *w32 = reinterpret_cast<const uint32_t *>(lds);
  const int n16 = tile_cols * 32;
  __amdgpu_buffer_rsrc_t orsrc;
  if constexpr (WT) orsrc = byte_buffer(dst, uint32_t(n16) * 16u);
  for (int v = threadIdx.x; v < n16; v += NT) {
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
        if (!FLAT) b += int((uint32_t(addr) + uint32_t(r) * uint32_t(ld)) & 15u);  // (addr + r*ld) mod 16
        if (ALIGNED) {
          x = w32[b >> 2];
        } else {
          x = __builtin_amdgcn_alignbyte(w32[(b >> 2) + 1], w32[b >> 2], b & 3);
        }
        x &= mask;
      }
      w[q] = x;
    }
    if constexpr (WT)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, orsrc, 16 * v, 0, kStoreNtSc1);
    else
      store16(dst + 16 * int64_t(v), w[0], w[1], w[2], w[3]);
  }
}

// Stages one unit of `nrows` rows x `ncols` source columns starting at
// row_base (row stride ld) and writes its tile_cols tiles at dst.
template <int MODE, bool WT>
__device__ __forceinline__ void copy_unit(uint8_t *__restrict__ lds, const Params &p, const uint8_t *row_base,
                                          int nrows, int ncols, int tile_cols, uint8_t *dst) {
  constexpr int NT = threads_for(MODE);
  constexpr bool FLAT = MODE == kModeMFlat;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row_base);
  bool aligned;
  if (FLAT) {
    stage_flat<NT, load_iters_for(MODE), kFlatLoadPolicy>(lds, row_base, nrows * ncols);
    aligned = ((a & 3) == 0) && ((ncols & 3) == 0);
  } else {
    stage_rows<NT, load_iters_for(MODE), load_policy_for(MODE)>(lds, p.trash, row_base, p.ld, nrows, ncols,
                                                                p.pitch, p.pieces);
    aligned = ((a & 3) == 0) && ((p.ld & 3) == 0);
  }
  __syncthreads();
  const int first = FLAT ? int(a & 15) : 0;
  const int step = FLAT ? ncols : p.pitch;
  if (aligned)
    emit_tiles<NT, FLAT, true, WT>(lds, dst, tile_cols, nrows, ncols, first, step, a, p.ld);
  else
    emit_tiles<NT, FLAT, false, WT>(lds, dst, tile_cols, nrows, ncols, first, step, a, p.ld);
}

// K groups: the unit of 128-row block `block` and input window `slot` (columns
// [W*slot, W*slot + W) with W the mode's window width, plus up to 3 past it).
// The window's loads go out first; the first 64 end offsets (end_raw, loaded
// before them) are scanned while they are in flight. Then, for every group with
// a tile starting in the window, the run of those tiles is written at the
// group's place: group g's blocked matrix starts at byte padded_rows * (padded
// widths before g), its row block `block` 128 * width_g bytes further per
// block, tile k 512*k on.
template <int NT, int MODE, bool WT>
__device__ __forceinline__ void window_unit(uint8_t *__restrict__ lds, const Params &p, int64_t block, int slot,
                                            __amdgpu_buffer_rsrc_t offs, int end_raw, int64_t padded_rows) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr bool LINE_ALIGNED = is_line_window(MODE);
  constexpr int W = win_cols_for(MODE);
  const int c_lo = slot * W;                            // < cols
  const int64_t c_hi = int64_t(c_lo) + W;
  const int nrows = min(kTileRows, p.rows - kTileRows * int(block));
  const int seg = int(std::min<int64_t>(win_span_for(MODE), int64_t(p.cols) - c_lo));
  const uint8_t *row_base = p.src + block * kTileRows * p.ld + c_lo;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row_base);
  KSlice first;
  auto scan = [&] { first = k_slice(end_raw, 0, p.groups, p.cols, 0, 0); };
  if constexpr (LINE_ALIGNED) {
    const uint32_t span = uint32_t((int64_t(nrows - 1) * p.ld + seg + 15) & ~int64_t(15));
    stage_window<NT, W, kWindowLoadPolicy>(lds, p.trash, byte_buffer(row_base, span), p.ld, nrows, seg > W,
                                           p.pitch, scan);
  } else {
    stage_rows<NT, load_iters_for(MODE), load_policy_for(MODE)>(lds, p.trash, row_base, p.ld, nrows, seg, p.pitch,
                                                                p.pieces, scan);
  }
  __syncthreads();
  const bool aligned = ((a | uintptr_t(p.ld)) & 3) == 0;
  int carry_end = 0, carry_width = 0;
  for (int base = 0; base < p.groups; base += kWave) {
    const KSlice sl = base == 0 ? first
                                : k_slice(end_offset(offs, base + lane), base, p.groups, p.cols, carry_end,
                                          carry_width);
    // a group has a tile starting in the window iff its first tile starts
    // before the window ends and its last tile (at start + width - 4) does
    // not start before the window
    const bool hit = base + lane < p.groups && sl.width > 0 && sl.start < c_hi &&
                     sl.start + sl.width - 4 >= c_lo;
    for (unsigned long long m = __ballot(hit); m != 0; m &= m - 1) {
      const int n = __builtin_ctzll(m);
      const int gs = lane_value(sl.start, n), ge = lane_value(sl.end, n);
      const int gw = lane_value(sl.width, n), gb = lane_value(sl.before, n);
      const int k_lo = gs >= c_lo ? 0 : (c_lo - gs + 3) >> 2;
      const int k_hi = int(std::min<int64_t>(gw >> 2, (c_hi - gs + 3) >> 2));
      const int col0 = gs + 4 * k_lo;                   // first column of the run, in the window
      const int64_t dst_off = padded_rows * gb + block * kTileRows * gw + int64_t(512) * k_lo;
      // (a correct table always passes: the run lies inside the output)
      if (k_hi <= k_lo || !fits(dst_off, int64_t(512) * (k_hi - k_lo), p.out_bytes)) continue;
      uint8_t *dst = p.out + dst_off;
      if (aligned && ((col0 - c_lo) & 3) == 0)
        emit_tiles<NT, false, true, WT>(lds, dst, k_hi - k_lo, nrows, ge - col0, col0 - c_lo, p.pitch, a, p.ld);
      else
        emit_tiles<NT, false, false, WT>(lds, dst, k_hi - k_lo, nrows, ge - col0, col0 - c_lo, p.pitch, a, p.ld);
    }
    carry_end = lane_value(sl.end, kWave - 1);
    carry_width = lane_value(sl.before + sl.width, kWave - 1);
    if (carry_end >= c_hi) break;  // later groups start past the window
  }
}

// ---------------------------------------------------------------------------
// the kernel: one work unit per workgroup (a grid-stride loop only when the
// grid is capped). A workgroup ends as soon as its stores are issued, so the
// next one on the CU loads while those stores drain.
// ---------------------------------------------------------------------------

template <int MODE, bool WT, bool IL>
__global__ __launch_bounds__(threads_for(MODE)) __attribute__((amdgpu_waves_per_eu(kMinWavesPerEu)))
void rearrange_kernel(Params p) {
  constexpr int NT = threads_for(MODE);
  constexpr bool KGROUPS = is_k(MODE);
  extern __shared__ __align__(16) uint8_t lds[];
  bool first_iter = true;
  for (int64_t vb = blockIdx.x; vb < p.vunits; vb += gridDim.x) {
    // the order of units over the XCDs (launch_order.h): runs of p.deal units
    // dealt in turn (IL) or contiguous ranges
    const int64_t unit = unit_of_slot<IL>(vb, p.vunits, p.deal);
    if (unit >= p.units) continue;
    if (!first_iter) __syncthreads();  // LDS of the previous unit is no longer read
    first_iter = false;

    const int64_t block = unit / p.per_row;             // output row block (M) / 128-row block (K)
    const int slot = int(unit - block * p.per_row);     // column chunk (M) / unit within the row block (K)

    if constexpr (is_3d(MODE)) {
      // expert e's row block rb is output row block e*row_blocks + rb; every
      // unit holds data (rows >= 1, and a chunk starts below round_up(cols,4)
      // at a multiple of 4, hence below cols), so the units cover the output
      const int64_t e = block / p.row_blocks;
      const int rb = int(block - e * p.row_blocks);
      const int nrows = min(kTileRows, p.rows - kTileRows * rb);
      const int c0 = slot * p.unit_cols;
      const int ncols = min(p.unit_cols, p.cols - c0);
      const int tile_cols = min(p.unit_cols, p.padded_cols - c0) >> 2;
      uint8_t *dst = p.out + block * int64_t(kTileRows) * p.padded_cols + int64_t(c0) * kTileRows;
      if (nrows > 0 && ncols > 0)
        copy_unit<MODE, WT>(lds, p, p.src + e * p.expert_stride + int64_t(kTileRows) * rb * p.ld + c0, nrows, ncols,
                        tile_cols, dst);
    } else if constexpr (!KGROUPS) {
      const GroupHit h = find_group(p.offs, p.groups, p.rows, int(block));
      const int64_t row_block_bytes = int64_t(kTileRows) * p.padded_cols;
      if (h.group < p.groups) {
        const int k = int(block) - h.first_unit;
        const int row0 = h.start + kTileRows * k;
        // the min() with rows - row0 only restates what a correct scan guarantees
        const int nrows = min(min(kTileRows, h.size - kTileRows * k), p.rows - row0);
        const int c0 = slot * p.unit_cols;
        const int ncols = min(p.unit_cols, p.cols - c0);
        const int tile_cols = min(p.unit_cols, p.padded_cols - c0) >> 2;
        uint8_t *dst = p.out + block * row_block_bytes + int64_t(c0) * kTileRows;
        // the last two conditions, too, hold for every unit of a correct scan
        if (nrows > 0 && ncols > 0 && row0 >= 0 && (block + 1) * row_block_bytes <= p.out_bytes)
          copy_unit<MODE, WT>(lds, p, p.src + int64_t(row0) * p.ld + c0, nrows, ncols, tile_cols, dst);
      } else {
        const int64_t nblocks = p.units / p.per_row;
        const int64_t tail_units = int64_t(p.per_row) * (nblocks - h.first_unit);
        const int64_t tail_index = (block - h.first_unit) * p.per_row + slot;
        zero_part<NT>(p.out, int64_t(h.first_unit) * row_block_bytes, p.out_bytes, p.out_bytes, tail_index,
                      tail_units);
      }
    } else {
      // the end offsets of the first 64 groups are loaded ahead of everything
      // else, so that waiting for them does not wait for the strip loads
      const __amdgpu_buffer_rsrc_t offs = byte_buffer(p.offs, 4 * uint32_t(p.groups));
      const int end_raw = end_offset(offs, int(threadIdx.x & (kWave - 1)));
      __builtin_amdgcn_sched_barrier(0);
      const int64_t padded_rows = int64_t(((p.rows + kTileRows - 1) / kTileRows)) * kTileRows;
      if (slot < p.windows) {
        window_unit<NT, MODE, WT>(lds, p, block, slot, offs, end_raw, padded_rows);
      } else {
        // tail: round_up(rows,128) * (cols + 4G - padded total) zero bytes, a
        // 128 * (cols + 4G - padded total) slice per 128-row block
        const int lane = threadIdx.x & (kWave - 1);
        int carry_end = 0, carry_width = 0;
        for (int base = 0; base < p.groups; base += kWave) {
          const KSlice sl = k_slice(base == 0 ? end_raw : end_offset(offs, base + lane), base, p.groups, p.cols,
                                    carry_end, carry_width);
          carry_end = lane_value(sl.end, kWave - 1);
          carry_width = lane_value(sl.before + sl.width, kWave - 1);
        }
        const int64_t tail_cols = int64_t(p.cols) + 4 * int64_t(p.groups) - carry_width;
        const int64_t lo = padded_rows * carry_width + block * kTileRows * tail_cols;
        zero_part<NT>(p.out, lo, lo + kTileRows * tail_cols, p.out_bytes, slot - p.windows, p.tail_units);
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

int dispatch(Params &p, int mode, int64_t units, hipStream_t stream);

// Workgroups of the K window kernels (256- and 512-column windows) that the
// current GPU holds at once: CUs times the workgroups one CU holds (registers,
// LDS, waves), as the runtime's occupancy query reports them, found once per
// device. The 512-column kernel's LDS allowance is raised above 64 KB in the
// same step. 0 when a query fails (the 256-column windows are used then).
constexpr int kMaxDevices = 64;
struct Resident {
  int64_t narrow = 0, wide = 0;
};

Resident resident_windows() {
  static std::once_flag once[kMaxDevices];
  static Resident cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Resident();
  std::call_once(once[dev], [dev] {
    const void *narrow = reinterpret_cast<const void *>(&rearrange_kernel<kModeKWindows, false, false>);
    const void *wide = reinterpret_cast<const void *>(&rearrange_kernel<kModeKWindowsWide, false, false>);
    int cus = 0, per_cu_narrow = 0, per_cu_wide = 0;
    const size_t lds_narrow = size_t(kTileRows) * (16 * win_pieces_for(kModeKWindows) + 4) + kLdsSlack + 32;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipFuncSetAttribute(wide, hipFuncAttributeMaxDynamicSharedMemorySize, kWideLdsBytes) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_narrow, narrow, threads_for(kModeKWindows),
                                                     lds_narrow) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_wide, wide, threads_for(kModeKWindowsWide),
                                                     kWideLdsBytes) != hipSuccess)
      return;   // cache stays {0, 0}
    cache[dev].narrow = int64_t(cus) * per_cu_narrow;
    cache[dev].wide = int64_t(cus) * per_cu_wide;
  });
  return cache[dev];
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

  Params p = {};
  p.src = scales;
  p.offs = offs;
  p.out = out;
  p.ld = ld;
  p.out_bytes = out_bytes;
  p.rows = int(rows);
  p.cols = int(cols);
  p.groups = groups;
  p.padded_cols = int(round_up(cols, 4));
  p.write_through = rows * cols + out_bytes > kWriteThroughBytes;
  int mode;
  int64_t units;
  if (!kgroups) {
    // row blocks: every group's data plus at least one block of tail
    const int64_t blocks = (rows + kTileRows - 1) / kTileRows + groups;
    if (ld == cols && cols <= kFlatMaxCols && (cols % 16) != 0) {
      // packed narrow rows that are not whole 16-byte pieces: one flat range per strip
      mode = kModeMFlat;
      p.unit_cols = p.padded_cols;
    } else {
      // split row blocks into column chunks while there are too few units to fill the chip
      int uc = std::min<int>(kMaxUnitCols, p.padded_cols);
      while (uc > kMinUnitCols && blocks * ((p.padded_cols + uc - 1) / uc) < kTargetUnits)
        uc = std::max<int>(kMinUnitCols, int(round_up(uc / 2, 4)));
      p.unit_cols = uc;
      mode = uc <= kNarrowUnitCols ? kModeMRowsNarrow : kModeMRows;
    }
    p.per_row = (p.padded_cols + p.unit_cols - 1) / p.unit_cols;
    units = blocks * p.per_row;
  } else {
    // windows stream their own lines when every row starts on a 128-byte line
    mode = ((reinterpret_cast<uintptr_t>(scales) | uintptr_t(ld)) & 127) == 0 ? kModeKWindows : kModeKWindowsAny;
    const int64_t row_blocks = (rows + kTileRows - 1) / kTileRows;
    p.tail_units = int((4 * int64_t(groups) + kTailColsPerUnit - 1) / kTailColsPerUnit);
    if (mode == kModeKWindows) {
      // 512-column windows when the 256-column grid needs more than one pass
      // over the workgroups the GPU holds at once but the 512-column grid fits
      // in one: the second pass would run a few hundred workgroups on an
      // otherwise idle chip (measured on (7168, 4096): 14.1 vs 15.3 us; on
      // shapes with several passes or with room to spare 256 columns are
      // faster, e.g. (28672, 8192) 82.4 vs 83.4, (4096, 4096) 10.5 vs 11.6)
      const Resident res = resident_windows();
      const int64_t units_narrow = row_blocks * ((cols + kWinCols - 1) / kWinCols + p.tail_units);
      const int64_t units_wide = row_blocks * ((cols + kWinColsWide - 1) / kWinColsWide + p.tail_units);
      if (res.narrow > 0 && res.wide > 0 && units_narrow > res.narrow && units_wide <= res.wide)
        mode = kModeKWindowsWide;
    }
    p.unit_cols = win_cols_for(mode);
    // units per 128-row block: its input windows, then the tail units
    p.windows = int((cols + p.unit_cols - 1) / p.unit_cols);
    p.per_row = p.windows + p.tail_units;
    units = row_blocks * p.per_row;
  }
  return dispatch(p, mode, units, stream);
}

// Per-expert matrices: one unit per (expert, 128-row block, column chunk).
int launch_3d(const uint8_t *scales, int64_t experts, int64_t rows, int64_t cols, int64_t expert_stride,
              int64_t ld, uint8_t *out, hipStream_t stream) {
  const int64_t out_bytes = mx_rearrange_3d_out_bytes(experts, rows, cols);
  if (out_bytes < 0 || ld < cols || ld > kMaxRowStride || expert_stride < 0) return MX_REARRANGE_ESHAPE;
  if (experts > 1 && expert_stride > INT64_MAX / experts) return MX_REARRANGE_ESHAPE;
  if (experts * rows * cols > 0 && scales == nullptr) return MX_REARRANGE_ENULL;
  if (out_bytes > 0 && out == nullptr) return MX_REARRANGE_ENULL;
  if (reinterpret_cast<uintptr_t>(out) & 15) return MX_REARRANGE_EALIGN;
  if (out_bytes == 0) return MX_REARRANGE_OK;

  Params p = {};
  p.src = scales;
  p.out = out;
  p.ld = ld;
  p.out_bytes = out_bytes;
  p.rows = int(rows);
  p.cols = int(cols);
  p.groups = 0;
  p.padded_cols = int(round_up(cols, 4));
  p.expert_stride = expert_stride;
  p.row_blocks = (rows + kTileRows - 1) / kTileRows;
  const int64_t blocks = experts * p.row_blocks;
  // balanced column chunks of at most k3dMaxUnitCols; more of them while the
  // grid is too small to fill the chip
  int per_row = (p.padded_cols + k3dMaxUnitCols - 1) / k3dMaxUnitCols;
  auto chunk = [&](int n) { return int(round_up((p.padded_cols + n - 1) / n, 4)); };
  while (blocks * per_row < kTargetUnits && chunk(per_row + 1) >= kMinUnitCols && chunk(per_row + 1) < chunk(per_row))
    ++per_row;
  p.unit_cols = chunk(per_row);
  p.per_row = (p.padded_cols + p.unit_cols - 1) / p.unit_cols;
  const int64_t units = blocks * p.per_row;
  return dispatch(p, units > k3dWideUnits ? kMode3dWide : kMode3d, units, stream);
}

// The kernel of a mode: <MODE, WT (sc1 stores), IL (interleaved grid)>. The
// sc1 stores are built for the modes that run launches past the MALL size (M
// row segments and flat strips, K windows of line-aligned rows and of other
// rows), and such launches always take more than one pass over the chip, so
// they come interleaved. Per-expert launches measured the same with and
// without sc1 (336 MB: 57.4 us) and narrow M units never reach that size.
// 512-column K windows are chosen only for grids of one pass.
template <int MODE>
const void *kernel_of(bool wt, bool il) {
  if (wt) return reinterpret_cast<const void *>(&rearrange_kernel<MODE, true, true>);
  return il ? reinterpret_cast<const void *>(&rearrange_kernel<MODE, false, true>)
            : reinterpret_cast<const void *>(&rearrange_kernel<MODE, false, false>);
}

template <int MODE>
const void *kernel_plain(bool il) {
  return il ? reinterpret_cast<const void *>(&rearrange_kernel<MODE, false, true>)
            : reinterpret_cast<const void *>(&rearrange_kernel<MODE, false, false>);
}

constexpr bool is_write_through_mode(int mode) {
  return mode == kModeMFlat || mode == kModeMRows || mode == kModeKWindows || mode == kModeKWindowsAny;
}

const void *kernel_for(int mode, bool wt, bool il) {
  switch (mode) {
    case kModeMFlat: return kernel_of<kModeMFlat>(wt, il);
    case kModeMRows: return kernel_of<kModeMRows>(wt, il);
    case kModeKWindows: return kernel_of<kModeKWindows>(wt, il);
    case kModeKWindowsAny: return kernel_of<kModeKWindowsAny>(wt, il);
    case kModeMRowsNarrow: return kernel_plain<kModeMRowsNarrow>(il);
    case kMode3d: return kernel_plain<kMode3d>(il);
    case kMode3dWide: return kernel_plain<kMode3dWide>(il);
    default: return reinterpret_cast<const void *>(&rearrange_kernel<kModeKWindowsWide, false, false>);
  }
}

int dispatch(Params &p, int mode, int64_t units, hipStream_t stream) {
  // widest row segment of a unit; K windows always get room for a whole
  // window row and the piece past it
  const int64_t seg = is_k(mode) ? p.unit_cols + 3 : std::min<int64_t>(p.cols, p.unit_cols);
  p.pieces = std::max<int>(1, int((seg + 30) / 16));
  p.pitch = 16 * p.pieces + 4;
  p.units = units;
  // staged strip, then kLdsSlack bytes read past it by unaligned reads, then 16 trash bytes
  size_t lds_bytes = mode == kModeMFlat ? size_t(kTileRows) * size_t(p.cols) + 32 + kLdsSlack
                                        : size_t(kTileRows) * size_t(p.pitch) + kLdsSlack;
  lds_bytes = (lds_bytes + 15) & ~size_t(15);
  p.trash = int(lds_bytes);
  lds_bytes += 16;

  const int threads = threads_for(mode);
  // A grid of more than one pass over the workgroups the GPU holds at once
  // deals runs of units (row blocks, or for K a part of one) to the XCDs in
  // turn (rows of every XCD's units are then neighbours in memory, and each
  // pass reads one region of the input),
  // measured 3-11% faster on such grids: (28672, 8192) K groups 75.8 against
  // 80.3 us, 64 x 8192 x 160 per-expert 28.85 against 30.1, (1048576, 160) M
  // groups 60.8 against 63.2. A grid of one pass keeps contiguous ranges per
  // XCD (interleaved, the (131072, 44) M shape took 4.54 against 4.18 us).
  const bool wt = p.write_through != 0;
  const int64_t resident = resident_workgroups(kernel_for(mode, false, false), threads, lds_bytes);
  const bool il = mode != kModeKWindowsWide && (wt || (resident > 0 && units > resident));
  const void *fn = kernel_for(mode, wt && is_write_through_mode(mode), il);
  // The interleaved order deals runs of consecutive units to the XCDs in turn.
  // M and per-expert units: four whole row blocks per run (a row block's units
  // share lines at their edges), measured 60.1 against 60.9 us on (1048576,
  // 160) M groups, 34.5 against 34.9 on (524288, 160), the same on (6291456,
  // 44) and on 64 x 8192 x 160 per-expert scales; a run of half a row block
  // took 83.4 us on (1048576, 160). K windows: runs of kKDealWindows windows
  // when a row block holds at least twice that many units, else whole row
  // blocks: (28672, 8192) 74.9 against 75.9 us, (8192, 16384) 44.2 against
  // 45.1, (28672, 12288) 112.1 against 113.0, rows off 128-byte lines (14336,
  // 8196) 43.0 against 43.7; with 4096 columns (17 units per row block) whole
  // row blocks stayed best (runs of 11: 23.7 against 23.1 us on (14336, 4096)).
  if (is_k(mode))
    p.deal = p.per_row >= 2 * kKDealWindows ? kKDealWindows : p.per_row;
  else
    p.deal = int64_t(kMDealBlocks) * p.per_row;
  p.vunits = slots_for(il, units, p.deal);
  // one workgroup per unit slot; the grid is a multiple of 8, so a workgroup
  // that loops (only past kMaxGrid slots) stays on its XCD
  const int64_t grid = std::min<int64_t>(p.vunits, kMaxGrid);

  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(threads), args, lds_bytes, stream);
  return e == hipSuccess ? MX_REARRANGE_OK : MX_REARRANGE_ELAUNCH;
}

}  // namespace

extern "C" {

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

int mx_block_rearrange_3d(const uint8_t *scales, int64_t experts, int64_t rows, int64_t cols,
                          int64_t expert_stride, int64_t row_stride, uint8_t *out, hipStream_t stream) {
  return launch_3d(scales, experts, rows, cols, expert_stride, row_stride, out, stream);
}

}  // extern "C"
