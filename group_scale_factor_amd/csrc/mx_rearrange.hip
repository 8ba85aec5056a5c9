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
//   * One workgroup handles one work unit: 128 rows x a column chunk of one
//     group, i.e. a run of whole output tiles that are contiguous in the output.
//   * Group lookup: every wave loads the end offsets, one group per lane,
//     clamps them into a non-decreasing sequence, and forms the padded sizes
//     and their prefix sums with DPP scans; a ballot over the cumulative unit
//     counts names the group of the unit. G > 64 is handled in 64-lane slices
//     with a carry.
//   * Load: the unit's source bytes are fetched as 16-byte aligned pieces
//     (buffer_load_dwordx4) covering each row segment (or, for packed narrow
//     rows, the whole strip as one range) and staged in LDS. A 16-byte aligned
//     piece that contains at least one byte of the matrix lies inside the same
//     memory page as that byte, so the cover never touches a page the matrix
//     does not; the extra bytes are never emitted.
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

constexpr int kWave = 64;
constexpr int kTileRows = 128;
// Widest column chunk of a unit: 240 columns are covered by at most 16 aligned
// 16-byte pieces per row at any alignment, so a 128-row unit is 2048 pieces,
// exactly 8 per producer lane.
constexpr int kMaxUnitCols = 240;
constexpr int kMinUnitCols = 32;              // narrowest chunk the host splits M row blocks into
constexpr int kTargetUnits = 1024;            // M: split row blocks into chunks until this many units
constexpr int kFlatMaxCols = 60;              // M: widest packed row staged as one flat range
constexpr int kMaxPieces = (kMaxUnitCols + 30) / 16;   // 16-byte pieces covering one row segment
constexpr int kMaxPitch = 16 * kMaxPieces + 4;         // LDS row pitch: 4*pieces+1 words, odd
constexpr int kMaxFlatPieces = (kTileRows * kFlatMaxCols + 30) / 16;
constexpr int kLdsSlack = 16;                 // room for the second word of an unaligned read
constexpr int64_t kMaxGrid = int64_t(1) << 20;
constexpr int64_t kMaxRowStride = int64_t(1) << 24;   // keeps a unit's byte span inside 32-bit buffer offsets
constexpr uint32_t kOutOfRange = 0xfffffff0u;          // buffer offset past any range: the load returns 0
constexpr int kRawBufferFlags = 0x00020000;            // buffer descriptor word 3: 32-bit raw data
// Cache policy of the staging loads (buffer instruction bit 1: non-temporal).
// Flat strips share at most one line with their neighbour, so they stream;
// row segments of neighbouring units share lines, which must stay in L2.
constexpr int kFlatLoadPolicy = 2;
constexpr int kRowsLoadPolicy = 0;

// Staging modes; each is its own kernel instantiation.
enum Mode : int {
  kModeMFlat = 0,   // M groups, packed rows of <= 64 bytes, one contiguous range per 128-row strip
  kModeMRows = 1,   // M groups, one row segment at a time
  kModeKRows = 2,   // K groups, one row segment at a time
};

// Each workgroup is split into producer waves, which only load (global ->
// registers -> LDS), and consumer waves, which only store (LDS -> global).
// On gfx9 one counter tracks both loads and stores of a wave, so a wave that
// did both would wait for its own stores to be acknowledged whenever it waited
// for a load; split roles keep the stores fire-and-forget.
constexpr int producers_for(int mode) { return mode == kModeMFlat ? 64 : 256; }
constexpr int consumers_for(int mode) { return mode == kModeMFlat ? 128 : 256; }
constexpr int threads_for(int mode) { return producers_for(mode) + consumers_for(mode); }
constexpr int load_iters_for(int mode) {
  return ((mode == kModeMFlat ? kMaxFlatPieces : kTileRows * kMaxPieces) + producers_for(mode) - 1) /
         producers_for(mode);
}
constexpr int store_iters_for(int mode) {
  return (kTileRows * (mode == kModeMFlat ? kFlatMaxCols : kMaxUnitCols) / 16 + consumers_for(mode) - 1) /
         consumers_for(mode);
}
// Persistent launch: as many workgroups as fit at once, each looping over its
// units with two LDS buffers (loads of the next unit overlap the stores of
// the current one). Otherwise one workgroup per unit.
constexpr bool kPersistent = true;
// Register budget: at least 4 waves per SIMD (<= 128 VGPRs), so that two
// 8-wave workgroups share a CU, as their LDS buffers allow.
constexpr int kMinWavesPerEu = 4;

static_assert(kMaxUnitCols % 4 == 0 && kMinUnitCols % 4 == 0, "units are whole tile columns");
static_assert(kTileRows * kMaxPitch + kLdsSlack <= 32 * 1024 + 4096, "LDS per buffer");
static_assert(producers_for(kModeMFlat) % kWave == 0 && producers_for(kModeKRows) % kWave == 0,
              "roles are whole waves");

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
  int unit_cols;       // columns per unit chunk (multiple of 4)
  int per_row;         // M: units per output row block; K: units per 128-row block
  int pitch;           // LDS row pitch (bytes) in per-row staging
  int pieces;          // 16-byte pieces per LDS row in per-row staging
  int lds_stride;      // bytes per LDS buffer
};

// ---------------------------------------------------------------------------
// wave64 scans with DPP (row shifts within 16-lane rows, then row broadcasts)
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ int dpp_shr(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, true);  // lanes without a source read 0
}

__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += dpp_shr<0x111>(x);                                          // row_shr:1
  x += dpp_shr<0x112>(x);                                          // row_shr:2
  x += dpp_shr<0x114>(x);                                          // row_shr:4
  x += dpp_shr<0x118>(x);                                          // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Inclusive running maximum of non-negative values.
__device__ __forceinline__ int wave_inclusive_max(int x) {
  x = max(x, dpp_shr<0x111>(x));
  x = max(x, dpp_shr<0x112>(x));
  x = max(x, dpp_shr<0x114>(x));
  x = max(x, dpp_shr<0x118>(x));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return x;
}

// Value of the previous lane (wave_shr:1); lane 0 gets `first`.
__device__ __forceinline__ int wave_shift_up(int x, int first) {
  return __builtin_amdgcn_update_dpp(first, x, 0x138, 0xf, 0xf, false);
}

__device__ __forceinline__ int lane_value(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// ---------------------------------------------------------------------------
// group scan and lookup
// ---------------------------------------------------------------------------

// Where a work unit sits among the groups. Group sizes are counted in rows (M)
// or scale columns (K); "units" are 128-row blocks (M) or unit_cols-column
// chunks of one 128-row block (K).
struct GroupHit {
  int group;        // index of the group holding the unit; == groups for the tail
  int start;        // first input row (M) / column (K) of the group
  int size;         // rows (M) / columns (K) of the group
  int first_unit;   // units of all earlier groups (all groups, for the tail)
  int padded_start; // K: padded columns of all earlier groups (all groups, for the tail)
};

// Scans the cumulative end offsets in 64-lane slices and finds the group that
// holds unit `target`. limit = rows (M) or cols (K): each end offset is clamped
// into [previous end, limit], which leaves valid offsets unchanged and keeps
// every access in bounds for invalid ones. Every lane of the wave must call it.
template <bool KGROUPS>
__device__ GroupHit find_group(const int32_t *__restrict__ offs, int groups, int limit, int unit_cols,
                               int target) {
  const int lane = threadIdx.x & (kWave - 1);
  int carry_end = 0, carry_units = 0, carry_padded = 0;
  for (int base = 0; base < groups; base += kWave) {
    const int g = base + lane;
    const bool active = g < groups;
    int end = active ? offs[g] : 0;
    end = min(max(end, 0), limit);
    end = max(wave_inclusive_max(end), carry_end);
    const int prev = wave_shift_up(end, carry_end);
    const int size = end - prev;                       // 0 for lanes past the last group
    const int padded = KGROUPS ? (size + 3) & ~3 : 0;  // K: width padded to 4 columns
    const int units = KGROUPS ? (padded + unit_cols - 1) / unit_cols : (size + kTileRows - 1) / kTileRows;
    const int cum_units = wave_inclusive_sum(units) + carry_units;
    const int cum_padded = KGROUPS ? wave_inclusive_sum(padded) + carry_padded : 0;
    const unsigned long long before = __ballot(active && cum_units <= target);
    const int n = __popcll(before);
    if (n < min(kWave, groups - base)) {
      GroupHit h;
      h.group = base + n;
      h.start = lane_value(prev, n);
      h.size = lane_value(size, n);
      h.first_unit = lane_value(cum_units, n) - lane_value(units, n);
      h.padded_start = KGROUPS ? lane_value(cum_padded, n) - lane_value(padded, n) : 0;
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
  return h;
}

// ---------------------------------------------------------------------------
// work units
// ---------------------------------------------------------------------------

enum UnitKind : int { kNone = 0, kData = 1, kTail = 2 };

struct Unit {
  int kind;
  // data: nrows x ncols source bytes from row_base (row stride ld) -> tile_cols tiles at dst
  const uint8_t *row_base;
  uint8_t *dst;
  int nrows, ncols, tile_cols;
  // tail: part `part` of `parts` of the zero range [lo, hi)
  int64_t lo, hi, part, parts;
};

// What consumers need of a unit, written into the head of its LDS buffer by
// the producers (consumers then issue no global load at all).
struct UnitDesc {
  int kind, nrows, ncols, tile_cols;
  uint32_t src_lo;  // low 32 bits of the unit's source address (row alignment)
  uint32_t unused;
  uint64_t dst;
  int64_t lo, hi, part, parts;
};
constexpr int kHeaderBytes = 64;  // LDS bytes before a buffer's data
static_assert(sizeof(UnitDesc) <= kHeaderBytes && kHeaderBytes % 16 == 0, "descriptor header");

// Maps virtual block vb to its unit and resolves it against the groups. Every
// lane of the wave must call it (it runs wave-wide scans).
template <bool KGROUPS>
__device__ Unit resolve(const Params &p, int64_t vb) {
  Unit u;
  u.kind = kNone;
  u.row_base = p.src;
  u.dst = p.out;
  u.nrows = u.ncols = u.tile_cols = 0;
  u.lo = u.hi = u.part = 0;
  u.parts = 1;
  if (vb >= p.vunits) return u;
  // consecutive units on one XCD: workgroup b runs on XCD b mod 8, and vb = b (mod 8)
  const int64_t unit = (vb & 7) * (p.vunits >> 3) + (vb >> 3);
  if (unit >= p.units) return u;
  const int64_t block = unit / p.per_row;           // output row block (M) / 128-row block (K)
  const int slot = int(unit - block * p.per_row);   // column chunk (M) / unit within the row block (K)
  if (!KGROUPS) {
    const GroupHit h = find_group<false>(p.offs, p.groups, p.rows, p.unit_cols, int(block));
    const int64_t row_block_bytes = int64_t(kTileRows) * p.padded_cols;
    if (h.group < p.groups) {
      const int k = int(block) - h.first_unit;
      const int row0 = h.start + kTileRows * k;
      const int c0 = slot * p.unit_cols;
      // the min() with rows - row0 and the output bound restate what a correct scan guarantees
      u.nrows = min(min(kTileRows, h.size - kTileRows * k), p.rows - row0);
      u.ncols = min(p.unit_cols, p.cols - c0);
      u.tile_cols = min(p.unit_cols, p.padded_cols - c0) >> 2;
      u.row_base = p.src + int64_t(row0) * p.ld + c0;
      u.dst = p.out + block * row_block_bytes + int64_t(c0) * kTileRows;
      if (u.nrows > 0 && u.ncols > 0 && (block + 1) * row_block_bytes <= p.out_bytes) u.kind = kData;
    } else {
      const int64_t nblocks = p.units / p.per_row;
      u.kind = kTail;
      u.lo = int64_t(h.first_unit) * row_block_bytes;
      u.hi = p.out_bytes;
      u.part = (block - h.first_unit) * p.per_row + slot;
      u.parts = int64_t(p.per_row) * (nblocks - h.first_unit);
    }
  } else {
    const GroupHit h = find_group<true>(p.offs, p.groups, p.cols, p.unit_cols, slot);
    const int64_t padded_rows = int64_t(((p.rows + kTileRows - 1) / kTileRows)) * kTileRows;
    if (h.group < p.groups) {
      const int chunk = slot - h.first_unit;
      const int padded_width = (h.size + 3) & ~3;
      const int c0 = h.start + chunk * p.unit_cols;
      u.nrows = min(kTileRows, p.rows - kTileRows * int(block));
      // the min() with cols - c0 and the output bound restate what a correct scan guarantees
      u.ncols = min(min(p.unit_cols, h.size - chunk * p.unit_cols), p.cols - c0);
      u.tile_cols = min(p.unit_cols, padded_width - chunk * p.unit_cols) >> 2;
      u.row_base = p.src + block * kTileRows * p.ld + c0;
      u.dst = p.out + padded_rows * h.padded_start + block * kTileRows * padded_width +
              int64_t(chunk) * p.unit_cols * kTileRows;
      if (u.nrows > 0 && u.ncols > 0 && padded_rows * (h.padded_start + padded_width) <= p.out_bytes)
        u.kind = kData;
    } else {
      // tail: round_up(rows,128) * (cols + 4G - padded total) zero bytes, a
      // 128 * (cols + 4G - padded total) slice per 128-row block
      const int64_t tail_cols = int64_t(p.cols) + 4 * int64_t(p.groups) - h.padded_start;
      u.kind = kTail;
      u.lo = padded_rows * h.padded_start + block * kTileRows * tail_cols;
      u.hi = u.lo + kTileRows * tail_cols;
      u.part = slot - h.first_unit;
      u.parts = p.per_row - h.first_unit;
    }
  }
  return u;
}

// ---------------------------------------------------------------------------
// producers: global -> registers -> LDS
// ---------------------------------------------------------------------------

// Buffer resource over [base, base + bytes) for raw (unswizzled) buffer loads.
// A load whose offset lies past `bytes` returns zeros and touches no memory.
// Base and size are the same for the whole workgroup; reading them from the
// first lane keeps the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_buffer(const uint8_t *base, uint32_t bytes) {
  // readfirstlane returns int: each half goes through uint32_t so that the low
  // half is not sign-extended into the high one
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))));
  void *ub = reinterpret_cast<void *>((hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, __builtin_amdgcn_readfirstlane(int(bytes)), kRawBufferFlags);
}

template <int POLICY>
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t offset) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(offset), 0, POLICY);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Per-row staging: row r's segment [a, a + seg) with a = row_base + r*ld is
// fetched as the 16-byte pieces covering it into LDS row r (pitch bytes); its
// first byte then sits at r*pitch + (a mod 16). Piece slot s = r*pieces + k
// goes to producer lane s mod NP; each lane issues exactly N loads back to back
// (N = slots per lane of this unit) before it waits for any of them.
template <int NP, int N, int POLICY>
__device__ __forceinline__ void stage_rows_n(uint8_t *__restrict__ buf, int t, __amdgpu_buffer_rsrc_t rsrc, uint32_t lead,
                                    int64_t ld, int nrows, int seg, int pitch, int pieces) {
  const int step_r = NP / pieces, step_k = NP % pieces;
  int r = t / pieces, k = t % pieces;
  uint4 v[N];
  uint32_t off[N];
#pragma unroll
  for (int it = 0; it < N; ++it) {
    const uint32_t row_off = lead + uint32_t(r) * uint32_t(ld);  // in range whenever r < nrows
    const int need = int(((row_off & 15) + seg + 15) >> 4);
    const bool valid = r < nrows && k < need;
    v[it] = load16<POLICY>(rsrc, valid ? (row_off & ~15u) + 16 * k : kOutOfRange);
    off[it] = valid ? uint32_t(r * pitch + 16 * k) : kOutOfRange;
    r += step_r;
    k += step_k;
    if (k >= pieces) { k -= pieces; ++r; }
  }
#pragma unroll
  for (int it = 0; it < N; ++it) {
    if (off[it] != kOutOfRange) {
      uint32_t *d = reinterpret_cast<uint32_t *>(buf + off[it]);  // 4-byte aligned rows
      d[0] = v[it].x;
      d[1] = v[it].y;
      d[2] = v[it].z;
      d[3] = v[it].w;
    }
  }
}

template <int NP, int ITERS, int POLICY>
__device__ __forceinline__ void stage_rows(uint8_t *__restrict__ buf, int t, const uint8_t *row_base, int64_t ld, int nrows,
                                  int seg, int pitch, int pieces) {
  static_assert(ITERS <= 8, "staging is unrolled for at most 8 pieces per lane");
  const uint32_t lead = uint32_t(reinterpret_cast<uintptr_t>(row_base) & 15);
  const uint8_t *base = row_base - lead;  // 16-byte aligned
  const uint32_t span = uint32_t((lead + int64_t(nrows - 1) * ld + seg + 15) & ~int64_t(15));
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(base, span);
  const int n = (nrows * pieces + NP - 1) / NP;  // uniform
  switch (n) {
    case 1: stage_rows_n<NP, 1, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
    case 2: stage_rows_n<NP, 2, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
    case 3: stage_rows_n<NP, 3, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
    case 4: stage_rows_n<NP, 4, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
    case 5: stage_rows_n<NP, 5, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
    case 6: stage_rows_n<NP, 6, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
    case 7: stage_rows_n<NP, 7, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
    default: stage_rows_n<NP, ITERS, POLICY>(buf, t, rsrc, lead, ld, nrows, seg, pitch, pieces); break;
  }
}

// Flat staging: the strip is one contiguous range [a, a + len); its 16-byte
// cover goes to LDS from offset 0, so byte a sits at LDS (a mod 16).
template <int NP, int N, int POLICY>
__device__ __forceinline__ void stage_flat_n(uint8_t *__restrict__ buf, int t, __amdgpu_buffer_rsrc_t rsrc, int n) {
  uint4 v[N];
#pragma unroll
  for (int it = 0; it < N; ++it) v[it] = load16<POLICY>(rsrc, t + it * NP < n ? uint32_t(16 * (t + it * NP)) : kOutOfRange);
#pragma unroll
  for (int it = 0; it < N; ++it)
    if (t + it * NP < n) *reinterpret_cast<uint4 *>(buf + 16 * (t + it * NP)) = v[it];
}

template <int NP, int ITERS, int POLICY>
__device__ __forceinline__ void stage_flat(uint8_t *__restrict__ buf, int t, const uint8_t *start, int len) {
  static_assert(ITERS <= 8, "staging is unrolled for at most 8 pieces per lane");
  const uint32_t lead = uint32_t(reinterpret_cast<uintptr_t>(start) & 15);
  const int n = int((lead + len + 15) >> 4);
  const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(start - lead, uint32_t(16 * n));
  switch ((n + NP - 1) / NP) {  // uniform
    case 1: stage_flat_n<NP, 1, POLICY>(buf, t, rsrc, n); break;
    case 2: stage_flat_n<NP, 2, POLICY>(buf, t, rsrc, n); break;
    case 3: stage_flat_n<NP, 3, POLICY>(buf, t, rsrc, n); break;
    case 4: stage_flat_n<NP, 4, POLICY>(buf, t, rsrc, n); break;
    case 5: stage_flat_n<NP, 5, POLICY>(buf, t, rsrc, n); break;
    case 6: stage_flat_n<NP, 6, POLICY>(buf, t, rsrc, n); break;
    case 7: stage_flat_n<NP, 7, POLICY>(buf, t, rsrc, n); break;
    default: stage_flat_n<NP, ITERS, POLICY>(buf, t, rsrc, n); break;
  }
}

// Resolves unit vb, publishes its descriptor and stages its bytes in buf.
template <int MODE>
__device__ __forceinline__ void produce(uint8_t *__restrict__ buf, const Params &p, int64_t vb) {
  constexpr int NP = producers_for(MODE);
  constexpr int ITERS = load_iters_for(MODE);
  const Unit u = resolve<MODE == kModeKRows>(p, vb);
  const int t = threadIdx.x;
  if (t == 0) {
    UnitDesc d;
    d.kind = u.kind;
    d.nrows = u.nrows;
    d.ncols = u.ncols;
    d.tile_cols = u.tile_cols;
    d.src_lo = uint32_t(reinterpret_cast<uintptr_t>(u.row_base));
    d.unused = 0;
    d.dst = reinterpret_cast<uint64_t>(u.dst);
    d.lo = u.lo;
    d.hi = u.hi;
    d.part = u.part;
    d.parts = u.parts;
    *reinterpret_cast<UnitDesc *>(buf) = d;
  }
  if (u.kind != kData) return;
  uint8_t *data = buf + kHeaderBytes;
  if (MODE == kModeMFlat)
    stage_flat<NP, ITERS, kFlatLoadPolicy>(data, t, u.row_base, u.nrows * u.ncols);
  else
    stage_rows<NP, ITERS, kRowsLoadPolicy>(data, t, u.row_base, p.ld, u.nrows, u.ncols, p.pitch, p.pieces);
}

// ---------------------------------------------------------------------------
// consumers: LDS -> global
// ---------------------------------------------------------------------------

// 16-byte store, streamed past the caches: the output is never read back here.
__device__ __forceinline__ void store16(uint8_t *dst, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = {a, b, c, d};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(dst));
}

// Zero-fill of part `part` of `parts` of the byte range [lo, hi); lo is
// 16-byte aligned and hi a multiple of 4. t: consumer thread index.
template <int NC>
__device__ __forceinline__ void zero_part(uint8_t *__restrict__ out, int t, int64_t lo, int64_t hi, int64_t part,
                                 int64_t parts) {
  if (lo >= hi || parts <= 0) return;
  const int64_t len16 = (hi - lo + 15) >> 4;
  const int64_t per = (len16 + parts - 1) / parts;
  const int64_t b = lo + 16 * min(per * part, len16);
  const int64_t e = min(lo + 16 * min(per * (part + 1), len16), hi);
  const int64_t full = b + ((e - b) & ~int64_t(15));
  for (int64_t q = b + 16 * t; q < full; q += 16 * NC) store16(out + q, 0, 0, 0, 0);
  for (int64_t q = full + 4 * t; q < e; q += 4 * NC) *reinterpret_cast<uint32_t *>(out + q) = 0u;
}

// Writes `tile_cols` tiles (128 rows x 4 columns each) contiguously at dst.
// Row r, column c of the unit is LDS byte row_off(r) + c with
// row_off(r) = first + r*row_step (FLAT) or r*row_step + (addr + r*ld) mod 16.
// Rows >= nrows and columns >= ncols are written as zero. Consumer thread t
// writes 16-byte units t, t + NC, ...
template <int NC, int ITERS, bool FLAT, bool ALIGNED>
__device__ __forceinline__ void emit_tiles(const uint8_t *__restrict__ buf, int t, uint8_t *__restrict__ dst,
                                  int tile_cols, int nrows, int ncols, int first, int row_step, uintptr_t addr,
                                  int64_t ld) {
  const uint32_t *w32 = reinterpret_cast<const uint32_t *>(buf);
  const int n16 = tile_cols * 32;
#pragma unroll 2
  for (int it = 0; it < ITERS; ++it) {
    const int v = t + it * NC;
    if (it * NC < n16 && v < n16) {
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
          int b = r * row_step + 4 * tc;
          if (FLAT)
            b += first;
          else
            b += int((addr + uintptr_t(int64_t(r) * ld)) & 15);
          if (ALIGNED) {
            x = w32[b >> 2];
          } else {
            x = __builtin_amdgcn_alignbyte(w32[(b >> 2) + 1], w32[b >> 2], b & 3);
          }
          x &= mask;
        }
        w[q] = x;
      }
      store16(dst + 16 * int64_t(v), w[0], w[1], w[2], w[3]);
    }
  }
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(x)))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(x) >> 32))));
  return int64_t((hi << 32) | lo);
}

// Writes out the unit whose descriptor heads buf.
template <int MODE>
__device__ __forceinline__ void consume(const uint8_t *__restrict__ buf, const Params &p) {
  constexpr int NC = consumers_for(MODE);
  constexpr int ITERS = store_iters_for(MODE);
  constexpr bool FLAT = MODE == kModeMFlat;
  const int t = threadIdx.x - producers_for(MODE);
  const UnitDesc &d = *reinterpret_cast<const UnitDesc *>(buf);
  const int kind = uniform(d.kind);
  if (kind == kTail) {
    zero_part<NC>(p.out, t, uniform64(d.lo), uniform64(d.hi), uniform64(d.part), uniform64(d.parts));
    return;
  }
  if (kind != kData) return;
  const int nrows = uniform(d.nrows), ncols = uniform(d.ncols), tile_cols = uniform(d.tile_cols);
  const uint32_t a = uint32_t(uniform(int(d.src_lo)));
  uint8_t *dst = reinterpret_cast<uint8_t *>(uniform64(int64_t(d.dst)));
  const uint8_t *data = buf + kHeaderBytes;
  const bool aligned = FLAT ? ((a & 3) == 0 && (ncols & 3) == 0) : ((a & 3) == 0 && (p.ld & 3) == 0);
  const int first = FLAT ? int(a & 15) : 0;
  const int step = FLAT ? ncols : p.pitch;
  if (aligned)
    emit_tiles<NC, ITERS, FLAT, true>(data, t, dst, tile_cols, nrows, ncols, first, step, a, p.ld);
  else
    emit_tiles<NC, ITERS, FLAT, false>(data, t, dst, tile_cols, nrows, ncols, first, step, a, p.ld);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Workgroup b handles virtual blocks b, b + grid, b + 2*grid, ... Producers
// stage unit n+1 into one LDS buffer while consumers write unit n out of the
// other; one barrier per unit hands the buffers over. Both roles resolve the
// same units, so they run the same number of iterations and barriers.
template <int MODE>
__global__ __launch_bounds__(threads_for(MODE)) __attribute__((amdgpu_waves_per_eu(kMinWavesPerEu)))
void rearrange_kernel(Params p) {
  extern __shared__ __align__(16) uint8_t lds[];
  const bool producer = threadIdx.x < producers_for(MODE);  // whole waves
  int64_t vb = blockIdx.x;
  int b = 0;
  if (producer) produce<MODE>(lds, p, vb);
  for (;;) {
    __syncthreads();  // buffer b holds unit vb; nothing reads buffer b ^ 1 any more
    const int64_t vb_next = vb + gridDim.x;
    if (producer) {
      if (vb_next < p.vunits) produce<MODE>(lds + (b ^ 1) * p.lds_stride, p, vb_next);
    } else {
      consume<MODE>(lds + b * p.lds_stride, p);
    }
    if (vb_next >= p.vunits) break;
    vb = vb_next;
    b ^= 1;
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Workgroups of `fn` that fit on the current device at once (0 if unknown).
int64_t resident_workgroups(const void *fn, int threads, size_t lds_bytes) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds_bytes) != hipSuccess) return 0;
  return int64_t(cus) * per_cu;
}

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
      mode = kModeMRows;
      int uc = std::min<int>(kMaxUnitCols, p.padded_cols);
      while (uc > kMinUnitCols && blocks * ((p.padded_cols + uc - 1) / uc) < kTargetUnits)
        uc = std::max<int>(kMinUnitCols, int(round_up(uc / 2, 4)));
      p.unit_cols = uc;
    }
    p.per_row = (p.padded_cols + p.unit_cols - 1) / p.unit_cols;
    units = blocks * p.per_row;
  } else {
    mode = kModeKRows;
    p.unit_cols = kMaxUnitCols;
    // units per 128-row block: every group's chunks plus at least one of tail
    p.per_row = int((cols + 4 * int64_t(groups) + p.unit_cols - 1) / p.unit_cols + groups);
    units = ((rows + kTileRows - 1) / kTileRows) * p.per_row;
  }
  const int64_t seg = std::min<int64_t>(cols, p.unit_cols);   // widest row segment of a unit
  p.pieces = std::max<int>(1, int((seg + 30) / 16));
  p.pitch = 16 * p.pieces + 4;
  p.units = units;
  p.vunits = round_up(units, 8);
  size_t stride = kHeaderBytes + (mode == kModeMFlat ? size_t(kTileRows) * size_t(cols) + 32 + kLdsSlack
                                                    : size_t(kTileRows) * size_t(p.pitch) + kLdsSlack);
  stride = (stride + 15) & ~size_t(15);
  p.lds_stride = int(stride);
  size_t lds_bytes = 2 * stride;

  const void *fn = mode == kModeMFlat   ? reinterpret_cast<const void *>(&rearrange_kernel<kModeMFlat>)
                   : mode == kModeMRows ? reinterpret_cast<const void *>(&rearrange_kernel<kModeMRows>)
                                        : reinterpret_cast<const void *>(&rearrange_kernel<kModeKRows>);
  const int threads = mode == kModeMFlat ? threads_for(kModeMFlat) : threads_for(kModeMRows);
  // as many workgroups as can be resident at once (a multiple of 8, so that a
  // workgroup's units all map to its own XCD), each looping over its units;
  // when every workgroup gets a single unit, one LDS buffer is enough
  int64_t grid = std::min<int64_t>(p.vunits, kMaxGrid);
  if (kPersistent) {
    const int64_t resident = resident_workgroups(fn, threads, lds_bytes);
    if (resident >= 8) grid = std::min<int64_t>(grid, resident / 8 * 8);
  }
  if (grid >= p.vunits) lds_bytes = stride;

  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(threads), args, lds_bytes, stream);
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
    case MX_REARRANGE_ESHAPE: return "invalid shape: rows/cols negative or too large, or row_stride outside [cols, 2^24]";
    case MX_REARRANGE_EGROUPS: return "num_groups must be >= 1";
    case MX_REARRANGE_EALIGN: return "out must be 16-byte aligned";
    case MX_REARRANGE_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
