// MXFP8 quantisation along rows (dim0 cast) for gfx950 (MI355X), with the E8M0
// scales written straight into the grouped, blocked 128x4-tile layout.
//
// Pages: "[mxfp8 moe training] use dim1 cast cuda kernel for 3d weights by
// reshaping to 2d" (first notes and Benchmarks tables: bf16 activations A of
// shape (16640, 5120) cast to MXFP8 with blocks of 32 before the grouped GEMM);
// "[mxfp8 moe training] compute prefix sum of group sizes inside kernel intead
// of precomputing" (Context, Changes: the blocked scale layout of token groups,
// each group's rows padded to 128, group starts as an in-kernel prefix sum).
// The pages do not state the numerics; the rule implemented is the OCP
// Microscaling (MX) v1.0 one for MXFP8 with E4M3 elements:
//   scale of a 32-element block = 2^s, s = floor(log2(amax)) - 8, clamped to
//   [-127, 127], stored as the E8M0 byte s + 127 (0 for an all-zero block);
//   element code = nearest E4M3 (finite variant) to x / 2^s, ties to even,
//   saturated at +-448; a block holding a NaN or an infinity gets the byte 0xFF
//   and the E4M3 NaN code 0x7F for all its elements.
//
// The work is HBM-bound streaming (2 bytes read, 1 byte written per element plus
// 1/32 byte of scale). Design:
//   * A work unit is 512 consecutive elements of one row (1 KB of bf16); one
//     wave handles kUnroll consecutive units (row-major), issuing all their
//     16-byte buffer loads before the first wait. Lane l holds elements
//     8l..8l+7 of a unit, so four lanes hold one 32-element block.
//   * Block maximum: integer maximum of the binary32 magnitude bits (bf16 widened
//     by a shift; NaN and infinity compare above every finite value), reduced
//     over the four lanes with two DPP quad permutations.
//   * Scale: the exponent comes from the bits of the maximum (count of leading
//     zeros for subnormal maxima); x * 2^-s is a multiplication by a normal
//     power of two, exact wherever the result matters; the hardware conversion
//     v_cvt_pk_fp8_f32 (round to nearest even) packs two codes at a time after a
//     clamp to +-448.
//   * Codes: lanes store 8 bytes each, a wave 512 contiguous bytes (non-temporal).
//   * Scales: a 16-lane DPP row holds the four blocks of one tile column of its
//     row; an OR over the row assembles the 4-byte tile word, which one lane
//     stores at the row's place in its group's padded blocked matrix. The row's
//     group and the group's padded start come from the end offsets (clamped,
//     prefix maximum, padded prefix sums), scanned by every wave into two
//     registers when G <= 64, else once per workgroup into LDS.
//   * Padding rows of each group's last row block and the tail of the scale
//     allocation are written with zeros by extra workgroups of the same launch,
//     one per output row block, so the scale output needs no memset.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "group_table.h"
#include "launch_order.h"
#include "mx_quantize.h"
#include "mx_rearrange.h"
#include "write_ranges.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / kWave;
constexpr int kUnitElems = 512;       // elements per wave-unit: 16 blocks, 4 tile columns of scales
constexpr int kUnroll = 4;            // units per wave, loads issued back to back (swept: 2..16)
constexpr int kDim0DealWgs = 48;      // workgroups per run of the interleaved XCD order (dim0 cast)
constexpr int kDim1DealUnits = 64;    // workgroups per run of the interleaved XCD order (2-D dim1 cast)
constexpr int kMaxGroups = 4096;      // LDS holds two int arrays of this many groups
constexpr int64_t kMaxRowStride = int64_t(1) << 26;   // elements; keeps unit offsets in 32 bits
constexpr int kStreamPolicy = 2;      // buffer load bit 1: non-temporal
constexpr uint32_t kE4m3Nan = 0x7f7f7f7fu;

struct QParams {
  const uint16_t *x;
  const int32_t *offs;
  uint8_t *q;
  uint8_t *scales;
  int64_t ld;            // row stride of x in elements
  int64_t units;         // rows * chunks
  int64_t data_groups;   // workgroups that quantise
  int64_t pad_blocks;    // output row blocks handled by the zero-fill workgroups
  int64_t scale_bytes;   // whole blocked-scale allocation
  int rows;
  int K;
  int chunks;            // units per row
  int groups;
  int tile_cols;         // round_up(K/32, 4) / 4
  int64_t data_slots;    // workgroup slots of the quantising workgroups (a multiple of 8 covering them)
  int64_t deal;          // interleaved order: consecutive workgroups dealt to one XCD at a time
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t mag_lo(uint32_t w) { return (w << 16) & 0x7fffffffu; }
__device__ __forceinline__ uint32_t mag_hi(uint32_t w) { return w & 0x7fff0000u; }

__device__ __forceinline__ float clamp448(float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); }

// Four E4M3 codes of y0..y3 (already clamped), first element in the low byte.
__device__ __forceinline__ uint32_t e4m3x4(float y0, float y1, float y2, float y3) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, p, true);
  return uint32_t(p);
}

__device__ __forceinline__ void store8_nt(uint8_t *dst, uint32_t a, uint32_t b) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 t = {a, b};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2 *>(dst));
}

// Byte offset of scale row R, tile column tc inside the blocked matrix of tile_cols tile columns.
__host__ __device__ inline int64_t scale_word_offset(int64_t R, int tc, int tile_cols) {
  const int64_t tile = (R / kTileRows) * tile_cols + tc;
  const int r = int(R % kTileRows);
  return tile * 512 + (r % 32) * 16 + (r / 32) * 4;
}

// One wave's loads: the 16-byte piece of each of kUnroll consecutive units
// starting at unit u0, out of range (zeros, no memory access) past a row's end
// or past the last unit.
__device__ __forceinline__ void load_units(const QParams &p, int64_t u0, uint4 (&v)[kUnroll]) {
  const int lane = threadIdx.x & (kWave - 1);
  {
    int64_t r = u0 / p.chunks;
    int c = int(u0 - r * p.chunks);
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const bool valid = u0 + i < p.units;
      const int elems = valid ? min(kUnitElems, p.K - c * kUnitElems) : 0;
      const uint16_t *base = p.x + (valid ? r * p.ld + int64_t(c) * kUnitElems : 0);
      const __amdgpu_buffer_rsrc_t rsrc = byte_buffer(base, uint32_t(2 * elems));
      const uint32_t off = 16 * lane < 2 * elems ? uint32_t(16 * lane) : kOutOfRange;
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(off), 0, kStreamPolicy);
      v[i] = make_uint4(t[0], t[1], t[2], t[3]);
      if (++c == p.chunks) {
        c = 0;
        ++r;
      }
    }
  }
}

// One wave: quantises the kUnroll units loaded by load_units.
template <class GROUPS>
__device__ __forceinline__ void quantize_units(const QParams &p, int64_t u0, const uint4 (&v)[kUnroll],
                                               const GROUPS &grp) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t r = u0 / p.chunks;
  int c = int(u0 - r * p.chunks);
  int64_t looked_up = -1;
  int64_t scale_row = -1;   // row of r inside the blocked scales, -1 when r is in no group
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    if (u0 + i < p.units) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max(m, max(mag_lo(w[k]), mag_hi(w[k])));
      m = max(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0xb1, 0xf, 0xf, false)));  // quad_perm [1,0,3,2]
      m = max(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0x4e, 0xf, 0xf, false)));  // quad_perm [2,3,0,1]
      const bool finite = m < 0x7f800000u;
      int e;   // floor(log2(amax)), amax > 0
      if (m >= 0x00800000u)
        e = int(m >> 23) - 127;
      else
        e = 31 - __builtin_clz(m | 1u) - 149;   // subnormal maximum (m = 0 handled by the clamp below)
      int s = min(max(e - 8, -127), 127);
      if (m == 0) s = -127;
      const float f = __uint_as_float(uint32_t(127 - s) << 23);   // 2^-s, a normal binary32 for s <= 119
      uint32_t c0 = e4m3x4(clamp448(bf16_lo(w[0]) * f), clamp448(bf16_hi(w[0]) * f), clamp448(bf16_lo(w[1]) * f),
                           clamp448(bf16_hi(w[1]) * f));
      uint32_t c1 = e4m3x4(clamp448(bf16_lo(w[2]) * f), clamp448(bf16_hi(w[2]) * f), clamp448(bf16_lo(w[3]) * f),
                           clamp448(bf16_hi(w[3]) * f));
      uint32_t byte = uint32_t(s + 127);
      if (!finite) {
        c0 = c1 = kE4m3Nan;
        byte = 0xffu;
      }
      const int col = c * kUnitElems + 8 * lane;
      if (col < p.K) store8_nt(p.q + r * p.K + col, c0, c1);

      // tile word of this row: lanes 16j..16j+15 hold blocks 4j..4j+3 of the unit
      int word = (lane & 3) == 0 ? int(byte << (8 * ((lane >> 2) & 3))) : 0;
      word |= dpp<0x114>(word);   // row_shr:4
      word |= dpp<0x118>(word);   // row_shr:8
      if (r != looked_up) {
        looked_up = r;
        scale_row = dim0_scale_row(grp, p.groups, r);
      }
      const int tc = 4 * c + (lane >> 4);
      if ((lane & 15) == 12 && scale_row >= 0 && tc < p.tile_cols) {
        const int64_t off = scale_word_offset(scale_row, tc, p.tile_cols);
        if (fits(off, 4, p.scale_bytes)) *reinterpret_cast<uint32_t *>(p.scales + off) = uint32_t(word);
      }
    }
    if (++c == p.chunks) {
      c = 0;
      ++r;
    }
  }
}

// Row of input row r inside the blocked scales (its group's padded start plus
// its place in the group), or -1 when r lies in no group. count_ends_le(key):
// groups whose clamped end is <= key; end(g), pend_at(g): clamped cumulative
// end and padded cumulative end of group g.
template <class TABLE>
__host__ __device__ inline int64_t dim0_scale_row(const TABLE &grp, int groups, int64_t r) {
  const int g = grp.count_ends_le(r);
  if (g < 0 || g >= groups) return -1;
  const int start = g ? grp.end(g - 1) : 0;
  const int pstart = g ? grp.pend_at(g - 1) : 0;
  return int64_t(pstart) + (r - start);
}

// Zero-fill of output row block ob of the blocked scales: the padding rows
// [valid, 128) of the group the block belongs to, or (past the last group)
// the byte range `tail` of the block. Both stay inside the scale allocation:
// valid is clamped into [0, 128], every padding-row word is checked with
// fits(), and the tail is clamped by zero_share.
struct Dim0ZeroBlock {
  bool in_group;
  int valid;
  ZeroSpan tail;
};

template <class TABLE>
__host__ __device__ inline Dim0ZeroBlock dim0_zero_block(const QParams &p, const TABLE &grp, int64_t ob) {
  Dim0ZeroBlock z = {false, kTileRows, {0, 0, 0}};
  const int64_t block_bytes = int64_t(kTileRows) * p.tile_cols * 4;
  const int g = grp.count_pends_le(ob * kTileRows);
  if (g < p.groups) {
    const int start = g ? grp.end(g - 1) : 0;
    const int pstart = g ? grp.pend_at(g - 1) : 0;
    const int size = grp.end(g) - start;
    const int64_t k = ob - pstart / kTileRows;
    z.in_group = true;
    z.valid = int(clamp64(int64_t(size) - kTileRows * k, 0, kTileRows));
  } else {
    const int64_t lo = ob * block_bytes > int64_t(grp.pend_at(p.groups - 1)) * p.tile_cols * 4
                           ? ob * block_bytes
                           : int64_t(grp.pend_at(p.groups - 1)) * p.tile_cols * 4;
    z.tail = zero_share(lo, (ob + 1) * block_bytes, p.scale_bytes, 0, 1);
  }
  return z;
}

template <class GROUPS>
__device__ __forceinline__ void zero_block(const QParams &p, int64_t ob, const GROUPS &grp) {
  const Dim0ZeroBlock z = dim0_zero_block(p, grp, ob);
  if (z.in_group) {
    const int n = (kTileRows - z.valid) * p.tile_cols;
    for (int t = threadIdx.x; t < n; t += kThreads) {
      const int rr = z.valid + t / p.tile_cols;
      const int tc = t % p.tile_cols;
      const int64_t off = scale_word_offset(ob * kTileRows + rr, tc, p.tile_cols);
      if (fits(off, 4, p.scale_bytes)) *reinterpret_cast<uint32_t *>(p.scales + off) = 0u;
    }
  } else {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int64_t a = z.tail.begin + 16 * threadIdx.x; a < z.tail.full; a += 16 * kThreads)
      *reinterpret_cast<u32x4 *>(p.scales + a) = zero;
    for (int64_t a = z.tail.full + 4 * threadIdx.x; a < z.tail.end; a += 4 * kThreads)
      *reinterpret_cast<uint32_t *>(p.scales + a) = 0u;
  }
}

// Shape, units and grid of the dim0 cast (sizes validated by the caller);
// returns the grid: the quantising workgroups, then one zero-fill workgroup
// per output row block.
int64_t dim0_geometry(QParams &p, int64_t rows, int64_t K, int32_t num_groups) {
  p.rows = int(rows);
  p.K = int(K);
  p.chunks = int((K + kUnitElems - 1) / kUnitElems);
  p.groups = num_groups;
  p.tile_cols = int((K / 32 + 3) / 4);
  p.units = rows * p.chunks;
  p.scale_bytes = mx_quantize_dim0_M_groups_scale_bytes(rows, K, num_groups);
  const int64_t waves = (p.units + kUnroll - 1) / kUnroll;
  p.data_groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  p.pad_blocks = (rows + kTileRows - 1) / kTileRows + num_groups;
  return p.data_groups + p.pad_blocks;
}

template <bool SMALL, bool IL>
__global__ __launch_bounds__(kThreads) void quantize_dim0_kernel(QParams p) {
  extern __shared__ __align__(16) int lds_groups[];
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  MGroups<SMALL> grp;
  if (int64_t(blockIdx.x) < p.data_slots) {
    // Workgroup b runs on XCD b mod 8. Each XCD takes a contiguous range of
    // units, or, for grids of more than one pass, runs of p.deal workgroups in
    // turn (launch_order.h). Slots past the last workgroup quantise nothing.
    const int64_t b = unit_of_slot<IL>(blockIdx.x, p.data_slots, p.deal);
    // the data loads go out first; the group scan overlaps them
    const int64_t u0 = (b * kWavesPerGroup + wave) * kUnroll;
    uint4 v[kUnroll];
    load_units(p, u0, v);
    grp.init(p.offs, p.groups, p.rows, lds_groups);
    if (u0 < p.units) quantize_units(p, u0, v, grp);
  } else {
    grp.init(p.offs, p.groups, p.rows, lds_groups);
    const int64_t ob = int64_t(blockIdx.x) - p.data_slots;
    if (ob < p.pad_blocks) zero_block(p, ob, grp);
  }
}


// ===========================================================================
// dim1 cast: blocks of 32 tokens per feature column, codes written transposed,
// scales placed in the K-groups blocked layout (each token group's scale
// columns are its own blocked matrix of round_up(N,128) x round_up(w_g,4)).
//
// A unit is one tile of output scales: 128 features x one 4-column tile column
// of one group, i.e. up to 128 tokens of that group (4 blocks) x 128 features.
// Its input is a 128 x 128 bf16 tile of x (token rows of 256 bytes), staged in
// LDS; each thread then reads two feature columns of one 32-token block (one
// dword per token: features 2p and 2p+1), quantises both, writes 32 code bytes
// into each of the two transposed rows (four lanes write 128 contiguous bytes
// of a row) and contributes its two scale bytes to the tile words, which a
// quad assembles with DPP and stores: the unit writes its whole 512-byte tile,
// padding included. Tokens after the last group are quantised by extra units
// that place no scales; spare units zero the tail of the scale allocation.
// Within a feature block the token chunks vary fastest and the code rows are
// written with ordinary (write-back) stores, so units running together fill
// each other's partial 128-byte lines in L2; feature-block-first order and
// non-temporal stores each cost about a third more time (measured).
// ===========================================================================

constexpr int kTileTok = 128;                 // tokens per unit (4 blocks)
constexpr int kTileFeat = 128;                // features per unit
constexpr int kMaxGroupsDim1 = 2048;          // LDS: the staged tile plus 3 ints per group
constexpr int64_t kMaxRowStrideDim1 = int64_t(1) << 23;   // 128 rows of a unit stay in 32-bit offsets
// LDS dword offset of token row t of the staged tile: rows 68 dwords apart
// (64 of data, 4 of skew) plus 16 more per 32-row block, so that the 64 lanes
// reading one dword of 16 column pairs in 4 blocks hit 64 distinct banks.
__device__ __forceinline__ int tile_row(int t) { return 68 * t + 16 * (t >> 5); }
constexpr int kTileDwords = 68 * (kTileTok - 1) + 16 * ((kTileTok - 1) >> 5) + 64;

struct Q1Params {
  const uint16_t *x;
  const int32_t *offs;   // token group ends (unused when group_tokens > 0)
  uint8_t *qT;
  uint8_t *scales;
  int64_t ld;            // row stride of x in elements
  int64_t T;             // tokens (multiple of 32)
  int64_t q_ld;          // row stride of the codes: T, or group_tokens for per-group code matrices
  int64_t x_gstride;     // per-group inputs: elements between groups' first rows
  int64_t q_gstride;     // per-group codes: bytes between groups' code matrices
  int group_tokens;      // > 0: every group holds exactly this many tokens (stacked expert weights),
                         // each with its own input matrix and its own N x group_tokens code matrix
  int diagonal;          // unit order: 0 token chunks fastest, 1 diagonal over feature blocks
                         // (with two feature blocks per workgroup, quantize_dim1_kernel<., true>)
  int64_t padded_rows;   // round_up(N, 128)
  int64_t scale_bytes;   // padded_rows * (T/32 + 4G)
  int64_t units;         // chunk_units * nb
  int64_t wg_units;      // workgroups: chunk_units * nbw
  int64_t deal;          // > 0: runs of this many workgroups dealt to the XCDs in turn; 0: contiguous ranges
  int64_t slots;         // workgroups launched: wg_units, or more for runs (the extra ones do nothing)
  int N;
  int nb;                // feature blocks of 128
  int nbw;               // feature-block groups of one workgroup each (nb, or ceil(nb/2) in pairs)
  int groups;
};

// Scan of one 64-group slice: e = clamped cumulative end in scale columns,
// cch = cumulative tile columns (chunks), cw = cumulative padded widths.
__device__ __forceinline__ void scan_slice_dim1(const Q1Params &p, int base, int carry_e, int carry_ch, int carry_w,
                                                int &e, int &cch, int &cw) {
  const int g = base + int(threadIdx.x & (kWave - 1));
  int64_t et = 0;
  if (p.group_tokens > 0)
    et = g < p.groups ? int64_t(g + 1) * p.group_tokens : 0;
  else if (g < p.groups)
    et = p.offs[g];
  et = min(max(et, int64_t(0)), p.T);
  e = max(wave_inclusive_max(int(et / 32)), carry_e);
  const int prev = wave_shift_up(e, carry_e);
  const int w = g < p.groups ? e - prev : 0;
  const int W = (w + 3) & ~3;
  cch = wave_inclusive_sum(W / 4) + carry_ch;
  cw = wave_inclusive_sum(W) + carry_w;
}

template <bool SMALL>
struct Groups1;

template <>
struct Groups1<true> {
  int groups, e, cch, cw;
  __device__ __forceinline__ void init(const Q1Params &p, int *) {
    groups = p.groups;
    scan_slice_dim1(p, 0, 0, 0, 0, e, cch, cw);
  }
  __device__ __forceinline__ int count_cch_le(int64_t key) const {
    return __popcll(__ballot(int(threadIdx.x & (kWave - 1)) < groups && int64_t(cch) <= key));
  }
  __device__ __forceinline__ int end(int g) const { return __builtin_amdgcn_readlane(e, g); }
  __device__ __forceinline__ int chunks_through(int g) const { return __builtin_amdgcn_readlane(cch, g); }
  __device__ __forceinline__ int width_through(int g) const { return __builtin_amdgcn_readlane(cw, g); }
};

template <>
struct Groups1<false> {
  int groups;
  const int *es, *cchs, *cws;
  __device__ __forceinline__ void init(const Q1Params &p, int *lds) {
    groups = p.groups;
    int *e_out = lds, *ch_out = lds + p.groups, *w_out = lds + 2 * p.groups;
    if (threadIdx.x < kWave) {
      int ce = 0, cc = 0, cwd = 0;
      for (int base = 0; base < p.groups; base += kWave) {
        int e, cch, cw;
        scan_slice_dim1(p, base, ce, cc, cwd, e, cch, cw);
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

// What one unit of the dim1 cast reads and writes, decoded from its tile
// column ci and feature block fb and the scanned group table (end(g): clamped
// cumulative end in scale columns; chunks_through(g), width_through(g):
// cumulative tile columns and padded widths; count_cch_le(key): groups whose
// cumulative tile columns are <= key). Token runs are clamped into their token
// range and the scale tile into the scale allocation (write_ranges.h), so a
// wrong table can give a wrong output but no access outside the buffers.
struct Dim1Unit {
  int64_t t0;         // first token of the unit (over all tokens)
  int ntok;           // tokens of the unit: a multiple of 32, <= 128
  int64_t x_row0;     // element offset of the unit's first input row
  int64_t q_col0;     // byte offset of the unit's first code in code row 0
  int64_t tile_off;   // byte offset of the unit's 512-byte scale tile, -1: no scales
  bool spare;         // a unit past the data: zero its share of the scale tail
  ZeroSpan zero;      // that share
};

template <class TABLE>
__host__ __device__ inline Dim1Unit dim1_unit(const Q1Params &p, const TABLE &grp, int64_t ci, int fb) {
  Dim1Unit un = {0, 0, 0, 0, -1, false, {0, 0, 0}};
  const int total_chunks = grp.chunks_through(p.groups - 1);
  const int last_end = grp.end(p.groups - 1);   // scale columns covered by groups
  const int64_t cols = p.T / 32;
  if (ci < total_chunks) {
    const int g = int(clamp64(grp.count_cch_le(ci), 0, p.groups - 1));
    const int first_chunk = g ? grp.chunks_through(g - 1) : 0;
    const int64_t k = ci - first_chunk;
    const int S = g ? grp.end(g - 1) : 0;
    const int w = grp.end(g) - S;
    const int C = g ? grp.width_through(g - 1) : 0;
    const int W = (w + 3) & ~3;
    const int64_t t0 = 32 * (int64_t(S) + 4 * k);
    const int64_t n = 32 * (int64_t(w) - 4 * k < 4 ? int64_t(w) - 4 * k : int64_t(4));
    un.tile_off = p.padded_rows * C + (int64_t(fb) * (W / 4) + k) * 512;
    if (!fits(un.tile_off, 512, p.scale_bytes)) un.tile_off = -1;
    if (p.group_tokens > 0) {   // group g's own input and code matrices
      const Run tl = clamp_run(t0 - int64_t(g) * p.group_tokens, n, p.group_tokens);
      un.t0 = int64_t(g) * p.group_tokens + tl.first;
      un.ntok = int(tl.n);
      un.x_row0 = int64_t(g) * p.x_gstride + tl.first * p.ld;
      un.q_col0 = int64_t(g) * p.q_gstride + tl.first;
    } else {
      const Run t = clamp_run(t0, n, p.T);
      un.t0 = t.first;
      un.ntok = int(t.n);
      un.x_row0 = t.first * p.ld;
      un.q_col0 = t.first;
    }
  } else {
    // chunks of tokens after the last group (none with group_tokens > 0: the groups cover every token)
    const int64_t trailing = p.group_tokens > 0 ? 0 : (cols - last_end + 3) / 4;
    const int64_t c2 = ci - total_chunks;
    if (c2 < trailing) {
      const int64_t left = cols - last_end - 4 * c2;
      const Run t = clamp_run(32 * (last_end + 4 * c2), 32 * (left < 4 ? left : 4), p.T);
      un.t0 = t.first;
      un.ntok = int(t.n);
      un.x_row0 = t.first * p.ld;
      un.q_col0 = t.first;
    } else {
      // spare unit: a share of the zero tail of the scale allocation
      un.spare = true;
      const int64_t spare = (p.units / p.nb - total_chunks - trailing) * p.nb;
      const int64_t part = (c2 - trailing) * p.nb + fb;
      un.zero = zero_share(p.padded_rows * grp.width_through(p.groups - 1), p.scale_bytes, p.scale_bytes, part, spare);
    }
  }
  return un;
}

// 8 bf16 of a staged piece with the features at or past N zeroed (f0 = feature of the first).
__device__ __forceinline__ uint4 mask_features(uint4 v, int f0, int N) {
  const int valid = N - f0;
  if (valid >= 8) return v;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t keep = (2 * k + 1 < valid ? 0xffff0000u : 0u) | (2 * k < valid ? 0x0000ffffu : 0u);
    w[k] &= keep;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// E8M0 byte and the factor 2^-s of a block whose largest magnitude has binary32 bits m (finite).
__device__ __forceinline__ int scale_exponent(uint32_t m) {
  int e;
  if (m >= 0x00800000u)
    e = int(m >> 23) - 127;
  else
    e = 31 - __builtin_clz(m | 1u) - 149;
  int s = min(max(e - 8, -127), 127);
  if (m == 0) s = -127;
  return s;
}

// Feature blocks per workgroup: two with the diagonal order, else one.
__host__ __device__ inline int dim1_blocks(const Q1Params &p) { return p.diagonal ? 2 : 1; }

// The unit (tile column ci, feature block fb) of half `half` of workgroup b,
// with `blocks` feature blocks per workgroup. Workgroups form contiguous
// ranges per XCD (workgroup b runs on XCD b mod 8), or, with p.deal > 0, runs
// of p.deal workgroups dealt to the XCDs in turn. Token chunks vary fastest:
// units that run together write neighbouring pieces of the same transposed
// code rows, which meet in L2 as whole lines. When every unit writes whole
// lines (per-group codes, groups of a multiple of 128 tokens) the diagonal
// order instead spreads the units that run together over feature blocks, so
// their reads of the token rows do not all fall on the same column slice (4%
// faster at token rows 16 KB apart). live is false for the idle half of a
// last, single block and for slots past the workgroups. A host test checks
// that every unit gets exactly one slot.
struct Dim1Slot {
  int64_t ci;
  int fb;
  bool live;
};
__host__ __device__ inline Dim1Slot dim1_slot(const Q1Params &p, int64_t b, int blocks, int half) {
  int64_t u;
  if (p.deal > 0) {
    u = unit_of_slot<true>(b, p.slots, p.deal);
  } else {
    const int64_t n8 = p.wg_units / 8 * 8;
    u = b < n8 ? (b & 7) * (n8 >> 3) + (b >> 3) : b;
  }
  const int64_t chunk_units = p.units / p.nb;
  const int64_t ci = u % chunk_units;
  const int fbw = p.diagonal ? int((u / chunk_units + ci) % p.nbw) : int(u / chunk_units);
  const int fb = blocks * fbw + half;
  return Dim1Slot{ci, fb, fb < p.nb && u < p.wg_units};
}

// PAIR: one workgroup of twice the threads takes two neighbouring feature
// blocks of the same token chunk; its halves quantise one block each from the
// two staged tiles (each token row then reads 512 bytes, not 256). Used with
// the diagonal order: 395.4 against 405.8 us on the (16, 5120, 8192) expert
// weights; in token-chunk-first order on (131072, 7168) tokens it was slower
// (579 against 550 us), so that order keeps one block per workgroup.
template <bool PAIR>
constexpr int dim1_threads() { return PAIR ? 2 * kThreads : kThreads; }
// LDS of a paired workgroup at most: two staged tiles and the group table
constexpr int kDim1PairMaxLds = 2 * kTileDwords * 4 + 3 * kMaxGroupsDim1 * 4;
static_assert(kDim1PairMaxLds <= 160 * 1024 && kTileDwords * 4 + 3 * kMaxGroupsDim1 * 4 <= 64 * 1024,
              "LDS per workgroup");

template <bool SMALL, bool PAIR>
__global__ __launch_bounds__(dim1_threads<PAIR>()) void quantize_dim1_kernel(Q1Params p) {
  constexpr int kBlocks = PAIR ? 2 : 1;            // feature blocks per workgroup
  constexpr int kThreadsW = dim1_threads<PAIR>();
  extern __shared__ __align__(16) int lds1[];
  int *group_lds = lds1 + kBlocks * kTileDwords;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave_w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int half = wave_w / kWavesPerGroup;          // the feature block of this half of the workgroup
  const int wave = wave_w % kWavesPerGroup;
  const int ht = int(threadIdx.x) % kThreads;        // thread index within the half
  uint32_t *tile = reinterpret_cast<uint32_t *>(lds1) + half * kTileDwords;

  const Dim1Slot sl = dim1_slot(p, blockIdx.x, kBlocks, half);
  const int64_t ci = sl.ci;                     // tile column (chunk) index over all groups
  const int fb = sl.fb;                         // feature block of this half
  const int fb0 = fb - half;                    // first feature block of the workgroup
  const bool live = sl.live;

  Groups1<SMALL> grp;
  grp.init(p, group_lds);
  const Dim1Unit un = dim1_unit(p, grp, ci, fb);
  if (un.spare) {   // (spare depends on ci only: the whole workgroup returns here)
    if (!live) return;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t a = un.zero.begin + 16 * ht; a < un.zero.full; a += 16 * kThreads)
      *reinterpret_cast<u32x4 *>(p.scales + a) = z;
    for (int64_t a = un.zero.full + 4 * ht; a < un.zero.end; a += 4 * kThreads)
      *reinterpret_cast<uint32_t *>(p.scales + a) = 0u;
    return;
  }
  const int ntok = un.ntok;
  const int64_t x_row0 = un.x_row0, q_col0 = un.q_col0, tile_off = un.tile_off;

  // stage the 128 x 128 bf16 tile of each feature block: 16 pieces of 16
  // bytes per token row and block, 8 per lane (the token range is the same
  // for both halves, it depends on ci only)
  {
    constexpr int kPieces = 16 * kBlocks;      // pieces per token row
    const int f_base = fb0 * kTileFeat;
    const __amdgpu_buffer_rsrc_t rsrc =
        byte_buffer(p.x + x_row0 + f_base, uint32_t(int64_t(ntok) * p.ld * 2));
    uint32_t *tiles = reinterpret_cast<uint32_t *>(lds1);
    uint4 v[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int slot = int(threadIdx.x) + it * kThreadsW;
      const int t = slot / kPieces, k = slot % kPieces;
      const bool valid = t < ntok && f_base + 8 * k < p.N;
      const uint32_t off = valid ? uint32_t(t) * uint32_t(p.ld) * 2u + 16u * uint32_t(k) : kOutOfRange;
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(off), 0, kStreamPolicy);
      v[it] = make_uint4(r[0], r[1], r[2], r[3]);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int slot = int(threadIdx.x) + it * kThreadsW;
      const int t = slot / kPieces, k = slot % kPieces;
      *reinterpret_cast<uint4 *>(tiles + (k / 16) * kTileDwords + tile_row(t) + 4 * (k % 16)) =
          mask_features(v[it], f_base + 8 * k, p.N);
    }
  }
  __syncthreads();
  if (!live) return;

  // quantise two feature columns (2p, 2p+1) of one 32-token block (tb)
  const int pl = lane >> 2, tb = lane & 3;
  const int pair = 16 * wave + pl;
  uint32_t d[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) d[i] = tile[tile_row(32 * tb + i) + pair];
  uint32_t m0 = 0, m1 = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    m0 = max(m0, mag_lo(d[i]));
    m1 = max(m1, mag_hi(d[i]));
  }
  const bool fin0 = m0 < 0x7f800000u, fin1 = m1 < 0x7f800000u;
  const int s0 = scale_exponent(m0), s1 = scale_exponent(m1);
  const float f0 = __uint_as_float(uint32_t(127 - s0) << 23), f1 = __uint_as_float(uint32_t(127 - s1) << 23);
  uint32_t c0[8], c1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c0[j] = fin0 ? e4m3x4(clamp448(bf16_lo(d[4 * j]) * f0), clamp448(bf16_lo(d[4 * j + 1]) * f0),
                          clamp448(bf16_lo(d[4 * j + 2]) * f0), clamp448(bf16_lo(d[4 * j + 3]) * f0))
                 : kE4m3Nan;
    c1[j] = fin1 ? e4m3x4(clamp448(bf16_hi(d[4 * j]) * f1), clamp448(bf16_hi(d[4 * j + 1]) * f1),
                          clamp448(bf16_hi(d[4 * j + 2]) * f1), clamp448(bf16_hi(d[4 * j + 3]) * f1))
                 : kE4m3Nan;
  }
  const int n0 = fb * kTileFeat + 2 * pair;
  if (32 * tb < ntok) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t col = q_col0 + 32 * tb;
    if (n0 < p.N) {
      uint8_t *dst = p.qT + int64_t(n0) * p.q_ld + col;
      *reinterpret_cast<u32x4 *>(dst) = u32x4{c0[0], c0[1], c0[2], c0[3]};
      *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{c0[4], c0[5], c0[6], c0[7]};
    }
    if (n0 + 1 < p.N) {
      uint8_t *dst = p.qT + int64_t(n0 + 1) * p.q_ld + col;
      *reinterpret_cast<u32x4 *>(dst) = u32x4{c1[0], c1[1], c1[2], c1[3]};
      *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{c1[4], c1[5], c1[6], c1[7]};
    }
  }
  if (tile_off >= 0) {
    // tile words of features 2p and 2p+1: byte tb of each comes from lane 4p+tb
    const uint32_t b0 = fin0 ? uint32_t(s0 + 127) : 0xffu, b1 = fin1 ? uint32_t(s1 + 127) : 0xffu;
    int w0 = int(b0 << (8 * tb)), w1 = int(b1 << (8 * tb));
    w0 |= __builtin_amdgcn_update_dpp(0, w0, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    w0 |= __builtin_amdgcn_update_dpp(0, w0, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    w1 |= __builtin_amdgcn_update_dpp(0, w1, 0xb1, 0xf, 0xf, false);
    w1 |= __builtin_amdgcn_update_dpp(0, w1, 0x4e, 0xf, 0xf, false);
    const int r = 2 * pair + (tb & 1);          // tile row written by this lane (lanes tb = 0, 1)
    if (tb < 2) {
      const int64_t off = tile_off + (r % 32) * 16 + (r / 32) * 4;
      *reinterpret_cast<uint32_t *>(p.scales + off) = uint32_t(tb == 0 ? w0 : w1);
    }
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Grid of the dim1 cast: p holds the sources, outputs, strides, groups and
// scale size (validated by the caller, scale_bytes > 0); sets the feature
// blocks and the units. False when the grid exceeds one launch.
bool dim1_geometry(Q1Params &p, int64_t N) {
  p.N = int(N);
  p.nb = int((N + kTileFeat - 1) / kTileFeat);
  p.padded_rows = round_up(N, 128);
  // tile columns: every group's plus the trailing tokens' plus at least one spare
  const int64_t chunk_units = (p.T + kTileTok - 1) / kTileTok + p.groups + 1;
  p.units = chunk_units * p.nb;
  const bool pair = dim1_blocks(p) == 2;
  p.nbw = pair ? (p.nb + 1) / 2 : p.nb;
  p.wg_units = chunk_units * p.nbw;
  p.deal = 0;
  p.slots = p.wg_units;
  return slots_for(true, p.wg_units, kDim1DealUnits) <= max_grid(pair ? dim1_threads<true>() : dim1_threads<false>());
}

template <bool PAIR>
const void *dim1_kernel_of(bool small) {
  return small ? reinterpret_cast<const void *>(&quantize_dim1_kernel<true, PAIR>)
               : reinterpret_cast<const void *>(&quantize_dim1_kernel<false, PAIR>);
}

// Grid and launch of the dim1 cast.
int launch_dim1(Q1Params &p, int64_t N, hipStream_t stream) {
  if (!dim1_geometry(p, N)) return MX_REARRANGE_ESHAPE;
  const bool small = p.groups <= kWave;
  const bool pair = dim1_blocks(p) == 2;
  const size_t lds = size_t(pair ? 2 : 1) * kTileDwords * 4 + (small ? 0 : size_t(3) * p.groups * sizeof(int));
  const void *fn = pair ? dim1_kernel_of<true>(small) : dim1_kernel_of<false>(small);
  // two staged tiles take more than the default 64 KB of LDS (gfx950: up to
  // 160 KB per workgroup); the allowance is always set to the same largest
  // size, so that concurrent calls never lower it under one another
  if (pair && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kDim1PairMaxLds) != hipSuccess)
    return MX_REARRANGE_ELAUNCH;
  const int threads = pair ? dim1_threads<true>() : dim1_threads<false>();
  // The token-chunk-first order of a grid of more than one pass deals runs of
  // kDim1DealUnits workgroups (token chunks of one feature block) to the XCDs
  // in turn; units that run together on one XCD still complete each other's
  // code lines in its L2. On 131072 x 7168 tokens: 528-529 us against 549-550
  // with contiguous ranges per XCD (runs of 48 to 128: 526-530 us; 16: 543;
  // 256: 537; whole feature blocks: 563). The diagonal order of the paired
  // expert cast keeps contiguous ranges (runs of 64: the same; 16 and 256
  // slower).
  if (!pair) {
    const int64_t resident = resident_workgroups(fn, threads, lds);
    if (resident > 0 && p.wg_units > resident) {
      p.deal = kDim1DealUnits;
      p.slots = slots_for(true, p.wg_units, p.deal);
    }
  }
  void *args[] = {&p};
  const hipError_t e = hipLaunchKernel(fn, dim3(unsigned(p.slots)), dim3(unsigned(threads)), args, lds, stream);
  return e == hipSuccess ? MX_REARRANGE_OK : MX_REARRANGE_ELAUNCH;
}

template <bool SMALL>
const void *dim0_kernel_of(bool il) {
  return il ? reinterpret_cast<const void *>(&quantize_dim0_kernel<SMALL, true>)
            : reinterpret_cast<const void *>(&quantize_dim0_kernel<SMALL, false>);
}

const void *dim0_kernel_for(bool small, bool il) { return small ? dim0_kernel_of<true>(il) : dim0_kernel_of<false>(il); }

}  // namespace

extern "C" {

int mx_quantize_dim0_M_groups(const uint16_t *x, int64_t rows, int64_t K, int64_t row_stride,
                              const int32_t *group_end_offsets, int32_t num_groups, uint8_t *q,
                              uint8_t *blocked_scales, hipStream_t stream) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (rows < 0 || K < 0 || K % 32 != 0 || row_stride < K || row_stride > kMaxRowStride) return MX_REARRANGE_ESHAPE;
  if (num_groups < 1 || num_groups > kMaxGroups) return MX_REARRANGE_EGROUPS;
  if (rows > lim - 128 * int64_t(num_groups) || K > lim) return MX_REARRANGE_ESHAPE;
  if (group_end_offsets == nullptr) return MX_REARRANGE_ENULL;
  const int64_t scale_bytes = mx_quantize_dim0_M_groups_scale_bytes(rows, K, num_groups);
  if (rows * K > 0 && (x == nullptr || q == nullptr)) return MX_REARRANGE_ENULL;
  if (scale_bytes > 0 && blocked_scales == nullptr) return MX_REARRANGE_ENULL;
  // alignment matters only for buffers that are touched
  if (rows * K > 0 && ((reinterpret_cast<uintptr_t>(x) & 15) || (row_stride & 7) || (reinterpret_cast<uintptr_t>(q) & 15)))
    return MX_REARRANGE_EALIGN;
  if (scale_bytes > 0 && (reinterpret_cast<uintptr_t>(blocked_scales) & 15)) return MX_REARRANGE_EALIGN;
  if (scale_bytes == 0) return MX_REARRANGE_OK;   // K == 0: nothing to write

  QParams p = {};
  p.x = x;
  p.offs = group_end_offsets;
  p.q = q;
  p.scales = blocked_scales;
  p.ld = row_stride;
  int64_t grid = dim0_geometry(p, rows, K, num_groups);
  if (grid - p.data_groups + slots_for(true, p.data_groups, int64_t(kDim0DealWgs)) > max_grid(kThreads))
    return MX_REARRANGE_ESHAPE;
  const bool small = num_groups <= kWave;
  const size_t lds = small ? 0 : size_t(2) * num_groups * sizeof(int);
  // A grid of more than one pass over the GPU deals runs of kDim0DealWgs
  // workgroups to the XCDs in turn (launch_order.h). With whole 128-row blocks
  // as the runs (the 32 rows whose scale words share a tile line then write
  // them through one L2) it measured 92.0 against 95.1 us on the (131072, 1408)
  // cast and 45.5 against 45.7 on (16640, 5120) next to contiguous ranges;
  // runs of 48 workgroups then measured faster or the same on six of seven
  // shapes: (131072, 1408) 90.0 against 91.3 us, (16640, 5120) 45.0 against
  // 45.5, (49152, 4096) 97.1 against 98.2, (262144, 512) 66.4 against 67.0,
  // (100000, 1024) 52.2 against 52.5, (65536, 2048) the same, (32768, 7168)
  // 114.1 against 113.9. A grid of one pass keeps contiguous ranges.
  const bool il = [&] {
    const int64_t resident = resident_workgroups(dim0_kernel_for(small, false), kThreads, lds);
    return resident > 0 && p.data_groups > resident;
  }();
  p.deal = kDim0DealWgs;
  p.data_slots = slots_for(il, p.data_groups, p.deal);
  grid = p.data_slots + p.pad_blocks;
  const void *fn = dim0_kernel_for(small, il);
  void *args[] = {&p};
  const hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(kThreads), args, lds, stream);
  return e == hipSuccess ? MX_REARRANGE_OK : MX_REARRANGE_ELAUNCH;
}


int mx_quantize_dim1_K_groups(const uint16_t *x, int64_t T, int64_t N, int64_t row_stride,
                              const int32_t *token_group_end_offsets, int32_t num_groups, uint8_t *qT,
                              uint8_t *blocked_scales, hipStream_t stream) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (T < 0 || N < 0 || T % 32 != 0 || row_stride < N || row_stride > kMaxRowStrideDim1) return MX_REARRANGE_ESHAPE;
  if (num_groups < 1 || num_groups > kMaxGroupsDim1) return MX_REARRANGE_EGROUPS;
  if (T > lim || N > lim - 128 || T / 32 + 4 * int64_t(num_groups) > lim) return MX_REARRANGE_ESHAPE;
  if (token_group_end_offsets == nullptr) return MX_REARRANGE_ENULL;
  const int64_t scale_bytes = mx_quantize_dim1_K_groups_scale_bytes(T, N, num_groups);
  if (T * N > 0 && (x == nullptr || qT == nullptr)) return MX_REARRANGE_ENULL;
  if (scale_bytes > 0 && blocked_scales == nullptr) return MX_REARRANGE_ENULL;
  if (T * N > 0 && ((reinterpret_cast<uintptr_t>(x) & 15) || (row_stride & 7) || (reinterpret_cast<uintptr_t>(qT) & 15)))
    return MX_REARRANGE_EALIGN;
  if (scale_bytes > 0 && (reinterpret_cast<uintptr_t>(blocked_scales) & 15)) return MX_REARRANGE_EALIGN;
  if (scale_bytes == 0) return MX_REARRANGE_OK;   // N == 0: nothing to write

  Q1Params p = {};
  p.x = x;
  p.offs = token_group_end_offsets;
  p.qT = qT;
  p.scales = blocked_scales;
  p.ld = row_stride;
  p.T = T;
  p.q_ld = T;
  p.groups = num_groups;
  p.scale_bytes = scale_bytes;
  return launch_dim1(p, N, stream);
}

int mx_quantize_dim1_3d(const uint16_t *w, int64_t experts, int64_t K, int64_t N, int64_t expert_stride,
                        int64_t row_stride, uint8_t *q, uint8_t *blocked_scales, hipStream_t stream) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (experts < 0 || K < 0 || N < 0 || K % 32 != 0 || row_stride < N || row_stride > kMaxRowStrideDim1 ||
      expert_stride < 0)
    return MX_REARRANGE_ESHAPE;
  if (experts > kMaxGroupsDim1) return MX_REARRANGE_EGROUPS;
  if (K > lim || N > lim - 128 || (experts > 0 && K > lim / experts)) return MX_REARRANGE_ESHAPE;
  if (experts > 1 && expert_stride > INT64_MAX / experts) return MX_REARRANGE_ESHAPE;
  const int64_t scale_bytes = mx_quantize_dim1_3d_scale_bytes(experts, K, N);
  if (scale_bytes == 0) return MX_REARRANGE_OK;   // no experts, no tokens or no features: nothing to write
  if (w == nullptr || q == nullptr || blocked_scales == nullptr) return MX_REARRANGE_ENULL;
  if ((reinterpret_cast<uintptr_t>(w) & 15) || (row_stride & 7) || (expert_stride & 7) ||
      (reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(blocked_scales) & 15))
    return MX_REARRANGE_EALIGN;

  Q1Params p = {};
  p.x = w;
  p.offs = nullptr;
  p.qT = q;
  p.scales = blocked_scales;
  p.ld = row_stride;
  p.T = experts * K;
  p.q_ld = K;
  p.x_gstride = expert_stride;
  p.q_gstride = N * K;
  p.group_tokens = int(K);
  p.diagonal = K % kTileTok == 0;
  p.groups = int(experts);
  p.scale_bytes = scale_bytes;
  return launch_dim1(p, N, stream);
}

}  // extern "C"
