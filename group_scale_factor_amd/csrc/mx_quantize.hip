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

#include "mx_quantize.h"
#include "mx_rearrange.h"

namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / kWave;
constexpr int kUnitElems = 512;       // elements per wave-unit: 16 blocks, 4 tile columns of scales
constexpr int kUnroll = 4;            // units per wave, loads issued back to back (swept: 2..16)
constexpr int kTileRows = 128;
constexpr int kMaxGroups = 4096;      // LDS holds two int arrays of this many groups
constexpr int64_t kMaxRowStride = int64_t(1) << 26;   // elements; keeps unit offsets in 32 bits
constexpr int kRawBufferFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0xfffffff0u;
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
};

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += dpp<0x111>(x);
  x += dpp<0x112>(x);
  x += dpp<0x114>(x);
  x += dpp<0x118>(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}

__device__ __forceinline__ int wave_inclusive_max(int x) {
  x = max(x, dpp<0x111>(x));
  x = max(x, dpp<0x112>(x));
  x = max(x, dpp<0x114>(x));
  x = max(x, dpp<0x118>(x));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return x;
}

__device__ __forceinline__ int wave_shift_up(int x, int first) {
  return __builtin_amdgcn_update_dpp(first, x, 0x138, 0xf, 0xf, false);
}

// One 64-group slice of the end-offset scan: e = clamped cumulative end
// (prefix maximum of clamp(offs[g], 0, rows), continuing from carry_end),
// pend = sum over h <= g of round_up(size_h, 128) (continuing from carry_pend).
__device__ __forceinline__ void scan_slice(const int32_t *__restrict__ offs, int groups, int rows, int base,
                                           int carry_end, int carry_pend, int &e, int &pend) {
  const int g = base + int(threadIdx.x & (kWave - 1));
  e = g < groups ? offs[g] : 0;
  e = min(max(e, 0), rows);
  e = max(wave_inclusive_max(e), carry_end);
  const int prev = wave_shift_up(e, carry_end);
  const int padded = g < groups ? (e - prev + kTileRows - 1) / kTileRows * kTileRows : 0;
  pend = wave_inclusive_sum(padded) + carry_pend;
}

// The scanned groups: end(g) = clamped cumulative end of group g, pend(g) =
// padded cumulative end (rows of the blocked scales up to the end of group g).
// Up to 64 groups they live in two registers of every wave (lane g holds
// group g) and each wave scans for itself: no LDS, no barrier. Beyond that one
// wave scans into LDS and the workgroup synchronises.
template <bool SMALL>
struct Groups;

template <>
struct Groups<true> {
  int groups, e, pend;
  __device__ __forceinline__ void init(const QParams &p, int *) {
    groups = p.groups;
    scan_slice(p.offs, p.groups, p.rows, 0, 0, 0, e, pend);
  }
  __device__ __forceinline__ int count_ends_le(int64_t key) const {
    return __popcll(__ballot(int(threadIdx.x & (kWave - 1)) < groups && int64_t(e) <= key));
  }
  __device__ __forceinline__ int count_pends_le(int64_t key) const {
    return __popcll(__ballot(int(threadIdx.x & (kWave - 1)) < groups && int64_t(pend) <= key));
  }
  __device__ __forceinline__ int end(int g) const { return __builtin_amdgcn_readlane(e, g); }
  __device__ __forceinline__ int pend_at(int g) const { return __builtin_amdgcn_readlane(pend, g); }
};

template <>
struct Groups<false> {
  int groups;
  const int *ends, *pends;
  __device__ __forceinline__ void init(const QParams &p, int *lds) {
    groups = p.groups;
    int *e_out = lds, *p_out = lds + p.groups;
    if (threadIdx.x < kWave) {
      int carry_end = 0, carry_pend = 0;
      for (int base = 0; base < p.groups; base += kWave) {
        int e, pend;
        scan_slice(p.offs, p.groups, p.rows, base, carry_end, carry_pend, e, pend);
        const int g = base + int(threadIdx.x);
        if (g < p.groups) {
          e_out[g] = e;
          p_out[g] = pend;
        }
        carry_end = __builtin_amdgcn_readlane(e, kWave - 1);
        carry_pend = __builtin_amdgcn_readlane(pend, kWave - 1);
      }
    }
    __syncthreads();
    ends = e_out;
    pends = p_out;
  }
  // number of entries of arr (non-decreasing) that are <= key
  __device__ __forceinline__ int count_le(const int *arr, int64_t key) const {
    const int lane = threadIdx.x & (kWave - 1);
    int n = 0;
    for (int base = 0; base < groups; base += kWave) {
      const int c = __popcll(__ballot(base + lane < groups && int64_t(arr[base + lane]) <= key));
      n += c;
      if (c < kWave) break;
    }
    return n;
  }
  __device__ __forceinline__ int count_ends_le(int64_t key) const { return count_le(ends, key); }
  __device__ __forceinline__ int count_pends_le(int64_t key) const { return count_le(pends, key); }
  __device__ __forceinline__ int end(int g) const { return ends[g]; }
  __device__ __forceinline__ int pend_at(int g) const { return pends[g]; }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_buffer(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(int(bytes)), kRawBufferFlags);
}

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
__device__ __forceinline__ int64_t scale_word_offset(int64_t R, int tc, int tile_cols) {
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
        const int g = grp.count_ends_le(r);
        scale_row = -1;
        if (g < p.groups) {
          const int start = g ? grp.end(g - 1) : 0;
          const int pstart = g ? grp.pend_at(g - 1) : 0;
          scale_row = int64_t(pstart) + (r - start);
        }
      }
      const int tc = 4 * c + (lane >> 4);
      if ((lane & 15) == 12 && scale_row >= 0 && tc < p.tile_cols) {
        const int64_t off = scale_word_offset(scale_row, tc, p.tile_cols);
        *reinterpret_cast<uint32_t *>(p.scales + off) = uint32_t(word);
      }
    }
    if (++c == p.chunks) {
      c = 0;
      ++r;
    }
  }
}

// Zero-fill of output row block ob of the blocked scales: the padding rows of
// the group it belongs to, or all of it past the last group.
template <class GROUPS>
__device__ __forceinline__ void zero_block(const QParams &p, int64_t ob, const GROUPS &grp) {
  const int64_t block_bytes = int64_t(kTileRows) * p.tile_cols * 4;
  const int g = grp.count_pends_le(ob * kTileRows);
  if (g < p.groups) {
    const int start = g ? grp.end(g - 1) : 0;
    const int pstart = g ? grp.pend_at(g - 1) : 0;
    const int size = grp.end(g) - start;
    const int64_t k = ob - pstart / kTileRows;
    const int valid = int(min(int64_t(kTileRows), int64_t(size) - kTileRows * k));
    const int pad_rows = kTileRows - valid;
    const int n = pad_rows * p.tile_cols;
    for (int t = threadIdx.x; t < n; t += kThreads) {
      const int rr = valid + t / p.tile_cols;
      const int tc = t % p.tile_cols;
      const int64_t off = scale_word_offset(ob * kTileRows + rr, tc, p.tile_cols);
      if (off + 4 <= p.scale_bytes) *reinterpret_cast<uint32_t *>(p.scales + off) = 0u;
    }
  } else {
    const int64_t lo = max(ob * block_bytes, int64_t(grp.pend_at(p.groups - 1)) * p.tile_cols * 4);
    const int64_t hi = min((ob + 1) * block_bytes, p.scale_bytes);
    if (lo >= hi) return;
    // lo is a multiple of 512 (a row block boundary); hi a multiple of 4
    const int64_t full = lo + ((hi - lo) & ~int64_t(15));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t a = lo + 16 * threadIdx.x; a < full; a += 16 * kThreads)
      *reinterpret_cast<u32x4 *>(p.scales + a) = z;
    for (int64_t a = full + 4 * threadIdx.x; a < hi; a += 4 * kThreads) *reinterpret_cast<uint32_t *>(p.scales + a) = 0u;
  }
}

template <bool SMALL>
__global__ __launch_bounds__(kThreads) void quantize_dim0_kernel(QParams p) {
  extern __shared__ __align__(16) int lds_groups[];
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  Groups<SMALL> grp;
  if (int64_t(blockIdx.x) < p.data_groups) {
    // Workgroup b runs on XCD b mod 8: give each XCD one contiguous range of
    // units, so that the 32 rows whose scale words share a 128-byte line of a
    // tile are written through one L2 (whole-line write-backs instead of
    // partial ones from several XCDs).
    const int64_t n8 = p.data_groups / 8 * 8;
    const int64_t b = int64_t(blockIdx.x) < n8 ? (int64_t(blockIdx.x) & 7) * (n8 >> 3) + (int64_t(blockIdx.x) >> 3)
                                              : int64_t(blockIdx.x);
    // the data loads go out first; the group scan overlaps them
    const int64_t u0 = (b * kWavesPerGroup + wave) * kUnroll;
    uint4 v[kUnroll];
    load_units(p, u0, v);
    grp.init(p, lds_groups);
    if (u0 < p.units) quantize_units(p, u0, v, grp);
  } else {
    grp.init(p, lds_groups);
    const int64_t ob = int64_t(blockIdx.x) - p.data_groups;
    if (ob < p.pad_blocks) zero_block(p, ob, grp);
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

extern "C" {

int64_t mx_quantize_dim0_M_groups_scale_bytes(int64_t rows, int64_t K, int32_t num_groups) {
  if (rows < 0 || K < 0 || K % 32 != 0 || num_groups < 1) return -1;
  return (rows + 128 * int64_t(num_groups)) * round_up(K / 32, 4);
}

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
  p.rows = int(rows);
  p.K = int(K);
  p.chunks = int((K + kUnitElems - 1) / kUnitElems);
  p.groups = num_groups;
  p.tile_cols = int(round_up(K / 32, 4) / 4);
  p.units = rows * p.chunks;
  p.scale_bytes = scale_bytes;
  const int64_t waves = (p.units + kUnroll - 1) / kUnroll;
  p.data_groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  p.pad_blocks = (rows + kTileRows - 1) / kTileRows + num_groups;
  const int64_t grid = p.data_groups + p.pad_blocks;
  if (grid > lim) return MX_REARRANGE_ESHAPE;
  const bool small = num_groups <= kWave;
  const size_t lds = small ? 0 : size_t(2) * num_groups * sizeof(int);
  const void *fn = small ? reinterpret_cast<const void *>(&quantize_dim0_kernel<true>)
                         : reinterpret_cast<const void *>(&quantize_dim0_kernel<false>);
  void *args[] = {&p};
  const hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(kThreads), args, lds, stream);
  return e == hipSuccess ? MX_REARRANGE_OK : MX_REARRANGE_ELAUNCH;
}

}  // extern "C"
