// Per-group padding of MXFP8 data rows for gfx950 (MI355X), and its inverse.
//
// "Add CuTeDSL MXFP8 K-groups scale rearrange kernel" lists MXFP8 pad/unpad
// kernels in its stack by title only. Reading implemented: padding places
// group g's rows (input rows [offs[g-1], offs[g])) at output rows
// [P_g, P_g + size_g), P_g = sum over h < g of round_up(size_h, 128) — the row
// placement of the M-groups scale layout ("[mxfp8 moe training] compute prefix
// sum of group sizes inside kernel intead of precomputing", Context and
// Changes), so data rows line up with their padded scale rows — and zeroes every
// other row of the (rows + 128*G) x cols output; unpadding reads them back and
// zeroes the rows past the last group.
//
// Pure data movement, HBM-bound. A work unit is 1 KB of one output row; a wave
// takes 4 consecutive units (row-major), finds each unit's source row from the
// group table (scanned into registers for G <= 64, into LDS beyond), issues all
// its 16-byte buffer loads (rows without a source load nothing and store zeros)
// and then its stores. Rows whose bytes are 16-byte aligned everywhere use
// 16-byte accesses; any other alignment copies byte by byte in the same layout.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "group_table.h"
#include "launch_order.h"
#include "mx_pad.h"
#include "mx_rearrange.h"
#include "write_ranges.h"

namespace {

constexpr int kPadThreads = 128;       // swept: 128, 256, 512
constexpr int kPadWaves = kPadThreads / kWave;
constexpr int kPadUnit = 1024;          // bytes of one output row per unit (64 lanes x 16 bytes)
constexpr int kPadUnroll = 2;           // units per wave (swept: 1, 2, 3, 4, 8)
constexpr int kPadMaxGroups = 4096;
constexpr int64_t kPadMaxRowStride = int64_t(1) << 30;
constexpr int kStreamPolicy = 2;        // buffer load bit 1: non-temporal

struct PadParams {
  const uint8_t *src;
  const int32_t *offs;
  uint8_t *dst;
  int64_t src_ld;       // bytes between source rows
  int64_t dst_ld;       // bytes between destination rows
  int64_t out_rows;     // destination rows
  int64_t units;        // out_rows * chunks
  int rows;             // unpadded rows (the group offsets' range)
  int cols;             // bytes per row
  int chunks;           // units per row
  int groups;
};

// Source row of destination row R, or -1 for a row of zeros. A source row
// outside the source matrix (src_rows rows), which only a wrong group table
// could give, is -1 as well: the kernel then reads nothing outside its input.
template <bool PAD, class TABLE>
__host__ __device__ inline int64_t source_row(const TABLE &grp, int groups, int64_t R, int64_t src_rows) {
  int64_t s = -1;
  if (PAD) {
    const int g = grp.count_pends_le(R);
    if (g >= groups) return -1;                       // tail past the last group's padded rows
    const int start = g ? grp.end(g - 1) : 0;
    const int pstart = g ? grp.pend_at(g - 1) : 0;
    const int64_t local = R - pstart;
    s = local < grp.end(g) - start ? start + local : -1;   // past the group's rows: padding
  } else {
    const int g = grp.count_ends_le(R);
    if (g >= groups) return -1;                       // rows past the last end
    const int start = g ? grp.end(g - 1) : 0;
    const int pstart = g ? grp.pend_at(g - 1) : 0;
    s = int64_t(pstart) + (R - start);
  }
  return s >= 0 && s < src_rows ? s : -1;
}

template <bool PAD, bool SMALL, bool VEC, bool IL>
__global__ __launch_bounds__(kPadThreads) void pad_kernel(PadParams p) {
  extern __shared__ __align__(16) int pad_lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  MGroups<SMALL> grp;
  grp.init(p.offs, p.groups, p.rows, pad_lds);
  // the order of workgroups over the XCDs (launch_order.h): contiguous ranges,
  // or, for grids of more than one pass, workgroups dealt to the XCDs in turn
  // (a workgroup's rows share no line with another's)
  const int64_t b = unit_of_slot<IL>(blockIdx.x, gridDim.x, 1);
  const int64_t u0 = (b * kPadWaves + wave) * kPadUnroll;
  if (u0 >= p.units) return;

  int64_t R = u0 / p.chunks;
  int c = int(u0 - R * p.chunks);
  int64_t src_row[kPadUnroll];
  int64_t dst_row[kPadUnroll];
  int col0[kPadUnroll];
  int64_t looked_up = -1, s_row = -1;
#pragma unroll
  for (int i = 0; i < kPadUnroll; ++i) {
    const bool valid = u0 + i < p.units;
    if (valid && R != looked_up) {
      looked_up = R;
      s_row = source_row<PAD>(grp, p.groups, R, PAD ? int64_t(p.rows) : p.rows + 128 * int64_t(p.groups));
    }
    src_row[i] = valid ? s_row : -1;
    dst_row[i] = valid ? R : -1;
    col0[i] = c * kPadUnit;
    if (++c == p.chunks) {
      c = 0;
      ++R;
    }
  }
  if (VEC) {
    uint4 v[kPadUnroll];
#pragma unroll
    for (int i = 0; i < kPadUnroll; ++i) {
      const int n = src_row[i] >= 0 ? min(kPadUnit, p.cols - col0[i]) : 0;
      const __amdgpu_buffer_rsrc_t rsrc =
          byte_buffer(p.src + (src_row[i] >= 0 ? src_row[i] * p.src_ld + col0[i] : 0), uint32_t(n));
      const uint32_t off = 16 * lane < n ? uint32_t(16 * lane) : kOutOfRange;
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(off), 0, kStreamPolicy);
      v[i] = make_uint4(t[0], t[1], t[2], t[3]);
    }
#pragma unroll
    for (int i = 0; i < kPadUnroll; ++i) {
      const int col = col0[i] + 16 * lane;
      if (dst_row[i] >= 0 && col < p.cols) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4{v[i].x, v[i].y, v[i].z, v[i].w},
                                    reinterpret_cast<u32x4 *>(p.dst + dst_row[i] * p.dst_ld + col));
      }
    }
  } else {
    // any alignment: 16 bytes per lane, byte by byte
#pragma unroll
    for (int i = 0; i < kPadUnroll; ++i) {
      if (dst_row[i] < 0) continue;
      const int col = col0[i] + 16 * lane;
      const int n = min(16, p.cols - col);
      uint8_t *d = p.dst + dst_row[i] * p.dst_ld + col;
      if (src_row[i] >= 0) {
        const uint8_t *s = p.src + src_row[i] * p.src_ld + col;
        for (int k = 0; k < n; ++k) d[k] = s[k];
      } else {
        for (int k = 0; k < n; ++k) d[k] = 0;
      }
    }
  }
}

template <bool PAD, bool SMALL, bool VEC>
const void *pad_kernel_of(bool il) {
  return il ? reinterpret_cast<const void *>(&pad_kernel<PAD, SMALL, VEC, true>)
            : reinterpret_cast<const void *>(&pad_kernel<PAD, SMALL, VEC, false>);
}

const void *pad_kernel_for(bool pad, bool small, bool vec, bool il) {
  if (pad)
    return small ? (vec ? pad_kernel_of<true, true, true>(il) : pad_kernel_of<true, true, false>(il))
                 : (vec ? pad_kernel_of<true, false, true>(il) : pad_kernel_of<true, false, false>(il));
  return small ? (vec ? pad_kernel_of<false, true, true>(il) : pad_kernel_of<false, true, false>(il))
               : (vec ? pad_kernel_of<false, false, true>(il) : pad_kernel_of<false, false, false>(il));
}

int launch_pad(bool pad, const uint8_t *src, int64_t rows, int64_t cols, int64_t src_ld, int64_t dst_ld,
               const int32_t *offs, int32_t num_groups, uint8_t *dst, hipStream_t stream) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (rows < 0 || cols < 0 || cols > lim || (pad ? src_ld : dst_ld) < cols ||
      (pad ? src_ld : dst_ld) > kPadMaxRowStride)
    return MX_REARRANGE_ESHAPE;
  if (num_groups < 1 || num_groups > kPadMaxGroups) return MX_REARRANGE_EGROUPS;
  if (rows > lim - 128 * int64_t(num_groups)) return MX_REARRANGE_ESHAPE;
  if (offs == nullptr) return MX_REARRANGE_ENULL;
  const int64_t padded_rows = rows + 128 * int64_t(num_groups);
  const int64_t out_rows = pad ? padded_rows : rows;
  const int64_t in_bytes = (pad ? rows : padded_rows) * cols;
  if (out_rows * cols == 0) return MX_REARRANGE_OK;   // nothing to write (and nothing read)
  if (in_bytes > 0 && src == nullptr) return MX_REARRANGE_ENULL;
  if (dst == nullptr) return MX_REARRANGE_ENULL;

  PadParams p = {};
  p.src = src;
  p.offs = offs;
  p.dst = dst;
  p.src_ld = src_ld;
  p.dst_ld = dst_ld;
  p.out_rows = out_rows;
  p.rows = int(rows);
  p.cols = int(cols);
  p.chunks = int((cols + kPadUnit - 1) / kPadUnit);
  p.groups = num_groups;
  p.units = out_rows * p.chunks;
  const bool vec = (cols % 16) == 0 && (src_ld % 16) == 0 && (dst_ld % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(src) % 16) == 0 && (reinterpret_cast<uintptr_t>(dst) % 16) == 0;
  const int64_t waves = (p.units + kPadUnroll - 1) / kPadUnroll;
  int64_t grid = (waves + kPadWaves - 1) / kPadWaves;
  if (slots_for(false, grid, 1) > max_grid(kPadThreads)) return MX_REARRANGE_ESHAPE;
  const bool small = num_groups <= kWave;
  const size_t lds = small ? 0 : size_t(2) * num_groups * sizeof(int);
  // A grid of more than one pass over the GPU deals its workgroups to the XCDs
  // in turn (launch_order.h): measured on the (16640, 5120) pad 29.8-29.9
  // against 32.0-32.2 us (whole 128-row blocks in turn: 30.4). A grid of one
  // pass keeps contiguous ranges.
  const bool il = [&] {
    const int64_t resident = resident_workgroups(pad_kernel_for(pad, small, vec, false), kPadThreads, lds);
    return resident > 0 && grid > resident;
  }();
  const void *fn = pad_kernel_for(pad, small, vec, il);
  grid = slots_for(il, grid, 1);
  void *args[] = {&p};
  const hipError_t e = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(kPadThreads), args, lds, stream);
  return e == hipSuccess ? MX_REARRANGE_OK : MX_REARRANGE_ELAUNCH;
}

}  // namespace

extern "C" {

int mx_pad_M_groups(const uint8_t *data, int64_t rows, int64_t cols, int64_t row_stride,
                    const int32_t *group_end_offsets, int32_t num_groups, uint8_t *padded, hipStream_t stream) {
  return launch_pad(true, data, rows, cols, row_stride, cols, group_end_offsets, num_groups, padded, stream);
}

int mx_unpad_M_groups(const uint8_t *padded, int64_t rows, int64_t cols, const int32_t *group_end_offsets,
                      int32_t num_groups, uint8_t *data, int64_t row_stride, hipStream_t stream) {
  return launch_pad(false, padded, rows, cols, cols, row_stride, group_end_offsets, num_groups, data, stream);
}

}  // extern "C"
