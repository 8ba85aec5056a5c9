// Wave64 scans, buffer descriptors and the M-groups row table for gfx950,
// shared by the rearrangement kernels (forward and inverse), the MXFP8 casts
// and the per-group pad/unpad kernels.
//
// The table follows the M-groups layout ("[mxfp8 moe training] compute prefix
// sum of group sizes inside kernel intead of precomputing", Context and
// Changes): group g holds input rows [end(g-1), end(g)) and starts at output
// row pend(g-1), the sum of round_up(size_h, 128) over the groups before it.
// End offsets are clamped into [previous end, rows], which leaves valid
// offsets unchanged and keeps every access in bounds for invalid ones.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kTileRows = 128;
constexpr int kRawBufferFlags = 0x00020000;       // buffer descriptor word 3: 32-bit raw data
constexpr uint32_t kOutOfRange = 0xfffffff0u;     // buffer offset past any range: the load returns 0

// Largest grid of `threads`-thread workgroups one launch may have: the runtime
// limits gridDim.x * blockDim.x to below 2^32 work-items. Entry points whose
// grid would exceed it return MX_REARRANGE_ESHAPE (outputs of over 100 GB).
constexpr int64_t max_grid(int threads) { return ((int64_t(1) << 32) - 1) / threads; }

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, true);  // lanes without a source read 0
}

__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += dpp<0x111>(x);                                               // row_shr:1
  x += dpp<0x112>(x);                                               // row_shr:2
  x += dpp<0x114>(x);                                               // row_shr:4
  x += dpp<0x118>(x);                                               // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// Inclusive running maximum of non-negative values.
__device__ __forceinline__ int wave_inclusive_max(int x) {
  x = max(x, dpp<0x111>(x));
  x = max(x, dpp<0x112>(x));
  x = max(x, dpp<0x114>(x));
  x = max(x, dpp<0x118>(x));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return x;
}

// Value of the previous lane (wave_shr:1); lane 0 gets `first`.
//
// The empty asm keeps the shift a plain v_mov_b32_dpp. Without it the compiler
// folds the shift into a following `a - shifted` as v_subrev_u32_dpp, and on
// gfx950 that instruction returns `shifted - a` (measured for wave_shr, wave_shl,
// row_shr and quad_perm controls; v_add/v_sub/v_max with DPP are right): every
// group width would come out negated. A build check rejects reversed-operand
// DPP instructions in the generated code.
__device__ __forceinline__ int wave_shift_up(int x, int first) {
  int r = __builtin_amdgcn_update_dpp(first, x, 0x138, 0xf, 0xf, false);
  asm("" : "+v"(r));
  return r;
}

// One 64-group slice of the end-offset scan, continuing from the carries:
// e = clamped cumulative end, pend = padded cumulative end.
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

// The scanned groups. Up to 64 groups they live in two registers of every wave
// (lane g holds group g) and each wave scans for itself: no LDS, no barrier.
// Beyond that one wave scans into LDS (2 * groups ints) and the workgroup
// synchronises inside init, so every thread must call it.
template <bool SMALL>
struct MGroups;

template <>
struct MGroups<true> {
  int groups, e, pend;
  __device__ __forceinline__ void init(const int32_t *offs, int n, int rows, int *) {
    groups = n;
    scan_slice(offs, n, rows, 0, 0, 0, e, pend);
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
struct MGroups<false> {
  int groups;
  const int *ends, *pends;
  __device__ __forceinline__ void init(const int32_t *offs, int n, int rows, int *lds) {
    groups = n;
    int *e_out = lds, *p_out = lds + n;
    if (threadIdx.x < kWave) {
      int carry_end = 0, carry_pend = 0;
      for (int base = 0; base < n; base += kWave) {
        int e, pend;
        scan_slice(offs, n, rows, base, carry_end, carry_pend, e, pend);
        const int g = base + int(threadIdx.x);
        if (g < n) {
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

// Buffer resource over [base, base + bytes) for raw buffer loads; a load whose
// offset lies past `bytes` returns zeros and touches no memory. Base and size
// are the same for the whole wave; each half of the address goes through
// readfirstlane as uint32_t so that the low half is not sign-extended.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_buffer(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(int(bytes)), kRawBufferFlags);
}

}  // namespace
