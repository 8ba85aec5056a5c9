// How the kernels' work units are dealt to the eight XCDs of gfx950, and the
// occupancy query that decides it.
//
// Workgroup b of a launch runs on XCD b mod 8. A grid that fits the chip in
// one pass (no more workgroups than the GPU holds at once) gives each XCD a
// contiguous range of units: units that share cache lines at their edges run
// under one L2. A larger grid deals runs of `per_block` consecutive units
// (whole 128-row blocks, or a part of one where its units share no lines but
// the edges of the run) to the XCDs in turn, so that the eight XCDs sweep
// neighbouring rows of memory together, as a streaming copy does, while the
// lines shared inside a run stay in one L2. Each kernel is built in both
// orders; the host picks one per launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

namespace {

// Unit of workgroup slot `slot` in a grid of contiguous ranges (`slots` a
// multiple of 8) or of interleaved runs of `per_block` units. Host and
// device: a CPU test checks that every unit gets exactly one slot.
template <bool INTERLEAVED>
__host__ __device__ inline int64_t unit_of_slot(int64_t slot, int64_t slots, int64_t per_block) {
  if constexpr (INTERLEAVED) {
    const int64_t k = slot >> 3;
    return ((k / per_block) * 8 + (slot & 7)) * per_block + k % per_block;
  } else {
    return (slot & 7) * (slots >> 3) + (slot >> 3);
  }
}

// Workgroup slots for `units` units in runs of `per_block` (the last run may
// hold fewer): a multiple of 8 that covers every unit (slots past the last
// unit do nothing).
inline int64_t slots_for(bool interleaved, int64_t units, int64_t per_block) {
  if (interleaved) {
    const int64_t blocks = (units + per_block - 1) / per_block;
    return int64_t(8) * ((blocks + 7) / 8) * per_block;
  }
  return (units + 7) / 8 * 8;
}

// Workgroups of kernel `fn` (threads per workgroup, bytes of LDS) the current
// GPU holds at once: CUs times the runtime's occupancy answer, kept per
// device, kernel, size and LDS bytes. 0 when a query fails.
inline int64_t resident_workgroups(const void *fn, int threads, size_t lds) {
  struct Entry {
    int dev;
    const void *fn;
    int threads;
    size_t lds;
    int64_t n;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry &e : cache)
      if (e.dev == dev && e.fn == fn && e.threads == threads && e.lds == lds) return e.n;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess)
    return 0;
  const int64_t n = int64_t(cus) * per_cu;
  std::lock_guard<std::mutex> lock(mu);
  if (cache.size() < 1024) cache.push_back(Entry{dev, fn, threads, lds, n});
  return n;
}

}  // namespace
