// Byte ranges that the kernels derive from the scanned group table, kept inside
// the buffers they address.
//
// Every kernel here computes some of its load and store addresses from the
// group table it scans out of the end offsets (group starts, padded starts,
// padded widths). With a correct scan each clamp below leaves its value
// unchanged. Should a scan ever produce wrong sizes (a miscompiled shift once
// negated every group width), the output comes out wrong — a parity failure —
// but no load or store leaves its buffer.
//
// The functions are __host__ __device__: a CPU test compiles this header on the
// host and drives it with correct and with corrupted group tables.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// [begin, full): whole 16-byte pieces; [full, end): 4-byte words.
struct ZeroSpan {
  int64_t begin, full, end;
};

__host__ __device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Share `part` of `parts` of the zero-fill of [lo, hi) inside a buffer of
// `limit` bytes (limit a multiple of 4). lo is clamped into [0, limit] and down
// to a 16-byte boundary, hi into [lo, limit] and down to a multiple of 4; the
// shares of parts 0..parts-1 tile the clamped range in order, each non-empty
// one starting on a 16-byte boundary, so every byte is written once; a part
// outside [0, parts) gets nothing.
__host__ __device__ inline ZeroSpan zero_share(int64_t lo, int64_t hi, int64_t limit, int64_t part, int64_t parts) {
  ZeroSpan z = {0, 0, 0};
  limit = limit < 0 ? 0 : (limit & ~int64_t(3));
  lo = clamp64(lo, 0, limit) & ~int64_t(15);
  hi = clamp64(hi, lo, limit) & ~int64_t(3);
  if (hi <= lo || parts <= 0 || part < 0 || part >= parts) return z;
  const int64_t len16 = (hi - lo + 15) >> 4;
  const int64_t per = (len16 + parts - 1) / parts;
  const int64_t a = per * part < len16 ? per * part : len16;
  const int64_t b = per * (part + 1) < len16 ? per * (part + 1) : len16;
  z.begin = lo + 16 * a < hi ? lo + 16 * a : hi;
  z.end = lo + 16 * b < hi ? lo + 16 * b : hi;
  z.full = z.begin + ((z.end - z.begin) & ~int64_t(15));
  return z;
}

// Whether [off, off + bytes) lies inside a buffer of `limit` bytes.
__host__ __device__ inline bool fits(int64_t off, int64_t bytes, int64_t limit) {
  return bytes >= 0 && off >= 0 && off <= limit - bytes;
}

// A run of n items starting at `first`, kept inside [0, limit): first clamped
// into [0, limit], n into [0, limit - first].
struct Run {
  int64_t first, n;
};

__host__ __device__ inline Run clamp_run(int64_t first, int64_t n, int64_t limit) {
  Run r;
  r.first = clamp64(first, 0, limit < 0 ? 0 : limit);
  r.n = clamp64(n, 0, (limit < 0 ? 0 : limit) - r.first);
  return r;
}

}  // namespace
