/*
 * mx_rearrange.h — C ABI of the gfx950 grouped MXFP8 scale-factor rearrangement.
 *
 * Converts a row-major matrix of E8M0 scale bytes (one byte per 32 data
 * elements) into the blocked, swizzled scale-factor layout built from 128x4
 * tiles, one group at a time. Groups run along M (token groups, rows) or along
 * K (weight-gradient groups, scale columns). Each group's padded output start
 * is a prefix sum of the padded sizes of the groups before it, and it is
 * computed inside the kernel from the cumulative end offsets: no host
 * synchronisation, no device-to-host read, no extra launch.
 *
 * Sources (pytorch/ao pull-request pages):
 *   "[mxfp8 moe training] compute prefix sum of group sizes inside kernel intead
 *    of precomputing" — Context and Changes: the blocked swizzled target format,
 *    per-group padded starts, the prefix sum moved into the kernel.
 *   "[mxfp8 moe training] fallback cuda kernel for when input doesn't meet 2d
 *    TMA constraints" — Context: groups along M, rows of any byte width (44-byte
 *    rows), no 16-byte row-stride requirement.
 *   "[mxfp8 moe training] add bench script for scale conversion to blocked
 *    format kernels for groups along K" — the 128x4 scale-factor tiles of each
 *    group along K.
 *   "Add CuTeDSL MXFP8 K-groups scale rearrange kernel" — review notes: group
 *    widths padded to multiples of 4 scale columns, empty groups contribute
 *    nothing, padding is zero.
 *
 * Layout written (the pages name it but do not print the byte map; this is
 * the reading implemented):
 *   - A tile holds a 128-row x 4-column block; its element (r, c) is byte
 *     (r mod 32)*16 + (r div 32)*4 + c of the tile's 512 bytes.
 *   - The tiles of a matrix follow one another row-major over (row block,
 *     column block).
 *   - M groups: group g = input rows [offs[g-1], offs[g]) (offs[-1] = 0) is
 *     padded to round_up(size,128) rows and round_up(cols,4) columns; padded
 *     groups are stacked, so group g's tiles start at byte
 *     round_up(cols,4) * (sum over h < g of round_up(size_h,128)).
 *   - K groups: group g = input columns [offs[g-1], offs[g]) is its own blocked
 *     matrix of round_up(rows,128) rows and round_up(width,4) columns, stored
 *     contiguously from byte round_up(rows,128) * (sum over h < g of
 *     round_up(width_h,4)).
 *   - Every padding byte, and every byte after the last group's data up to the
 *     end of the output (the sizes below), is written as 0x00.
 *
 * Common arguments of both entry points:
 *   scales             device pointer to the uint8 scale matrix, `rows` rows of
 *                      `cols` bytes, row r starting at scales + r*row_stride.
 *                      Any byte alignment. May be NULL when rows*cols == 0.
 *                      Read only.
 *   rows, cols         matrix shape in bytes (scale elements); >= 0, with
 *                      rows + 128*num_groups < 2^31 and cols + 4*num_groups < 2^31.
 *   row_stride         bytes between consecutive rows; cols <= row_stride <= 2^24.
 *                      No alignment requirement.
 *   group_end_offsets  device pointer to int32[num_groups], cumulative
 *                      exclusive group ends, non-decreasing, in rows (M) or
 *                      scale columns (K); the last may be below rows (M) or
 *                      cols (K), leaving trailing rows or columns in no group.
 *                      Never NULL. Read only.
 *   num_groups         G >= 1.
 *   out                device pointer, 16-byte aligned, at least
 *                      mx_rearrange_M_groups_out_bytes(...) or
 *                      mx_rearrange_K_groups_out_bytes(...) bytes. Every byte of
 *                      that range is written (no pre-zeroing needed); no byte
 *                      past it is touched. Must not overlap the inputs. May be
 *                      NULL when the output size is 0.
 *   stream             HIP stream the single kernel is enqueued on (NULL: the
 *                      default stream).
 *
 * Ownership: the caller owns every buffer; the library allocates nothing and
 * holds no pointer after returning. Its only internal state is a per-device
 * cache of kernel occupancy answers (which pick the grid order), filled under
 * a lock on first use. Calls are thread-safe: any number of host threads may
 * call any entry point at once, each on its own stream.
 *
 * Errors: a negative status is returned and nothing is enqueued when an
 * argument is invalid (see MX_REARRANGE_E*); the checks read no device memory.
 * Offsets that break the preconditions above cannot be checked without a
 * synchronisation: the kernel then clamps each end offset into
 * [previous end, rows or cols], so it still reads only inside the scale
 * matrix and writes only inside out[0, out_bytes); the bytes written are then
 * those of the clamped offsets.
 */
#ifndef MX_REARRANGE_H
#define MX_REARRANGE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

#define MX_REARRANGE_OK 0
#define MX_REARRANGE_ENULL (-1)        /* a required pointer is NULL */
#define MX_REARRANGE_ESHAPE (-2)       /* a size negative or too large, or a row stride out of its range */
#define MX_REARRANGE_EGROUPS (-3)      /* num_groups < 1 (or above the cap of a cast) */
#define MX_REARRANGE_EALIGN (-4)       /* a buffer (or row stride) not aligned as required */
#define MX_REARRANGE_ELAUNCH (-5)      /* the HIP launch failed */

/*
 * The size helpers and the status text are static inline functions of this
 * header, not library symbols: the library exports only the entry points.
 */

/*
 * Output size in bytes for groups along M: (rows + 128*num_groups) *
 * round_up(cols, 4). This bounds the padded total for any group sizes, since
 * the sum of round_up(size_g, 128) is below rows + 128*num_groups. Returns -1
 * for invalid sizes (negative, num_groups < 1).
 */
static inline int64_t mx_rearrange_M_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups) {
  if (rows < 0 || cols < 0 || num_groups < 1) return -1;
  return (rows + 128 * (int64_t)num_groups) * ((cols + 3) / 4 * 4);
}

/*
 * Output size in bytes for groups along K: round_up(rows, 128) *
 * (cols + 4*num_groups) — the byte count behind every bandwidth figure printed
 * on the K-groups pages (the bench-script page's results table, the CuTeDSL
 * page's tables). Returns -1 for invalid sizes.
 */
static inline int64_t mx_rearrange_K_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups) {
  if (rows < 0 || cols < 0 || num_groups < 1) return -1;
  return (rows + 127) / 128 * 128 * (cols + 4 * (int64_t)num_groups);
}

/* Static text for a status code returned by any entry point of this library. */
static inline const char *mx_rearrange_strerror(int status) {
  switch (status) {
    case MX_REARRANGE_OK: return "success";
    case MX_REARRANGE_ENULL: return "a required pointer is NULL";
    case MX_REARRANGE_ESHAPE: return "invalid shape or stride: negative, too large, or a row stride out of its range";
    case MX_REARRANGE_EGROUPS: return "num_groups out of range (at least 1; the casts and the inverse also cap it)";
    case MX_REARRANGE_EALIGN: return "a buffer or row stride is not aligned as the entry point requires";
    case MX_REARRANGE_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

/*
 * Groups along M (token groups): rows [offs[g-1], offs[g]) of `scales` become
 * group g's blocked matrix, rows padded to a multiple of 128 and columns to a
 * multiple of 4, stacked after the previous groups' padded rows. One kernel
 * launch on `stream`; returns after enqueueing.
 */
int mx_block_rearrange_M_groups(const uint8_t *scales, int64_t rows, int64_t cols,
                                int64_t row_stride, const int32_t *group_end_offsets,
                                int32_t num_groups, uint8_t *out, hipStream_t stream);

/*
 * Groups along K (weight-gradient groups): columns [offs[g-1], offs[g]) of
 * `scales` become group g's blocked matrix, columns padded to a multiple of 4
 * and rows to a multiple of 128, stored contiguously after the previous
 * groups' matrices. One kernel launch on `stream`; returns after enqueueing.
 */
int mx_block_rearrange_K_groups(const uint8_t *scales, int64_t rows, int64_t cols,
                                int64_t row_stride, const int32_t *group_end_offsets,
                                int32_t num_groups, uint8_t *out, hipStream_t stream);

/*
 * Per-expert (3-D) weight scales. Source: "[mxfp8 moe training] use dim1 cast
 * cuda kernel for 3d weights by reshaping to 2d" — the grouped GEMM's weight
 * operand B of shape (E, N, K) (Benchmarks tables, B_shape), quantized in
 * blocks of 32 along K, has scales of shape (E, N, K/32). Each expert is one
 * group of exactly N rows, so no offsets and no scan are needed: expert e's
 * (rows x cols) scale matrix becomes its own blocked matrix of
 * round_up(rows,128) rows and round_up(cols,4) columns (the tile map above),
 * stored from byte e * round_up(rows,128) * round_up(cols,4). This equals the
 * M-groups layout of E equal groups of `rows` rows, without the M-groups tail.
 *
 * Output size in bytes: experts * round_up(rows,128) * round_up(cols,4);
 * -1 for invalid sizes (negative, rows or cols >= 2^31 - 128, or a size that
 * does not fit in int64).
 */
static inline int64_t mx_rearrange_3d_out_bytes(int64_t experts, int64_t rows, int64_t cols) {
  const int64_t lim = ((int64_t)1 << 31) - 128;
  if (experts < 0 || rows < 0 || cols < 0 || rows >= lim || cols >= lim) return -1;
  const int64_t per_expert = (rows + 127) / 128 * 128 * ((cols + 3) / 4 * 4);
  if (per_expert > 0 && experts > INT64_MAX / per_expert) return -1;
  return experts * per_expert;
}

/*
 * scales         device pointer; element (e, i, j) at
 *                scales + e*expert_stride + i*row_stride + j. Any byte
 *                alignment. May be NULL when experts*rows*cols == 0. Read only;
 *                experts may overlap (expert_stride 0 repeats one matrix).
 * experts        E >= 0.
 * rows, cols     N and K/32 of each expert's scale matrix, >= 0, below 2^31 - 128.
 * expert_stride  bytes between consecutive experts, >= 0.
 * row_stride     bytes between consecutive rows; cols <= row_stride <= 2^24.
 * out            device pointer, 16-byte aligned, at least
 *                mx_rearrange_3d_out_bytes(experts, rows, cols) bytes; every
 *                byte of that range is written, none past it. May be NULL when
 *                that size is 0. Must not overlap the input.
 * stream         HIP stream for the single kernel (NULL: the default stream).
 *
 * Ownership and errors as for the grouped entry points: nothing is
 * allocated or kept; an invalid argument returns a negative status
 * (MX_REARRANGE_ESHAPE for sizes and strides, MX_REARRANGE_ENULL,
 * MX_REARRANGE_EALIGN) with nothing enqueued.
 */
int mx_block_rearrange_3d(const uint8_t *scales, int64_t experts, int64_t rows, int64_t cols,
                          int64_t expert_stride, int64_t row_stride, uint8_t *out,
                          hipStream_t stream);

/*
 * The inverse rearrangement: reads a blocked layout as written by
 * mx_block_rearrange_M_groups / mx_block_rearrange_K_groups (same rows, cols,
 * offsets and num_groups; the pages describe no inverse kernel) and writes the
 * row-major rows x cols matrix: scales + r*row_stride holds row r (only its
 * first cols bytes are written; row_stride >= cols, any alignment). Positions
 * no group covers (rows at or past the last end offset for M groups, columns
 * at or past it for K groups) are written as 0x00.
 *   blocked  device, 16-byte aligned, the *_out_bytes(rows, cols, G) bytes of the
 *            forward output; read only. NULL allowed when rows*cols == 0.
 *   num_groups  1 <= G <= 4096; offsets as for the forward calls (clamped the
 *            same way when they break the order).
 * One kernel on `stream`; nothing allocated; errors as above.
 */
int mx_block_unrearrange_M_groups(const uint8_t *blocked, int64_t rows, int64_t cols,
                                  const int32_t *group_end_offsets, int32_t num_groups,
                                  uint8_t *scales, int64_t row_stride, hipStream_t stream);

int mx_block_unrearrange_K_groups(const uint8_t *blocked, int64_t rows, int64_t cols,
                                  const int32_t *group_end_offsets, int32_t num_groups,
                                  uint8_t *scales, int64_t row_stride, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_REARRANGE_H */
