/*
 * mx_pad.h — C ABI of the gfx950 per-group padding of MXFP8 data rows.
 *
 * Source: "Add CuTeDSL MXFP8 K-groups scale rearrange kernel" lists MXFP8
 * pad/unpad kernels in its stack by title only. Reading implemented: token
 * groups along M (group g = rows [offs[g-1], offs[g]), offs[-1] = 0) are padded
 * to multiples of 128 rows and stacked, exactly as the M-groups scale layout
 * places their scale rows ("[mxfp8 moe training] compute prefix sum of group
 * sizes inside kernel intead of precomputing", Context and Changes): group g's
 * rows start at output row P_g = sum over h < g of round_up(size_h, 128), so
 * each data row sits at the row of its padded scales. The padded start is
 * computed inside the kernel from the end offsets; no host synchronisation.
 *
 * Bytes are moved as they are (E4M3 codes or any 1-byte data; for wider
 * elements pass cols in bytes). Rows that are 16-byte aligned throughout
 * (cols, both row strides and both base pointers multiples of 16) move in
 * 16-byte accesses; any other alignment is handled byte by byte.
 *
 * Offsets: int32 device array, non-decreasing, last <= rows; offsets that
 * break this are clamped into [previous end, rows]. 1 <= num_groups <= 4096.
 * Sizes: rows + 128*num_groups < 2^31, cols < 2^31, row strides <= 2^30.
 * Ownership: the caller owns every buffer; nothing is allocated or kept.
 * Calls are thread-safe, as for the entry points of mx_rearrange.h.
 * Errors: the MX_REARRANGE_* status codes of mx_rearrange.h, nothing enqueued.
 */
#ifndef MX_PAD_H
#define MX_PAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

/* Rows of the padded matrix: rows + 128*num_groups (a bound on the padded total
 * for any group sizes); -1 for invalid sizes. A static inline function of this
 * header, not a library symbol. */
static inline int64_t mx_pad_M_groups_out_rows(int64_t rows, int32_t num_groups) {
  if (rows < 0 || num_groups < 1) return -1;
  return rows + 128 * (int64_t)num_groups;
}

/*
 * data     device, rows x cols bytes, row r at data + r*row_stride (row_stride
 *          >= cols). Read only. NULL allowed when rows*cols == 0.
 * padded   device, mx_pad_M_groups_out_rows(rows, G) x cols bytes, row stride
 *          cols. Every byte is written: group rows, zero padding rows and the
 *          zero tail after the last group. NULL allowed when cols == 0.
 */
int mx_pad_M_groups(const uint8_t *data, int64_t rows, int64_t cols, int64_t row_stride,
                    const int32_t *group_end_offsets, int32_t num_groups, uint8_t *padded,
                    hipStream_t stream);

/*
 * The inverse. padded: device, mx_pad_M_groups_out_rows(rows, G) x cols bytes,
 * row stride cols, read only. data: device, rows x cols bytes written at row
 * stride row_stride (>= cols; bytes between cols and row_stride untouched);
 * row r of group g comes from padded row P_g + (r - offs[g-1]); rows at or
 * past the last end offset are written as zeros.
 */
int mx_unpad_M_groups(const uint8_t *padded, int64_t rows, int64_t cols,
                      const int32_t *group_end_offsets, int32_t num_groups, uint8_t *data,
                      int64_t row_stride, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_PAD_H */
