/*
 * mx_quantize.h — C ABI of the gfx950 MXFP8 casts whose E8M0 scales are written
 * straight into the grouped blocked scale layouts: the dim0 cast for M groups
 * and the dim1 cast for K groups.
 *
 * Sources (pytorch/ao pull-request pages):
 *   "[mxfp8 moe training] use dim1 cast cuda kernel for 3d weights by reshaping
 *    to 2d" — first notes and Benchmarks tables: bf16 activations A of shape
 *    (16640, 5120) are cast to MXFP8 (blocks of 32 elements) before the grouped
 *    GEMM; the cast produces the E8M0 scales that the blocked layout holds.
 *   "[mxfp8 moe training] compute prefix sum of group sizes inside kernel intead
 *    of precomputing" — Context and Changes: the blocked layout of token-group
 *    scales, groups padded to 128 rows, padded starts computed in the kernel.
 *
 * Numerics (the pages do not state them; the OCP Microscaling (MX) v1.0 rule
 * for MXFP8 with E4M3 elements is the reading implemented):
 *   - a block is 32 consecutive elements of one row of x;
 *   - its scale is 2^s with s = floor(log2(max |x|)) - 8, clamped to
 *     [-127, 127], stored as the E8M0 byte s + 127; an all-zero block gets 0;
 *   - each element is stored as the E4M3 code (finite variant: 4 exponent bits
 *     with bias 7, 3 mantissa bits, largest 448, NaN 0x7F) nearest to x / 2^s,
 *     ties to the even code, saturated at +-448, sign kept;
 *   - a block holding a NaN or an infinity gets the byte 0xFF and every element
 *     of it the code 0x7F.
 *
 * Scale layout: exactly what mx_block_rearrange_M_groups (mx_rearrange.h)
 * writes for the row-major (rows, K/32) scale matrix of this cast and the same
 * group offsets: group g (rows [offs[g-1], offs[g])) padded to a multiple of
 * 128 rows and K/32 to a multiple of 4 columns, groups stacked, 128x4 tiles,
 * element (r, c) of a tile at byte (r mod 32)*16 + (r div 32)*4 + c, padding
 * and the tail of the allocation zero.
 */
#ifndef MX_QUANTIZE_H
#define MX_QUANTIZE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

/* The size helpers below are static inline functions of this header, not library symbols. */

/*
 * Bytes of the blocked scale output: (rows + 128*num_groups) * round_up(K/32, 4),
 * the M-groups output size for a (rows, K/32) scale matrix. -1 for invalid sizes
 * (negative, K not a multiple of 32, num_groups < 1).
 */
static inline int64_t mx_quantize_dim0_M_groups_scale_bytes(int64_t rows, int64_t K, int32_t num_groups) {
  if (rows < 0 || K < 0 || K % 32 != 0 || num_groups < 1) return -1;
  return (rows + 128 * (int64_t)num_groups) * ((K / 32 + 3) / 4 * 4);
}

/*
 * x                  device pointer to bf16 values (raw 16-bit patterns), rows x K,
 *                    row r at x + r*row_stride elements; 16-byte aligned. May be
 *                    NULL when rows*K == 0. Read only.
 * rows, K            shape; K a multiple of 32; rows + 128*num_groups < 2^31.
 * row_stride         elements between rows: K <= row_stride <= 2^26, a multiple of 8
 *                    (rows start on 16-byte boundaries).
 * group_end_offsets  device int32[num_groups], cumulative group ends in rows,
 *                    non-decreasing, the last <= rows (rows past it belong to no
 *                    group: they are quantised into q, their scales are not
 *                    placed). Never NULL. Offsets that break this are clamped into
 *                    [previous end, rows] as in mx_block_rearrange_M_groups.
 * num_groups         1 <= G <= 4096.
 * q                  device pointer, 16-byte aligned, rows*K bytes: E4M3 codes,
 *                    row-major with row stride K. May be NULL when rows*K == 0.
 * blocked_scales     device pointer, 16-byte aligned, at least
 *                    mx_quantize_dim0_M_groups_scale_bytes(rows, K, G) bytes; every
 *                    byte of that range is written, none past it. May be NULL when
 *                    that size is 0.
 * stream             HIP stream for the single kernel (NULL: the default stream).
 *
 * Stacked expert weights cast along their last dimension (E matrices of N x K)
 * need no entry point of their own: cast the (E*N) x K view with the E equal
 * group ends N, 2N, ..., E*N; the first E * round_up(N,128) * round_up(K/32,4)
 * bytes of blocked_scales are then the per-expert layout of mx_block_rearrange_3d
 * (the rest is the zero tail of the M-groups allocation).
 *
 * Ownership: the caller owns every buffer; nothing is allocated or kept.
 * Calls are thread-safe, as for the entry points of mx_rearrange.h.
 * Errors (negative status, nothing enqueued): MX_REARRANGE_ESHAPE for sizes and
 * strides, MX_REARRANGE_EGROUPS for num_groups, MX_REARRANGE_ENULL for a missing
 * pointer, MX_REARRANGE_EALIGN for alignment, MX_REARRANGE_ELAUNCH when the
 * launch fails (status values and mx_rearrange_strerror in mx_rearrange.h).
 */
int mx_quantize_dim0_M_groups(const uint16_t *x, int64_t rows, int64_t K, int64_t row_stride,
                              const int32_t *group_end_offsets, int32_t num_groups, uint8_t *q,
                              uint8_t *blocked_scales, hipStream_t stream);

/*
 * MXFP8 cast along the token dimension (dim1 cast) for the weight-gradient GEMM,
 * whose token groups run along K.
 *
 * Sources: "[mxfp8 moe training] use dim1 cast cuda kernel for 3d weights by
 * reshaping to 2d" — first notes: the dim1 cast quantises along the other
 * dimension and writes a column-major result; "Add CuTeDSL MXFP8 K-groups scale
 * rearrange kernel" — review notes: K-group offsets are token offsets divided
 * by the block size 32, group widths padded to 4 scale columns, empty groups
 * add nothing; "[mxfp8 moe training] add bench script for scale conversion to
 * blocked format kernels for groups along K" — the K-groups scale shape
 * (7168, 4096) of 131072 tokens.
 *
 * x is T x N (tokens x features) bf16; a block is 32 consecutive tokens of one
 * feature, quantised by the rule above. Codes are written transposed: qT is
 * N x T bytes, row n = feature n over all tokens (x's layout read column-major).
 * The N x T/32 scales go into the K-groups layout of mx_block_rearrange_K_groups
 * with scale-column offsets token_group_end_offsets[g] / 32 (integer division):
 * group g is its own blocked matrix of round_up(N,128) rows and
 * round_up(w_g,4) columns, stored from byte round_up(N,128) * (sum of the
 * earlier padded widths); padding and the tail are zero.
 *
 * Scale bytes: round_up(N, 128) * (T/32 + 4*num_groups); -1 for invalid sizes
 * (negative, T not a multiple of 32, num_groups < 1).
 */
static inline int64_t mx_quantize_dim1_K_groups_scale_bytes(int64_t T, int64_t N, int32_t num_groups) {
  if (T < 0 || N < 0 || T % 32 != 0 || num_groups < 1) return -1;
  return (N + 127) / 128 * 128 * (T / 32 + 4 * (int64_t)num_groups);
}

/*
 * x                        device bf16 bit patterns, T x N, row t at x + t*row_stride
 *                          elements; 16-byte aligned; NULL allowed when T*N == 0.
 * T, N                     T a multiple of 32; N + 128 < 2^31.
 * row_stride               N <= row_stride <= 2^23 elements, a multiple of 8.
 * token_group_end_offsets  device int32[num_groups], cumulative token ends,
 *                          non-decreasing, the last <= T; each a multiple of 32
 *                          for groups to own whole blocks (otherwise the scale
 *                          columns follow the integer division). Tokens past the
 *                          last end are quantised into qT without placed scales.
 *                          Offsets that break the order are clamped into
 *                          [previous end, T]. Never NULL.
 * num_groups               1 <= G <= 2048.
 * qT                       device, 16-byte aligned, N*T bytes of E4M3 codes (row
 *                          stride T); NULL allowed when T*N == 0.
 * blocked_scales           device, 16-byte aligned, at least
 *                          mx_quantize_dim1_K_groups_scale_bytes(T, N, G) bytes, all
 *                          written, none past it; NULL allowed when that is 0.
 * stream                   HIP stream for the single kernel.
 * Ownership and status codes as for mx_quantize_dim0_M_groups.
 */
int mx_quantize_dim1_K_groups(const uint16_t *x, int64_t T, int64_t N, int64_t row_stride,
                              const int32_t *token_group_end_offsets, int32_t num_groups, uint8_t *qT,
                              uint8_t *blocked_scales, hipStream_t stream);

/*
 * The dim1 cast of stacked expert weights, written per expert ("[mxfp8 moe
 * training] use dim1 cast cuda kernel for 3d weights by reshaping to 2d":
 * description and Next steps, a dim1 cast of the 3-D weights that writes each
 * expert's codes directly in column-major form; Benchmarks tables, weights of
 * shape (E, 8192, 5120)).
 *
 * w holds `experts` matrices of K x N bf16 bit patterns (expert e at
 * w + e*expert_stride elements, row k of it `row_stride` elements further per
 * row). Each is cast exactly as mx_quantize_dim1_K_groups casts a K x N
 * matrix with one group: blocks of 32 along K, codes transposed. Outputs:
 *   q               E x N x K E4M3 codes: expert e's row n (feature n over all K)
 *                   at q + e*N*K + n*K.
 *   blocked_scales  mx_quantize_dim1_3d_scale_bytes(E, K, N) bytes: expert e's
 *                   N x K/32 scales as one blocked matrix of round_up(N,128) x
 *                   round_up(K/32,4) bytes at e times that size — the layout
 *                   mx_block_rearrange_3d writes for (E, N, K/32) scales, and the
 *                   one mx_quantize_dim1_K_groups writes for the experts stacked
 *                   into E*K tokens with E equal groups, without its tail.
 * Arguments:
 *   experts         0 <= E <= 2048 (E == 0: nothing to do).
 *   K               a multiple of 32; E*K < 2^31.
 *   N               N + 128 < 2^31.
 *   expert_stride   >= 0 elements, a multiple of 8 (16-byte aligned experts; 0
 *                   repeats one matrix).
 *   row_stride      N <= row_stride <= 2^23 elements, a multiple of 8.
 *   w, q, blocked_scales  device, 16-byte aligned; NULL allowed only when
 *                   there is nothing to write (E, K or N zero).
 * One kernel on `stream`; nothing allocated; no device memory read during
 * validation. Status codes as for mx_quantize_dim0_M_groups (MX_REARRANGE_EGROUPS
 * for E > 2048).
 */
static inline int64_t mx_quantize_dim1_3d_scale_bytes(int64_t experts, int64_t K, int64_t N) {
  if (experts < 0 || K < 0 || N < 0 || K % 32 != 0) return -1;
  return experts * ((N + 127) / 128 * 128) * ((K / 32 + 3) / 4 * 4);
}

int mx_quantize_dim1_3d(const uint16_t *w, int64_t experts, int64_t K, int64_t N, int64_t expert_stride,
                        int64_t row_stride, uint8_t *q, uint8_t *blocked_scales, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_QUANTIZE_H */
