/*
 * CPU oracle for the grouped MXFP8 scale-factor rearrangement.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. The HIP library never
 * includes, links or calls it, and this file uses nothing of the HIP library.
 *
 * It is the plain definition written out as nested loops over groups, then over
 * every position of each group's padded matrix, with one byte copied (or a zero
 * written) per position. Nothing here is blocked, fused or reordered.
 *
 * What is computed, and where the pages state it:
 *   - The target format is the blocked, swizzled scale-factor layout made of
 *     128x4 tiles ("[mxfp8 moe training] compute prefix sum of group sizes inside
 *     kernel intead of precomputing", Context; "[mxfp8 moe training] add bench
 *     script for scale conversion to blocked format kernels for groups along K",
 *     description above its table).
 *   - The pages never print the in-tile byte map or the tile order. Reading
 *     taken here: element (r, c) of a 128x4 tile sits at byte
 *     (r mod 32)*16 + (r div 32)*4 + c, and the tiles of a matrix follow each
 *     other row-major over (row block, column block).
 *   - Groups along M: each group's rows are padded up to a multiple of 128 and
 *     the groups' padded row ranges follow one another; a group's output start
 *     is the prefix sum of the padded sizes of the groups before it (page on the
 *     in-kernel prefix sum, Context and Changes; page on the fallback CUDA
 *     kernel, Context). Columns are padded up to a multiple of 4.
 *   - Groups along K: each group's width in scale columns is padded up to a
 *     multiple of 4, an empty group adds nothing, and rows are padded up to a
 *     multiple of 128 ("Add CuTeDSL MXFP8 K-groups scale rearrange kernel",
 *     review: the notes on empty groups and on the zero-initialised output).
 *     Reading taken here: each group is its own blocked matrix of
 *     round_up(rows,128) x W_g bytes, stored contiguously from byte
 *     round_up(rows,128) * (sum of W_h for h < g). No page prints a K-groups
 *     byte position, so parity against the pages is unpinned for this
 *     placement; the tests pin the code to the reading (hand-worked
 *     positions that separate it from the other readings, the inverse map).
 *   - Padding bytes are zero (same review, the note on the output being
 *     allocated with zeros).
 *   - Output sizes: K groups, round_up(rows,128) * (cols + 4*G) bytes, which is
 *     the byte count that reproduces every bandwidth figure printed on the
 *     K-groups pages (bench-script page, results table; CuTeDSL page, both
 *     results tables). M groups, by the same rule turned on its side:
 *     (rows + 128*G) * round_up(cols,4) bytes. Bytes past the last group's
 *     padded end are zero.
 *   - Group end offsets are cumulative and exclusive: group g covers
 *     [offs[g-1], offs[g]) with offs[-1] = 0, in rows (M) or scale columns (K).
 */

#include <stdint.h>
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EBADPTR (-1)
#define ORACLE_EBADSHAPE (-2)
#define ORACLE_EBADGROUPS (-3)
#define ORACLE_EBADOFFSETS (-6)

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

/* Byte offset of element (r, c), 0 <= r < 128, 0 <= c < 4, inside one 512-byte tile. */
static int64_t tile_byte(int64_t r, int64_t c) { return (r % 32) * 16 + (r / 32) * 4 + c; }

/*
 * Byte offset of element (i, j) of a matrix with `ncols` columns (ncols a
 * multiple of 4, row count a multiple of 128) stored in the blocked layout:
 * tile (i div 128, j div 4) is tile number (i div 128) * (ncols / 4) + (j div 4).
 */
static int64_t blocked_byte(int64_t ncols, int64_t i, int64_t j) {
    int64_t tile = (i / 128) * (ncols / 4) + (j / 4);
    return tile * 512 + tile_byte(i % 128, j % 4);
}

int64_t oracle_M_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups) {
    return (rows + 128 * (int64_t)num_groups) * round_up(cols, 4);
}

int64_t oracle_K_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups) {
    return round_up(rows, 128) * (cols + 4 * (int64_t)num_groups);
}

static int check_args(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld,
                      const int32_t *offs, int32_t num_groups, const uint8_t *out,
                      int64_t out_bytes, int64_t limit) {
    if (rows < 0 || cols < 0 || ld < cols) return ORACLE_EBADSHAPE;
    if (num_groups < 1) return ORACLE_EBADGROUPS;
    if (offs == 0 || (out == 0 && out_bytes > 0) || (scales == 0 && rows * cols > 0))
        return ORACLE_EBADPTR;
    int64_t prev = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        if (offs[g] < prev || offs[g] > limit) return ORACLE_EBADOFFSETS;
        prev = offs[g];
    }
    return ORACLE_OK;
}

/*
 * Groups along M. Group g holds input rows [offs[g-1], offs[g]); its padded
 * block of round_up(size,128) rows starts at output row out_row, the sum of the
 * padded sizes of the groups before it. The output rows of all groups together
 * form one blocked matrix with round_up(cols,4) columns.
 */
int oracle_M_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld,
                    const int32_t *offs, int32_t num_groups, uint8_t *out) {
    int64_t total = oracle_M_groups_out_bytes(rows, cols, num_groups);
    int rc = check_args(scales, rows, cols, ld, offs, num_groups, out, total, rows);
    if (rc != ORACLE_OK) return rc;
    if (total == 0) return ORACLE_OK;
    int64_t padded_cols = round_up(cols, 4);
    memset(out, 0, (size_t)total);

    int64_t out_row = 0;
    int64_t group_start = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t size = offs[g] - group_start;
        int64_t padded_rows = round_up(size, 128);
        for (int64_t i = 0; i < padded_rows; ++i) {
            for (int64_t j = 0; j < padded_cols; ++j) {
                uint8_t v = 0;
                if (i < size && j < cols) v = scales[(group_start + i) * ld + j];
                out[blocked_byte(padded_cols, out_row + i, j)] = v;
            }
        }
        out_row += padded_rows;
        group_start = offs[g];
    }
    return ORACLE_OK;
}

/*
 * Groups along K. Group g holds input columns [offs[g-1], offs[g]); it becomes
 * its own blocked matrix of round_up(rows,128) rows and round_up(width,4)
 * columns, stored contiguously from byte round_up(rows,128) * out_col, where
 * out_col is the sum of the padded widths of the groups before it.
 */
int oracle_K_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld,
                    const int32_t *offs, int32_t num_groups, uint8_t *out) {
    int64_t total = oracle_K_groups_out_bytes(rows, cols, num_groups);
    int rc = check_args(scales, rows, cols, ld, offs, num_groups, out, total, cols);
    if (rc != ORACLE_OK) return rc;
    if (total == 0) return ORACLE_OK;
    int64_t padded_rows = round_up(rows, 128);
    memset(out, 0, (size_t)total);

    int64_t out_col = 0;
    int64_t group_start = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t width = offs[g] - group_start;
        int64_t padded_width = round_up(width, 4);
        uint8_t *group_out = out + padded_rows * out_col;
        for (int64_t i = 0; i < padded_rows; ++i) {
            for (int64_t j = 0; j < padded_width; ++j) {
                uint8_t v = 0;
                if (i < rows && j < width) v = scales[i * ld + group_start + j];
                group_out[blocked_byte(padded_width, i, j)] = v;
            }
        }
        out_col += padded_width;
        group_start = offs[g];
    }
    return ORACLE_OK;
}

/*
 * The same two definitions, one call shared among `threads` POSIX threads: the
 * CPU baseline of one conversion spread over the host's cores. The work is
 * split into pieces of (group, 128-row block) — for K groups a row block of one
 * group's matrix, for M groups a row block of one group's padded rows — and
 * each piece runs exactly the loop body of oracle_M_groups / oracle_K_groups
 * over its own positions; pieces are handed out one at a time from a shared
 * counter. The zero-fill of the whole output before the copy is split into
 * equal ranges the same way, and all of it ends (the threads are joined)
 * before the first piece is copied. Nothing else differs: the same positions receive
 * the same bytes, in another order.
 */

struct piece_job {
    int kgroups;
    const uint8_t *scales;
    int64_t rows, cols, ld;
    const int32_t *offs;
    int32_t num_groups;
    uint8_t *out;
    int64_t total;
    const int64_t *first_piece; /* pieces of groups before g; num_groups + 1 entries */
    const int64_t *group_start; /* first input row (M) or column (K) of group g */
    const int64_t *group_base;  /* output row (M) or padded column (K) where group g starts */
    int64_t zero_parts;
    int64_t next;               /* shared counter: next zero range, then next piece */
};

static int64_t take(struct piece_job *job) { return __atomic_fetch_add(&job->next, 1, __ATOMIC_RELAXED); }

static void run_piece(const struct piece_job *job, int64_t p) {
    int32_t g = 0;
    while (job->first_piece[g + 1] <= p) ++g;
    int64_t i0 = 128 * (p - job->first_piece[g]);
    int64_t start = job->group_start[g];
    int64_t size = job->offs[g] - start;
    if (!job->kgroups) {
        int64_t padded_cols = round_up(job->cols, 4);
        int64_t out_row = job->group_base[g];
        for (int64_t i = i0; i < i0 + 128; ++i) {
            for (int64_t j = 0; j < padded_cols; ++j) {
                uint8_t v = 0;
                if (i < size && j < job->cols) v = job->scales[(start + i) * job->ld + j];
                job->out[blocked_byte(padded_cols, out_row + i, j)] = v;
            }
        }
    } else {
        int64_t padded_rows = round_up(job->rows, 128);
        int64_t padded_width = round_up(size, 4);
        uint8_t *dst = job->out + padded_rows * job->group_base[g];
        for (int64_t i = i0; i < i0 + 128; ++i) {
            for (int64_t j = 0; j < padded_width; ++j) {
                uint8_t v = 0;
                if (i < job->rows && j < size) v = job->scales[i * job->ld + start + j];
                dst[blocked_byte(padded_width, i, j)] = v;
            }
        }
    }
}

static void *zero_worker(void *arg) {
    struct piece_job *job = (struct piece_job *)arg;
    for (;;) {
        int64_t z = take(job);
        if (z >= job->zero_parts) break;
        int64_t per = (job->total + job->zero_parts - 1) / job->zero_parts;
        int64_t lo = z * per, hi = lo + per < job->total ? lo + per : job->total;
        if (lo < hi) memset(job->out + lo, 0, (size_t)(hi - lo));
    }
    return 0;
}

static void *copy_worker(void *arg) {
    struct piece_job *job = (struct piece_job *)arg;
    int64_t pieces = job->first_piece[job->num_groups];
    for (;;) {
        int64_t p = take(job);
        if (p >= pieces) break;
        run_piece(job, p);
    }
    return 0;
}

/* Runs fn on `threads` threads (this one included) and joins them. */
static void run_workers(void *(*fn)(void *), struct piece_job *job, int threads) {
    pthread_t tid[256];
    int n = threads < 1 ? 1 : (threads > 256 ? 256 : threads), started = 0;
    for (; started < n - 1; ++started)
        if (pthread_create(&tid[started], 0, fn, job) != 0) break;
    fn(job);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], 0);
}

static int grouped_threads(int kgroups, const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld,
                           const int32_t *offs, int32_t num_groups, uint8_t *out, int threads) {
    int64_t total = kgroups ? oracle_K_groups_out_bytes(rows, cols, num_groups)
                            : oracle_M_groups_out_bytes(rows, cols, num_groups);
    int rc = check_args(scales, rows, cols, ld, offs, num_groups, out, total, kgroups ? cols : rows);
    if (rc != ORACLE_OK) return rc;
    if (total == 0) return ORACLE_OK;
    int64_t *first_piece = (int64_t *)malloc(3 * ((size_t)num_groups + 1) * sizeof(int64_t));
    if (!first_piece) return ORACLE_EBADPTR;
    int64_t *group_start = first_piece + num_groups + 1, *group_base = group_start + num_groups + 1;
    int64_t start = 0, base = 0, pieces = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t size = offs[g] - start;
        first_piece[g] = pieces;
        group_start[g] = start;
        group_base[g] = base;
        if (kgroups) {
            /* an empty group has no matrix and no piece */
            pieces += size > 0 ? round_up(rows, 128) / 128 : 0;
            base += round_up(size, 4);
        } else {
            pieces += round_up(size, 128) / 128;
            base += round_up(size, 128);
        }
        start = offs[g];
    }
    first_piece[num_groups] = pieces;
    struct piece_job job = {kgroups, scales, rows, cols, ld, offs, num_groups, out, total,
                            first_piece, group_start, group_base, 0, 0};
    job.zero_parts = 4 * (int64_t)(threads < 1 ? 1 : threads);
    run_workers(zero_worker, &job, threads); /* every zero store lands before any copy starts */
    job.next = 0;
    run_workers(copy_worker, &job, threads);
    free(first_piece);
    return ORACLE_OK;
}

int oracle_M_groups_threads(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld,
                            const int32_t *offs, int32_t num_groups, uint8_t *out, int threads) {
    return grouped_threads(0, scales, rows, cols, ld, offs, num_groups, out, threads);
}

int oracle_K_groups_threads(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld,
                            const int32_t *offs, int32_t num_groups, uint8_t *out, int threads) {
    return grouped_threads(1, scales, rows, cols, ld, offs, num_groups, out, threads);
}

/*
 * Per-expert weight scales: `experts` matrices of rows x cols scale bytes,
 * matrix e starting at scales + e * expert_stride, row stride ld. Each becomes
 * its own blocked matrix of round_up(rows,128) x round_up(cols,4) bytes, the
 * experts one after another. This is the weight operand of the grouped GEMM
 * on "[mxfp8 moe training] use dim1 cast cuda kernel for 3d weights by
 * reshaping to 2d" (Benchmarks tables: B of shape (E, N, K)), whose scales
 * are (E, N, K/32); every expert is one group of exactly N rows, so no
 * offsets are needed. The layout of each matrix is the one read above.
 */
int64_t oracle_3d_out_bytes(int64_t experts, int64_t rows, int64_t cols) {
    return experts * round_up(rows, 128) * round_up(cols, 4);
}

int oracle_3d(const uint8_t *scales, int64_t experts, int64_t rows, int64_t cols, int64_t expert_stride,
              int64_t ld, uint8_t *out) {
    if (experts < 0 || rows < 0 || cols < 0 || ld < cols || expert_stride < 0) return ORACLE_EBADSHAPE;
    int64_t total = oracle_3d_out_bytes(experts, rows, cols);
    if ((out == 0 && total > 0) || (scales == 0 && experts * rows * cols > 0)) return ORACLE_EBADPTR;
    if (total == 0) return ORACLE_OK;
    int64_t padded_rows = round_up(rows, 128);
    int64_t padded_cols = round_up(cols, 4);
    memset(out, 0, (size_t)total);
    for (int64_t e = 0; e < experts; ++e) {
        uint8_t *expert_out = out + e * padded_rows * padded_cols;
        for (int64_t i = 0; i < padded_rows; ++i) {
            for (int64_t j = 0; j < padded_cols; ++j) {
                uint8_t v = 0;
                if (i < rows && j < cols) v = scales[e * expert_stride + i * ld + j];
                expert_out[blocked_byte(padded_cols, i, j)] = v;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * ---------------------------------------------------------------------------
 * MXFP8 quantisation along rows (dim0 cast) with the scales written straight
 * into the grouped blocked layout.
 *
 * The pages name this step (the dim0 and dim1 casts that produce the scales;
 * "[mxfp8 moe training] use dim1 cast cuda kernel for 3d weights by reshaping
 * to 2d", first notes and Benchmarks tables: activations A of shape
 * (16640, 5120), blocks of 32) but never state its numerics. Reading taken
 * here, the shared-scale rule of the OCP Microscaling (MX) v1.0 format for
 * MXFP8 with E4M3 elements:
 *   - a block is 32 consecutive elements of one row;
 *   - its scale is the power of two 2^s with s = floor(log2(amax)) - 8, where
 *     amax is the largest magnitude in the block and 8 is the exponent of the
 *     largest E4M3 normal (448 = 1.75 * 2^8); s is clamped to [-127, 127] and
 *     stored as the E8M0 byte s + 127. An all-zero block gets byte 0 (s = -127);
 *   - each element becomes the E4M3 (finite, "fn" variant) code nearest to
 *     x / 2^s, ties to the even code, magnitudes above 448 saturated to 448,
 *     the sign kept (a negative value that rounds to zero gives -0, code 0x80);
 *   - a block holding a NaN or an infinity gets the E8M0 NaN byte 0xFF and
 *     every element of it the E4M3 NaN code 0x7F.
 * Since a bf16 value has 8 significant bits and the factor is a power of two,
 * x / 2^s is exact in binary64 and, wherever it is not far below the smallest
 * E4M3 subnormal, in binary32 as well, so the code chosen does not depend on
 * the precision the division is carried out in.
 * ---------------------------------------------------------------------------
 */

/* Value of a finite E4M3 code: sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 holds the subnormals m/8 * 2^-6. */
double oracle_e4m3_value(int code) {
    int sign = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
    return sign ? -v : v;
}

/* Nearest E4M3 code to y (finite), ties to the even code, saturating at 448:
 * every non-negative finite code (0x00 .. 0x7E, increasing in value) is tried. */
uint8_t oracle_e4m3_encode(double y) {
    static double value[0x7F];
    static int filled = 0;
    if (!filled) {
        for (int c = 0; c <= 0x7E; ++c) value[c] = oracle_e4m3_value(c);
        filled = 1;
    }
    double a = fabs(y);
    int best = 0;
    double best_err = fabs(a - value[0]);
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs(a - value[c]);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* bf16 is the upper half of a binary32. */
static double bf16_value(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* The E8M0 byte of one block's largest magnitude (finite, >= 0). */
int oracle_e8m0_of_amax(double amax) {
    if (amax == 0.0) return 0;
    int e;
    frexp(amax, &e); /* amax = f * 2^e, 0.5 <= f < 1, so floor(log2(amax)) = e - 1 */
    int s = (e - 1) - 8;
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return s + 127;
}

/* The scale bytes alone (rows x K/32, row-major) of the same cast. */
int oracle_scales_dim0(const uint16_t *x, int64_t rows, int64_t K, int64_t ld, uint8_t *scales) {
    if (rows < 0 || K < 0 || K % 32 != 0 || ld < K) return ORACLE_EBADSHAPE;
    if (rows * K > 0 && (x == 0 || scales == 0)) return ORACLE_EBADPTR;
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t b = 0; b < K / 32; ++b) {
            const uint16_t *blk = x + i * ld + 32 * b;
            double amax = 0.0;
            int finite = 1;
            for (int k = 0; k < 32; ++k) {
                double v = bf16_value(blk[k]);
                if (isnan(v) || isinf(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            scales[i * (K / 32) + b] = finite ? (uint8_t)oracle_e8m0_of_amax(amax) : 0xFF;
        }
    }
    return ORACLE_OK;
}

/* Quantises x (rows x K bf16, row stride ld elements, K a multiple of 32) into
 * q (rows x K codes, row stride K) and scales (rows x K/32 E8M0 bytes, row-major). */
int oracle_quantize_dim0(const uint16_t *x, int64_t rows, int64_t K, int64_t ld, uint8_t *q, uint8_t *scales) {
    if (rows < 0 || K < 0 || K % 32 != 0 || ld < K) return ORACLE_EBADSHAPE;
    if (rows * K > 0 && (x == 0 || q == 0 || scales == 0)) return ORACLE_EBADPTR;
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t b = 0; b < K / 32; ++b) {
            const uint16_t *blk = x + i * ld + 32 * b;
            double amax = 0.0;
            int finite = 1;
            for (int k = 0; k < 32; ++k) {
                double v = bf16_value(blk[k]);
                if (isnan(v) || isinf(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            uint8_t *qb = q + i * K + 32 * b;
            if (!finite) {
                scales[i * (K / 32) + b] = 0xFF;
                for (int k = 0; k < 32; ++k) qb[k] = 0x7F;
                continue;
            }
            int byte = oracle_e8m0_of_amax(amax);
            scales[i * (K / 32) + b] = (uint8_t)byte;
            for (int k = 0; k < 32; ++k) {
                double y = ldexp(bf16_value(blk[k]), -(byte - 127));
                if (y > 448.0) y = 448.0;
                if (y < -448.0) y = -448.0;
                qb[k] = oracle_e4m3_encode(y);
            }
        }
    }
    return ORACLE_OK;
}

/* The dim0 cast followed by the M-groups rearrangement of its scales:
 * blocked receives oracle_M_groups_out_bytes(rows, K/32, num_groups) bytes. */
int oracle_quantize_dim0_M_groups(const uint16_t *x, int64_t rows, int64_t K, int64_t ld, const int32_t *offs,
                                  int32_t num_groups, uint8_t *q, uint8_t *blocked) {
    if (rows < 0 || K < 0 || K % 32 != 0 || ld < K) return ORACLE_EBADSHAPE;
    int64_t n = rows * (K / 32);
    uint8_t *scales = (uint8_t *)malloc(n > 0 ? (size_t)n : 1);
    if (!scales) return ORACLE_EBADPTR;
    int rc = oracle_quantize_dim0(x, rows, K, ld, q, scales);
    if (rc == ORACLE_OK) rc = oracle_M_groups(scales, rows, K / 32, K / 32, offs, num_groups, blocked);
    free(scales);
    return rc;
}

/*
 * MXFP8 cast along the token dimension (dim1 cast) for the weight-gradient
 * GEMM, whose token groups run along K ("[mxfp8 moe training] use dim1 cast
 * cuda kernel for 3d weights by reshaping to 2d", first notes: the dim1 cast
 * writes a column-major result; "Add CuTeDSL MXFP8 K-groups scale rearrange
 * kernel", review: K offsets are token offsets divided by the block size 32).
 * x is T x N bf16 (tokens x features, row stride ld elements, T a multiple
 * of 32). A block is 32 consecutive tokens of one feature column, quantised
 * by the same rule as above. Codes are written transposed: qT is N x T (row
 * n holds feature n over all tokens, row stride T), i.e. x's layout read
 * column-major; scales are N x T/32, row-major.
 */
int oracle_quantize_dim1(const uint16_t *x, int64_t T, int64_t N, int64_t ld, uint8_t *qT, uint8_t *scales) {
    if (T < 0 || N < 0 || T % 32 != 0 || ld < N) return ORACLE_EBADSHAPE;
    if (T * N > 0 && (x == 0 || qT == 0 || scales == 0)) return ORACLE_EBADPTR;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < T / 32; ++b) {
            double amax = 0.0;
            int finite = 1;
            for (int k = 0; k < 32; ++k) {
                double v = bf16_value(x[(32 * b + k) * ld + n]);
                if (isnan(v) || isinf(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            uint8_t *qb = qT + n * T + 32 * b;
            if (!finite) {
                scales[n * (T / 32) + b] = 0xFF;
                for (int k = 0; k < 32; ++k) qb[k] = 0x7F;
                continue;
            }
            int byte = oracle_e8m0_of_amax(amax);
            scales[n * (T / 32) + b] = (uint8_t)byte;
            for (int k = 0; k < 32; ++k) {
                double y = ldexp(bf16_value(x[(32 * b + k) * ld + n]), -(byte - 127));
                if (y > 448.0) y = 448.0;
                if (y < -448.0) y = -448.0;
                qb[k] = oracle_e4m3_encode(y);
            }
        }
    }
    return ORACLE_OK;
}

/* The dim1 cast followed by the K-groups rearrangement of its N x T/32 scales,
 * with group g = scale columns [offs[g-1]/32, offs[g]/32) (token offsets,
 * integer division): blocked receives oracle_K_groups_out_bytes(N, T/32, G)
 * bytes. */
int oracle_quantize_dim1_K_groups(const uint16_t *x, int64_t T, int64_t N, int64_t ld, const int32_t *offs,
                                  int32_t num_groups, uint8_t *qT, uint8_t *blocked) {
    if (T < 0 || N < 0 || T % 32 != 0 || ld < N) return ORACLE_EBADSHAPE;
    if (num_groups < 1) return ORACLE_EBADGROUPS;
    if (offs == 0) return ORACLE_EBADPTR;
    int32_t *scale_offs = (int32_t *)malloc((size_t)num_groups * sizeof(int32_t));
    int64_t n = N * (T / 32);
    uint8_t *scales = (uint8_t *)malloc(n > 0 ? (size_t)n : 1);
    int rc = ORACLE_EBADPTR;
    if (scale_offs && scales) {
        int32_t prev = 0;
        rc = ORACLE_OK;
        for (int32_t g = 0; g < num_groups; ++g) {
            if (offs[g] < prev || offs[g] > T) rc = ORACLE_EBADOFFSETS;
            prev = offs[g];
            scale_offs[g] = offs[g] / 32;
        }
        if (rc == ORACLE_OK) rc = oracle_quantize_dim1(x, T, N, ld, qT, scales);
        if (rc == ORACLE_OK) rc = oracle_K_groups(scales, N, T / 32, T / 32, scale_offs, num_groups, blocked);
    }
    free(scale_offs);
    free(scales);
    return rc;
}

/*
 * The dim1 cast of stacked expert weights ("[mxfp8 moe training] use dim1 cast
 * cuda kernel for 3d weights by reshaping to 2d", description and Next steps:
 * cast the 3-D weights along their first matrix dimension and write the codes
 * directly in per-expert column-major form; Benchmarks tables: B of shape
 * (E, 8192, 5120)). x holds E matrices of K x N bf16 (expert e at x +
 * e*expert_stride elements, rows ld elements apart, K a multiple of 32). Each
 * expert is cast exactly as oracle_quantize_dim1 casts one K x N matrix: its
 * codes, N x K (feature rows of K codes), go to q + e*N*K; its N x K/32 scale
 * bytes are laid out as oracle_3d lays out expert e: one blocked matrix of
 * round_up(N,128) x round_up(K/32,4) bytes at e times that size. blocked
 * receives oracle_3d_out_bytes(E, N, K/32) bytes.
 */
int oracle_quantize_dim1_3d(const uint16_t *x, int64_t E, int64_t K, int64_t N, int64_t expert_stride, int64_t ld,
                            uint8_t *q, uint8_t *blocked) {
    if (E < 0 || K < 0 || N < 0 || K % 32 != 0 || ld < N || expert_stride < 0) return ORACLE_EBADSHAPE;
    int64_t per = N * (K / 32);
    uint8_t *scales = (uint8_t *)malloc(E * per > 0 ? (size_t)(E * per) : 1);
    if (!scales) return ORACLE_EBADPTR;
    int rc = ORACLE_OK;
    for (int64_t e = 0; e < E && rc == ORACLE_OK; ++e)
        rc = oracle_quantize_dim1(x + e * expert_stride, K, N, ld, q + e * N * K, scales + e * per);
    if (rc == ORACLE_OK) rc = oracle_3d(scales, E, N, K / 32, per, K / 32, blocked);
    free(scales);
    return rc;
}

/* The scale bytes alone (N x T/32, row-major) of the dim1 cast. The maximum of
 * each block is accumulated row by row of x (the same maximum, in an order
 * that reads x sequentially). */
int oracle_scales_dim1(const uint16_t *x, int64_t T, int64_t N, int64_t ld, uint8_t *scales) {
    if (T < 0 || N < 0 || T % 32 != 0 || ld < N) return ORACLE_EBADSHAPE;
    if (T * N > 0 && (x == 0 || scales == 0)) return ORACLE_EBADPTR;
    double *amax = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    int *finite = (int *)malloc((size_t)(N > 0 ? N : 1) * sizeof(int));
    if (!amax || !finite) {
        free(amax);
        free(finite);
        return ORACLE_EBADPTR;
    }
    for (int64_t b = 0; b < T / 32; ++b) {
        for (int64_t n = 0; n < N; ++n) {
            amax[n] = 0.0;
            finite[n] = 1;
        }
        for (int k = 0; k < 32; ++k) {
            for (int64_t n = 0; n < N; ++n) {
                double v = bf16_value(x[(32 * b + k) * ld + n]);
                if (isnan(v) || isinf(v)) finite[n] = 0;
                else if (fabs(v) > amax[n]) amax[n] = fabs(v);
            }
        }
        for (int64_t n = 0; n < N; ++n)
            scales[n * (T / 32) + b] = finite[n] ? (uint8_t)oracle_e8m0_of_amax(amax[n]) : 0xFF;
    }
    free(amax);
    free(finite);
    return ORACLE_OK;
}

/*
 * Per-group padding of MXFP8 data rows ("Add CuTeDSL MXFP8 K-groups scale
 * rearrange kernel", its stack lists MXFP8 pad/unpad kernels by title only).
 * Reading taken here: pad places group g's rows (input rows [offs[g-1],
 * offs[g]) of a rows x cols byte matrix, row stride ld) at output rows
 * [P_g, P_g + size_g), P_g = sum over h < g of round_up(size_h, 128) — the
 * row placement of the M-groups scale layout, so that data rows line up with
 * their padded scale rows; every other byte of the (rows + 128*G) x cols
 * output (row stride cols) is zero. unpad is the inverse: output row r of
 * group g (row stride ld, cols bytes written per row) is padded row
 * P_g + (r - offs[g-1]); rows past the last end are zero.
 */
int64_t oracle_pad_M_groups_out_rows(int64_t rows, int32_t num_groups) {
    return rows + 128 * (int64_t)num_groups;
}

int oracle_pad_M_groups(const uint8_t *data, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                        int32_t num_groups, uint8_t *padded) {
    int rc = check_args(data, rows, cols, ld, offs, num_groups, padded,
                        oracle_pad_M_groups_out_rows(rows, num_groups) * cols, rows);
    if (rc != ORACLE_OK) return rc;
    int64_t total = oracle_pad_M_groups_out_rows(rows, num_groups) * cols;
    if (total > 0) memset(padded, 0, (size_t)total);
    int64_t out_row = 0, start = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t size = offs[g] - start;
        for (int64_t i = 0; i < size; ++i)
            for (int64_t j = 0; j < cols; ++j) padded[(out_row + i) * cols + j] = data[(start + i) * ld + j];
        out_row += round_up(size, 128);
        start = offs[g];
    }
    return ORACLE_OK;
}

int oracle_unpad_M_groups(const uint8_t *padded, int64_t rows, int64_t cols, const int32_t *offs, int32_t num_groups,
                          uint8_t *data, int64_t ld) {
    int64_t in_total = oracle_pad_M_groups_out_rows(rows, num_groups) * cols;
    int rc = check_args(padded, rows, cols, ld, offs, num_groups, data, rows * cols, rows);
    if (rc != ORACLE_OK) return rc;
    if (padded == 0 && in_total > 0) return ORACLE_EBADPTR;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) data[r * ld + j] = 0;
    int64_t in_row = 0, start = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t size = offs[g] - start;
        for (int64_t i = 0; i < size; ++i)
            for (int64_t j = 0; j < cols; ++j) data[(start + i) * ld + j] = padded[(in_row + i) * cols + j];
        in_row += round_up(size, 128);
        start = offs[g];
    }
    return ORACLE_OK;
}

/*
 * The inverse rearrangement: from the blocked layout written above back to the
 * row-major scale matrix (rows x cols, row stride ld; only the first cols bytes
 * of each row are written). The pages describe no such kernel; it reads every
 * byte the forward map placed from the position it placed it at, and writes
 * zeros where no group holds data (rows past the last end for M groups,
 * columns past the last end for K groups).
 */
int oracle_unrearrange_M_groups(const uint8_t *blocked, int64_t rows, int64_t cols, const int32_t *offs,
                                int32_t num_groups, uint8_t *scales, int64_t ld) {
    int rc = check_args(blocked, rows, cols, ld, offs, num_groups, scales, rows * cols, rows);
    if (rc != ORACLE_OK) return rc;
    int64_t padded_cols = round_up(cols, 4);
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) scales[i * ld + j] = 0;
    int64_t out_row = 0, group_start = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t size = offs[g] - group_start;
        for (int64_t i = 0; i < size; ++i)
            for (int64_t j = 0; j < cols; ++j)
                scales[(group_start + i) * ld + j] = blocked[blocked_byte(padded_cols, out_row + i, j)];
        out_row += round_up(size, 128);
        group_start = offs[g];
    }
    return ORACLE_OK;
}

int oracle_unrearrange_K_groups(const uint8_t *blocked, int64_t rows, int64_t cols, const int32_t *offs,
                                int32_t num_groups, uint8_t *scales, int64_t ld) {
    int rc = check_args(blocked, rows, cols, ld, offs, num_groups, scales, rows * cols, cols);
    if (rc != ORACLE_OK) return rc;
    int64_t padded_rows = round_up(rows, 128);
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) scales[i * ld + j] = 0;
    int64_t out_col = 0, group_start = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        int64_t width = offs[g] - group_start;
        int64_t padded_width = round_up(width, 4);
        const uint8_t *group_in = blocked + padded_rows * out_col;
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < width; ++j)
                scales[i * ld + group_start + j] = group_in[blocked_byte(padded_width, i, j)];
        out_col += padded_width;
        group_start = offs[g];
    }
    return ORACLE_OK;
}
