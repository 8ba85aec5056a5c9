/*
 * The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built by tests/test_oracle_sanitize.py with gcc -fsanitize=address,undefined
 * -fno-sanitize-recover=all, linked with oracle/mx_rearrange_oracle.c itself
 * (not its shared library), and run on the CPU. Every buffer is a heap block of
 * exactly the size the call needs, so a read or write one byte outside it
 * stops the program. Each entry point runs over edge shapes (empty, one row,
 * ragged tiles, strided rows, many and empty groups, offsets short of the
 * total, non-finite inputs) and its error paths; rearrangements are also
 * undone by their inverses and compared with the input. Prints "ok" and exits
 * 0 when every check holds.
 */

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_M_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups);
int64_t oracle_K_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups);
int oracle_M_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                    int32_t num_groups, uint8_t *out);
int oracle_K_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                    int32_t num_groups, uint8_t *out);
int oracle_M_groups_threads(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                            int32_t num_groups, uint8_t *out, int threads);
int oracle_K_groups_threads(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                            int32_t num_groups, uint8_t *out, int threads);
int64_t oracle_3d_out_bytes(int64_t experts, int64_t rows, int64_t cols);
int oracle_3d(const uint8_t *scales, int64_t experts, int64_t rows, int64_t cols, int64_t expert_stride, int64_t ld,
              uint8_t *out);
double oracle_e4m3_value(int code);
uint8_t oracle_e4m3_encode(double y);
int oracle_e8m0_of_amax(double amax);
int oracle_scales_dim0(const uint16_t *x, int64_t rows, int64_t K, int64_t ld, uint8_t *scales);
int oracle_quantize_dim0(const uint16_t *x, int64_t rows, int64_t K, int64_t ld, uint8_t *q, uint8_t *scales);
int oracle_quantize_dim0_M_groups(const uint16_t *x, int64_t rows, int64_t K, int64_t ld, const int32_t *offs,
                                  int32_t num_groups, uint8_t *q, uint8_t *blocked);
int oracle_quantize_dim1(const uint16_t *x, int64_t T, int64_t N, int64_t ld, uint8_t *qT, uint8_t *scales);
int oracle_quantize_dim1_K_groups(const uint16_t *x, int64_t T, int64_t N, int64_t ld, const int32_t *offs,
                                  int32_t num_groups, uint8_t *qT, uint8_t *blocked);
int oracle_quantize_dim1_3d(const uint16_t *x, int64_t E, int64_t K, int64_t N, int64_t expert_stride, int64_t ld,
                            uint8_t *q, uint8_t *blocked);
int oracle_scales_dim1(const uint16_t *x, int64_t T, int64_t N, int64_t ld, uint8_t *scales);
int64_t oracle_pad_M_groups_out_rows(int64_t rows, int32_t num_groups);
int oracle_pad_M_groups(const uint8_t *data, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                        int32_t num_groups, uint8_t *padded);
int oracle_unpad_M_groups(const uint8_t *padded, int64_t rows, int64_t cols, const int32_t *offs,
                          int32_t num_groups, uint8_t *data, int64_t ld);
int oracle_unrearrange_M_groups(const uint8_t *blocked, int64_t rows, int64_t cols, const int32_t *offs,
                                int32_t num_groups, uint8_t *scales, int64_t ld);
int oracle_unrearrange_K_groups(const uint8_t *blocked, int64_t rows, int64_t cols, const int32_t *offs,
                                int32_t num_groups, uint8_t *scales, int64_t ld);

static int failures = 0;
#define CHECK(cond, ...)                              \
    do {                                              \
        if (!(cond)) {                                \
            fprintf(stderr, "check failed: " __VA_ARGS__); \
            fprintf(stderr, "\n");                    \
            ++failures;                               \
        }                                             \
    } while (0)

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 33);
}
static int64_t below(int64_t n) { return n > 0 ? (int64_t)(next_u32() % (uint64_t)n) : 0; }

/* A heap block of exactly n bytes (one byte when n is 0, never touched then). */
static void *exact(int64_t n) {
    void *p = malloc(n > 0 ? (size_t)n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int64_t span(int64_t rows, int64_t cols, int64_t ld) { return rows > 0 && cols > 0 ? (rows - 1) * ld + cols : 0; }

/* Non-decreasing cumulative ends in [0, total]; the last equals total unless `short_total`. */
static void random_offsets(int32_t *offs, int32_t G, int64_t total, int short_total, int multiple) {
    for (int32_t g = 0; g < G; ++g) offs[g] = (int32_t)(below(total / multiple + 1) * multiple);
    for (int32_t g = 1; g < G; ++g)
        for (int32_t h = g; h > 0 && offs[h] < offs[h - 1]; --h) {
            int32_t t = offs[h];
            offs[h] = offs[h - 1];
            offs[h - 1] = t;
        }
    if (!short_total) offs[G - 1] = (int32_t)total;
}

static uint16_t random_bf16(void) {
    uint32_t r = next_u32();
    switch (r % 16) {
    case 0: return 0x7f80;               /* +inf */
    case 1: return 0xffc1;               /* NaN */
    case 2: return (uint16_t)(r >> 16) & 0x007f; /* subnormal or zero */
    case 3: return 0x8000;               /* -0 */
    default: return (uint16_t)(0x3000 + (r >> 20) % 0x2000) | (uint16_t)((r & 0x10) << 11);
    }
}

static void rearrange_cases(void) {
    static const int64_t rows_set[] = {0, 1, 5, 127, 128, 129, 300};
    static const int64_t cols_set[] = {0, 1, 3, 4, 5, 44, 129};
    static const int32_t groups_set[] = {1, 2, 3, 8, 70};
    for (int kind = 0; kind < 2; ++kind)
        for (size_t a = 0; a < sizeof rows_set / sizeof *rows_set; ++a)
            for (size_t b = 0; b < sizeof cols_set / sizeof *cols_set; ++b)
                for (size_t c = 0; c < sizeof groups_set / sizeof *groups_set; ++c) {
                    int64_t rows = rows_set[a], cols = cols_set[b];
                    int32_t G = groups_set[c];
                    int64_t ld = cols + (int64_t)(below(2) * 3);
                    int short_total = below(4) == 0;
                    int64_t total = kind == 0 ? rows : cols;
                    int32_t *offs = exact(4 * (int64_t)G);
                    random_offsets(offs, G, total, short_total, 1);
                    int64_t n_in = span(rows, cols, ld);
                    uint8_t *in = exact(n_in);
                    for (int64_t i = 0; i < n_in; ++i) in[i] = (uint8_t)(1 + below(255));
                    int64_t n_out = kind == 0 ? oracle_M_groups_out_bytes(rows, cols, G)
                                              : oracle_K_groups_out_bytes(rows, cols, G);
                    uint8_t *out = exact(n_out);
                    int rc = kind == 0 ? oracle_M_groups(in, rows, cols, ld, offs, G, out)
                                       : oracle_K_groups(in, rows, cols, ld, offs, G, out);
                    CHECK(rc == 0, "%s rearrange rows %lld cols %lld G %d: rc %d", kind ? "K" : "M",
                          (long long)rows, (long long)cols, G, rc);
                    /* the same call shared among threads writes the same bytes */
                    uint8_t *par = exact(n_out);
                    int threads = 1 + (int)below(5);
                    rc = kind == 0 ? oracle_M_groups_threads(in, rows, cols, ld, offs, G, par, threads)
                                   : oracle_K_groups_threads(in, rows, cols, ld, offs, G, par, threads);
                    CHECK(rc == 0 && (n_out == 0 || memcmp(par, out, (size_t)n_out) == 0),
                          "%s threaded rearrange rows %lld cols %lld G %d threads %d: rc %d", kind ? "K" : "M",
                          (long long)rows, (long long)cols, G, threads, rc);
                    free(par);
                    /* the inverse restores every byte that lies in a group; the rest comes back zero */
                    uint8_t *back = exact(rows * cols);
                    rc = kind == 0 ? oracle_unrearrange_M_groups(out, rows, cols, offs, G, back, cols)
                                   : oracle_unrearrange_K_groups(out, rows, cols, offs, G, back, cols);
                    CHECK(rc == 0, "%s inverse: rc %d", kind ? "K" : "M", rc);
                    int64_t covered = offs[G - 1];
                    for (int64_t i = 0; i < rows; ++i)
                        for (int64_t j = 0; j < cols; ++j) {
                            int inside = kind == 0 ? i < covered : j < covered;
                            uint8_t want = inside ? in[i * ld + j] : 0;
                            if (back[i * cols + j] != want) {
                                CHECK(0, "%s round trip rows %lld cols %lld G %d at (%lld, %lld)", kind ? "K" : "M",
                                      (long long)rows, (long long)cols, G, (long long)i, (long long)j);
                                i = rows;
                                break;
                            }
                        }
                    free(back);
                    free(out);
                    free(in);
                    free(offs);
                }
    /* error paths: nothing is read or written */
    int32_t offs[2] = {3, 1};
    uint8_t one = 0;
    CHECK(oracle_M_groups(&one, 4, 1, 1, offs, 2, &one) == -6, "decreasing offsets");
    CHECK(oracle_M_groups(&one, 4, 1, 1, 0, 2, &one) == -1, "null offsets");
    CHECK(oracle_K_groups(&one, 1, 4, 3, offs, 1, &one) == -2, "stride below width");
    CHECK(oracle_K_groups(&one, 1, 4, 4, offs, 0, &one) == -3, "no groups");
}

static void experts_cases(void) {
    static const int64_t e_set[] = {0, 1, 3};
    static const int64_t rows_set[] = {0, 1, 129};
    static const int64_t cols_set[] = {0, 3, 160};
    for (size_t a = 0; a < 3; ++a)
        for (size_t b = 0; b < 3; ++b)
            for (size_t c = 0; c < 3; ++c)
                for (int stride_kind = 0; stride_kind < 3; ++stride_kind) {
                    int64_t E = e_set[a], rows = rows_set[b], cols = cols_set[c], ld = cols + 1;
                    int64_t one = span(rows, cols, ld);
                    int64_t es = stride_kind == 0 ? one : stride_kind == 1 ? one + 5 : 0;
                    int64_t n_in = E > 0 && one > 0 ? (E - 1) * es + one : 0;
                    uint8_t *in = exact(n_in);
                    for (int64_t i = 0; i < n_in; ++i) in[i] = (uint8_t)next_u32();
                    int64_t n_out = oracle_3d_out_bytes(E, rows, cols);
                    uint8_t *out = exact(n_out);
                    CHECK(oracle_3d(in, E, rows, cols, es, ld, out) == 0, "3d E %lld rows %lld cols %lld",
                          (long long)E, (long long)rows, (long long)cols);
                    free(out);
                    free(in);
                }
}

static void quantize_cases(void) {
    static const int64_t rows_set[] = {0, 1, 3, 130};
    static const int64_t k_set[] = {0, 32, 64, 96};
    for (size_t a = 0; a < 4; ++a)
        for (size_t b = 0; b < 4; ++b)
            for (int padded = 0; padded < 2; ++padded) {
                int64_t rows = rows_set[a], K = k_set[b], ld = K + 8 * padded;
                int64_t n_x = span(rows, K, ld);
                uint16_t *x = exact(2 * n_x);
                for (int64_t i = 0; i < n_x; ++i) x[i] = random_bf16();
                uint8_t *q = exact(rows * K), *s = exact(rows * (K / 32)), *s2 = exact(rows * (K / 32));
                CHECK(oracle_quantize_dim0(x, rows, K, ld, q, s) == 0, "dim0 rows %lld K %lld", (long long)rows,
                      (long long)K);
                CHECK(oracle_scales_dim0(x, rows, K, ld, s2) == 0, "dim0 scales");
                CHECK(rows * (K / 32) == 0 || memcmp(s, s2, (size_t)(rows * (K / 32))) == 0, "dim0 scales agree");
                for (int32_t G = 1; G <= 9; G += 8) {
                    int32_t *offs = exact(4 * (int64_t)G);
                    random_offsets(offs, G, rows, below(3) == 0, 1);
                    uint8_t *qg = exact(rows * K), *blk = exact(oracle_M_groups_out_bytes(rows, K / 32, G));
                    CHECK(oracle_quantize_dim0_M_groups(x, rows, K, ld, offs, G, qg, blk) == 0, "dim0 M groups");
                    CHECK(rows * K == 0 || memcmp(q, qg, (size_t)(rows * K)) == 0, "dim0 codes agree");
                    free(blk);
                    free(qg);
                    free(offs);
                }
                free(s2);
                free(s);
                free(q);
                free(x);
            }
    static const int64_t t_set[] = {0, 32, 64, 160};
    static const int64_t n_set[] = {0, 1, 3, 40};
    for (size_t a = 0; a < 4; ++a)
        for (size_t b = 0; b < 4; ++b) {
            int64_t T = t_set[a], N = n_set[b], ld = N + 5;
            int64_t n_x = span(T, N, ld);
            uint16_t *x = exact(2 * n_x);
            for (int64_t i = 0; i < n_x; ++i) x[i] = random_bf16();
            uint8_t *qT = exact(N * T), *s = exact(N * (T / 32)), *s2 = exact(N * (T / 32));
            CHECK(oracle_quantize_dim1(x, T, N, ld, qT, s) == 0, "dim1 T %lld N %lld", (long long)T, (long long)N);
            CHECK(oracle_scales_dim1(x, T, N, ld, s2) == 0, "dim1 scales");
            CHECK(N * (T / 32) == 0 || memcmp(s, s2, (size_t)(N * (T / 32))) == 0, "dim1 scales agree");
            for (int32_t G = 1; G <= 9; G += 8) {
                int32_t *offs = exact(4 * (int64_t)G);
                random_offsets(offs, G, T, below(3) == 0, below(2) ? 32 : 1);
                uint8_t *qg = exact(N * T), *blk = exact(oracle_K_groups_out_bytes(N, T / 32, G));
                CHECK(oracle_quantize_dim1_K_groups(x, T, N, ld, offs, G, qg, blk) == 0, "dim1 K groups");
                free(blk);
                free(qg);
                free(offs);
            }
            free(s2);
            free(s);
            free(qT);
            free(x);
        }
    for (int64_t E = 0; E <= 2; ++E)
        for (int64_t K = 0; K <= 64; K += 32)
            for (int64_t N = 1; N <= 5; N += 4) {
                int64_t ld = N + 3, one = span(K, N, ld), es = one + 7;
                int64_t n_x = E > 0 && one > 0 ? (E - 1) * es + one : 0;
                uint16_t *x = exact(2 * (n_x > 0 ? n_x : 1));
                for (int64_t i = 0; i < n_x; ++i) x[i] = random_bf16();
                uint8_t *q = exact(E * N * K), *blk = exact(oracle_3d_out_bytes(E, N, K / 32));
                CHECK(oracle_quantize_dim1_3d(x, E, K, N, es, ld, q, blk) == 0, "dim1 3d E %lld K %lld N %lld",
                      (long long)E, (long long)K, (long long)N);
                free(blk);
                free(q);
                free(x);
            }
    /* the scalar rules over their whole ranges */
    for (int c = 0; c < 0x7f; ++c) CHECK(oracle_e4m3_encode(oracle_e4m3_value(c)) == c, "e4m3 code %d", c);
    CHECK(oracle_e4m3_encode(1e30) == 0x7e && oracle_e4m3_encode(-1e30) == 0xfe, "e4m3 saturation");
    CHECK(oracle_e8m0_of_amax(0.0) == 0 && oracle_e8m0_of_amax(1e300) == 254 && oracle_e8m0_of_amax(1e-300) == 0,
          "e8m0 clamps");
}

static void pad_cases(void) {
    static const int64_t rows_set[] = {0, 1, 129, 300};
    static const int64_t cols_set[] = {1, 7, 64};
    for (size_t a = 0; a < 4; ++a)
        for (size_t b = 0; b < 3; ++b)
            for (int32_t G = 1; G <= 9; G += 4) {
                int64_t rows = rows_set[a], cols = cols_set[b], ld = cols + 2;
                int32_t *offs = exact(4 * (int64_t)G);
                random_offsets(offs, G, rows, 0, 1);
                int64_t n_in = span(rows, cols, ld);
                uint8_t *in = exact(n_in);
                for (int64_t i = 0; i < n_in; ++i) in[i] = (uint8_t)next_u32();
                int64_t n_pad = oracle_pad_M_groups_out_rows(rows, G) * cols;
                uint8_t *pad = exact(n_pad), *back = exact(rows * cols);
                CHECK(oracle_pad_M_groups(in, rows, cols, ld, offs, G, pad) == 0, "pad");
                CHECK(oracle_unpad_M_groups(pad, rows, cols, offs, G, back, cols) == 0, "unpad");
                for (int64_t i = 0; i < rows; ++i)
                    CHECK(memcmp(back + i * cols, in + i * ld, (size_t)cols) == 0, "pad round trip row %lld",
                          (long long)i);
                free(back);
                free(pad);
                free(in);
                free(offs);
            }
}

int main(void) {
    rearrange_cases();
    experts_cases();
    quantize_cases();
    pad_cases();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
