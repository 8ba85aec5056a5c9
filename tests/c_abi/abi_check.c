/*
 * A plain C caller of the library: no Python, no torch. It allocates device
 * memory with the HIP runtime, calls the C entry points declared in the include/ headers
 * on a stream of its own, copies the results back and compares them byte for
 * byte with the C oracle (test infrastructure, linked only into this checker).
 * Exit status 0 when every case matches and the error cases return the
 * documented status codes.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mx_rearrange.h"

/* oracle (oracle/mx_rearrange_oracle.c) */
int64_t oracle_M_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups);
int64_t oracle_K_groups_out_bytes(int64_t rows, int64_t cols, int32_t num_groups);
int oracle_M_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                    int32_t num_groups, uint8_t *out);
int oracle_K_groups(const uint8_t *scales, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs,
                    int32_t num_groups, uint8_t *out);
int oracle_unrearrange_M_groups(const uint8_t *blocked, int64_t rows, int64_t cols, const int32_t *offs,
                                int32_t num_groups, uint8_t *scales, int64_t ld);
int oracle_unrearrange_K_groups(const uint8_t *blocked, int64_t rows, int64_t cols, const int32_t *offs,
                                int32_t num_groups, uint8_t *scales, int64_t ld);

static int failures = 0;

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(2);                                                                    \
    }                                                                             \
  } while (0)

static void fill(uint8_t *p, size_t n, uint32_t seed) {
  uint32_t x = seed;
  for (size_t i = 0; i < n; ++i) {
    x = x * 1664525u + 1013904223u;
    p[i] = (uint8_t)(x >> 24);
  }
}

static void compare(const char *label, const uint8_t *got, const uint8_t *want, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    if (got[i] != want[i]) {
      printf("%s: MISMATCH at byte %zu of %zu (got %u want %u)\n", label, i, n, got[i], want[i]);
      ++failures;
      return;
    }
  }
  printf("%s: ok (%zu bytes)\n", label, n);
}

/* forward rearrangement, then the inverse of the oracle's blocked bytes */
static void run_case(int kgroups, int64_t rows, int64_t cols, int64_t ld, const int32_t *offs, int32_t G,
                     hipStream_t s) {
  char label[96];
  const size_t in_n = (size_t)(rows * ld);
  const int64_t out_n = kgroups ? mx_rearrange_K_groups_out_bytes(rows, cols, G)
                                : mx_rearrange_M_groups_out_bytes(rows, cols, G);
  const int64_t want_n = kgroups ? oracle_K_groups_out_bytes(rows, cols, G) : oracle_M_groups_out_bytes(rows, cols, G);
  snprintf(label, sizeof label, "%s rows %lld cols %lld ld %lld G %d", kgroups ? "K" : "M", (long long)rows,
           (long long)cols, (long long)ld, G);
  if (out_n != want_n) {
    printf("%s: size %lld, oracle %lld\n", label, (long long)out_n, (long long)want_n);
    ++failures;
    return;
  }
  uint8_t *h_in = malloc(in_n), *h_out = malloc((size_t)out_n), *h_want = malloc((size_t)out_n);
  uint8_t *h_back = malloc((size_t)(rows * cols)), *h_back_want = malloc((size_t)(rows * cols));
  fill(h_in, in_n, (uint32_t)(rows * 131 + cols));
  uint8_t *d_in, *d_out, *d_back;
  int32_t *d_offs;
  HIP_OK(hipMalloc((void **)&d_in, in_n));
  HIP_OK(hipMalloc((void **)&d_out, (size_t)out_n));
  HIP_OK(hipMalloc((void **)&d_back, (size_t)(rows * cols)));
  HIP_OK(hipMalloc((void **)&d_offs, sizeof(int32_t) * (size_t)G));
  HIP_OK(hipMemcpy(d_in, h_in, in_n, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_offs, offs, sizeof(int32_t) * (size_t)G, hipMemcpyHostToDevice));

  int rc = kgroups ? mx_block_rearrange_K_groups(d_in, rows, cols, ld, d_offs, G, d_out, s)
                   : mx_block_rearrange_M_groups(d_in, rows, cols, ld, d_offs, G, d_out, s);
  if (rc != MX_REARRANGE_OK) {
    printf("%s: status %d (%s)\n", label, rc, mx_rearrange_strerror(rc));
    ++failures;
  }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(h_out, d_out, (size_t)out_n, hipMemcpyDeviceToHost));
  if (kgroups)
    oracle_K_groups(h_in, rows, cols, ld, offs, G, h_want);
  else
    oracle_M_groups(h_in, rows, cols, ld, offs, G, h_want);
  compare(label, h_out, h_want, (size_t)out_n);

  /* inverse: the device reads the oracle's blocked bytes back into a packed matrix */
  HIP_OK(hipMemcpy(d_out, h_want, (size_t)out_n, hipMemcpyHostToDevice));
  rc = kgroups ? mx_block_unrearrange_K_groups(d_out, rows, cols, d_offs, G, d_back, cols, s)
               : mx_block_unrearrange_M_groups(d_out, rows, cols, d_offs, G, d_back, cols, s);
  if (rc != MX_REARRANGE_OK) {
    printf("%s inverse: status %d (%s)\n", label, rc, mx_rearrange_strerror(rc));
    ++failures;
  }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(h_back, d_back, (size_t)(rows * cols), hipMemcpyDeviceToHost));
  if (kgroups)
    oracle_unrearrange_K_groups(h_want, rows, cols, offs, G, h_back_want, cols);
  else
    oracle_unrearrange_M_groups(h_want, rows, cols, offs, G, h_back_want, cols);
  strncat(label, " inverse", sizeof label - strlen(label) - 1);
  compare(label, h_back, h_back_want, (size_t)(rows * cols));

  HIP_OK(hipFree(d_in));
  HIP_OK(hipFree(d_out));
  HIP_OK(hipFree(d_back));
  HIP_OK(hipFree(d_offs));
  free(h_in);
  free(h_out);
  free(h_want);
  free(h_back);
  free(h_back_want);
}

int main(void) {
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  const int32_t m_offs[] = {130, 130, 383, 700, 1000};
  const int32_t k_offs[] = {7, 7, 30, 45};
  const int32_t k_wide[] = {186, 3840, 4097};
  run_case(0, 1000, 44, 44, m_offs, 5, s);
  run_case(0, 1000, 45, 53, m_offs, 5, s);
  run_case(1, 300, 45, 45, k_offs, 4, s);
  run_case(1, 257, 4097, 4101, k_wide, 3, s);

  /* documented error returns, nothing enqueued */
  uint8_t *d_buf;
  int32_t *d_offs;
  HIP_OK(hipMalloc((void **)&d_buf, 1 << 16));
  HIP_OK(hipMalloc((void **)&d_offs, 64));
  struct { const char *what; int got, want; } errs[] = {
      {"offsets NULL", mx_block_rearrange_M_groups(d_buf, 4, 4, 4, NULL, 1, d_buf + 4096, s), MX_REARRANGE_ENULL},
      {"row stride < cols", mx_block_rearrange_M_groups(d_buf, 4, 8, 4, d_offs, 1, d_buf + 4096, s), MX_REARRANGE_ESHAPE},
      {"no groups", mx_block_rearrange_K_groups(d_buf, 4, 4, 4, d_offs, 0, d_buf + 4096, s), MX_REARRANGE_EGROUPS},
      {"out misaligned", mx_block_rearrange_K_groups(d_buf, 4, 4, 4, d_offs, 1, d_buf + 4100, s), MX_REARRANGE_EALIGN},
  };
  for (size_t i = 0; i < sizeof errs / sizeof errs[0]; ++i) {
    if (errs[i].got != errs[i].want) {
      printf("error case %s: status %d, want %d\n", errs[i].what, errs[i].got, errs[i].want);
      ++failures;
    } else {
      printf("error case %s: %d (%s)\n", errs[i].what, errs[i].got, mx_rearrange_strerror(errs[i].got));
    }
  }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipFree(d_buf));
  HIP_OK(hipFree(d_offs));
  HIP_OK(hipStreamDestroy(s));
  printf(failures ? "FAILED: %d\n" : "all ok\n", failures);
  return failures ? 1 : 0;
}
