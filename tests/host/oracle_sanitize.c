/*
 * Drives every exported function of the CPU oracle (oracle/convrot_oracle.c,
 * test infrastructure) on small seeded inputs and on its edge cases (empty
 * batches, group sizes 1 and 256, odd shapes, rejected arguments), so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer sees every
 * buffer the oracle touches.  Also checks a few facts that hold for any
 * input (code ranges, the packed int4 round trip, the GEMM against a direct
 * sum).  Exit status 0 when every check holds and no sanitizer fired.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's exports (it has no header: its Python binding declares them). */
void oracle_hadamard(int g, double *H);
int oracle_rotate_rows(const double *x, int64_t rows, int64_t K, int g, double *out);
int oracle_quantize_weight_i8(const float *w, int64_t N, int64_t K, int g, int8_t *wq, float *scale);
int oracle_rotate_quant(const uint16_t *x, int64_t M, int64_t K, int g, int8_t *xq, float *x_scale);
int oracle_gemm_i8(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc);
int oracle_epilogue(const int32_t *acc, const float *x_scale, const float *w_scale, int64_t M, int64_t N,
                    uint16_t *y);
int oracle_w8a8_linear(const uint16_t *x, int64_t M, int64_t K, const int8_t *wq, const float *w_scale,
                       int64_t N, int g, uint16_t *y);
int oracle_quantize_weight_i4_ex(const float *w, int64_t N, int64_t K, int g, const int32_t *force_index,
                                 uint8_t *wq4, float *scale, int32_t *clip_index, double *errors);
int oracle_quantize_weight_i4(const float *w, int64_t N, int64_t K, int g, uint8_t *wq4, float *scale,
                              int32_t *clip_index);
int oracle_unpack_i4(const uint8_t *wq4, int64_t N, int64_t K, int8_t *wq);
int oracle_w4a8_linear(const uint16_t *x, int64_t M, int64_t K, const uint8_t *wq4, const float *w_scale,
                       int64_t N, int g, uint16_t *y);
int oracle_rmsnorm_bf16(const uint16_t *x, const float *w, float eps, int64_t M, int64_t K, uint16_t *y);
int oracle_rmsnorm_rotate_quant(const uint16_t *x, const float *w, float eps, int64_t M, int64_t K, int g,
                                int8_t *xq, float *x_scale, uint16_t *y_norm);
int oracle_dequantize_weight(const int8_t *wq, const float *w_scale, int64_t N, int64_t K, int g,
                             uint16_t *w_out);
int oracle_gemm_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K, uint16_t *y);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

static int failures = 0;
#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);    \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

/* splitmix64: seeded inputs only (none of the method's arithmetic). */
static uint64_t rng_state = 0x243f6a8885a308d3ull;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static float next_normalish(void) { /* sum of four uniforms, centred */
  double s = 0.0;
  for (int i = 0; i < 4; ++i) s += (double)(next_u64() >> 11) * 0x1p-53;
  return (float)(s - 2.0);
}
static uint16_t to_bf16_trunc(float f) { /* an input generator: any bf16 pattern will do */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void *xmalloc(size_t n) { /* exact sizes: ASan sees one byte past the end */
  void *p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static void run_shape(int64_t M, int64_t N, int64_t K, int g) {
  uint16_t *x = xmalloc(sizeof(uint16_t) * (size_t)(M * K));
  float *w = xmalloc(sizeof(float) * (size_t)(N * K));
  float *nw = xmalloc(sizeof(float) * (size_t)K);
  for (int64_t i = 0; i < M * K; ++i) x[i] = to_bf16_trunc(next_normalish() * (i % 97 == 0 ? 40.f : 1.f));
  for (int64_t i = 0; i < N * K; ++i) w[i] = next_normalish() * 0.05f;
  for (int64_t i = 0; i < K; ++i) nw[i] = next_normalish() * 0.1f;
  if (M > 1) memset(x + K, 0, sizeof(uint16_t) * (size_t)K); /* an all-zero token */

  int8_t *wq = xmalloc((size_t)(N * K));
  float *ws = xmalloc(sizeof(float) * (size_t)N);
  CHECK(oracle_quantize_weight_i8(w, N, K, g, wq, ws) == 0);
  for (int64_t i = 0; i < N * K; ++i) CHECK(wq[i] >= -127 && wq[i] <= 127);

  int8_t *xq = xmalloc((size_t)(M * K));
  float *xs = xmalloc(sizeof(float) * (size_t)M);
  CHECK(oracle_rotate_quant(x, M, K, g, xq, xs) == 0);
  for (int64_t i = 0; i < M * K; ++i) CHECK(xq[i] >= -127 && xq[i] <= 127);
  if (M > 1) CHECK(xs[1] == 0.0f);

  int32_t *acc = xmalloc(sizeof(int32_t) * (size_t)(M * N));
  CHECK(oracle_gemm_i8(xq, wq, M, N, K, acc) == 0);
  for (int64_t m = 0; m < M; m += (M > 3 ? M / 3 : 1))
    for (int64_t n = 0; n < N; n += (N > 3 ? N / 3 : 1)) {
      int64_t s = 0;
      for (int64_t k = 0; k < K; ++k) s += (int64_t)xq[m * K + k] * wq[n * K + k];
      CHECK(acc[m * N + n] == (int32_t)s);
    }
  uint16_t *y = xmalloc(sizeof(uint16_t) * (size_t)(M * N));
  uint16_t *y2 = xmalloc(sizeof(uint16_t) * (size_t)(M * N));
  CHECK(oracle_epilogue(acc, xs, ws, M, N, y) == 0);
  CHECK(oracle_w8a8_linear(x, M, K, wq, ws, N, g, y2) == 0);
  CHECK(memcmp(y, y2, sizeof(uint16_t) * (size_t)(M * N)) == 0);

  if (K % 2 == 0) {
    uint8_t *wq4 = xmalloc((size_t)(N * K / 2));
    float *ws4 = xmalloc(sizeof(float) * (size_t)N);
    int32_t *ci = xmalloc(sizeof(int32_t) * (size_t)N);
    int32_t *force = xmalloc(sizeof(int32_t) * (size_t)N);
    double *err = xmalloc(sizeof(double) * (size_t)N * 51); /* every candidate of every row */
    int8_t *wu = xmalloc((size_t)(N * K));
    CHECK(oracle_quantize_weight_i4(w, N, K, g, wq4, ws4, ci) == 0);
    for (int64_t n = 0; n < N; ++n) {
      CHECK(ci[n] >= 0 && ci[n] <= 50);
      force[n] = (int32_t)(n % 51);
    }
    CHECK(oracle_unpack_i4(wq4, N, K, wu) == 0);
    for (int64_t i = 0; i < N * K; ++i) CHECK(wu[i] >= -8 && wu[i] <= 7);
    CHECK(oracle_quantize_weight_i4_ex(w, N, K, g, force, wq4, ws4, ci, err) == 0);
    for (int64_t n = 0; n < N; ++n) CHECK(ci[n] == force[n] && err[n * 51 + force[n]] >= 0.0);
    CHECK(oracle_w4a8_linear(x, M, K, wq4, ws4, N, g, y) == 0);
    force[0] = 51;
    CHECK(oracle_quantize_weight_i4_ex(w, N, K, g, force, wq4, ws4, ci, err) != 0);
    uint16_t *wd = xmalloc(sizeof(uint16_t) * (size_t)(N * K));
    CHECK(oracle_dequantize_weight(wu, ws4, N, K, g, wd) == 0);
    free(wd);
    free(wq4); free(ws4); free(ci); free(force); free(err); free(wu);
  }

  uint16_t *yn = xmalloc(sizeof(uint16_t) * (size_t)(M * K));
  uint16_t *yn2 = xmalloc(sizeof(uint16_t) * (size_t)(M * K));
  CHECK(oracle_rmsnorm_bf16(x, nw, 1e-6f, M, K, yn) == 0);
  CHECK(oracle_rmsnorm_rotate_quant(x, nw, 1e-6f, M, K, g, xq, xs, yn2) == 0);
  CHECK(memcmp(yn, yn2, sizeof(uint16_t) * (size_t)(M * K)) == 0);
  CHECK(oracle_rmsnorm_rotate_quant(x, nw, 1e-6f, M, K, g, xq, xs, NULL) != 0); /* the norm output is required */

  uint16_t *wd = xmalloc(sizeof(uint16_t) * (size_t)(N * K));
  CHECK(oracle_dequantize_weight(wq, ws, N, K, g, wd) == 0);
  CHECK(oracle_gemm_bf16(x, wd, M, N, K, y) == 0);

  double *xr = xmalloc(sizeof(double) * (size_t)(M * K));
  double *xo = xmalloc(sizeof(double) * (size_t)(M * K));
  for (int64_t i = 0; i < M * K; ++i) xr[i] = next_normalish();
  CHECK(oracle_rotate_rows(xr, M, K, g, xo) == 0);

  free(xr); free(xo); free(wd); free(yn); free(yn2);
  free(x); free(w); free(nw); free(wq); free(ws); free(xq); free(xs); free(acc); free(y); free(y2);
}

int main(void) {
  oracle_set_num_threads(2);
  CHECK(oracle_num_threads() >= 1);

  double *H = xmalloc(sizeof(double) * 256 * 256);
  oracle_hadamard(256, H);
  CHECK(fabs(H[0] - 1.0 / 16.0) == 0.0 && H[256 + 1] == -1.0 / 16.0);
  oracle_hadamard(1, H);
  CHECK(H[0] == 1.0);
  free(H);

  run_shape(5, 7, 512, 256);  /* ragged M and N, two groups */
  run_shape(3, 4, 48, 16);    /* group 16 */
  run_shape(2, 3, 6, 1);      /* group 1 */
  run_shape(1, 1, 256, 256);  /* one token, one row */
  run_shape(4, 2, 24, 8);     /* three groups of 8 */

  /* empty batches are no-ops */
  uint16_t xb[256] = {0}, yb[256] = {0};
  int8_t qb[256] = {0};
  float sb[4] = {0}, wb[256] = {0};
  uint8_t pb[128] = {0};
  CHECK(oracle_rotate_quant(xb, 0, 256, 256, qb, sb) == 0);
  CHECK(oracle_w8a8_linear(xb, 0, 256, qb, sb, 4, 256, yb) == 0);
  CHECK(oracle_w8a8_linear(xb, 1, 256, qb, sb, 0, 256, yb) == 0);
  CHECK(oracle_w4a8_linear(xb, 0, 256, pb, sb, 1, 256, yb) == 0);
  CHECK(oracle_gemm_i8(qb, qb, 0, 0, 256, (int32_t *)wb) == 0);
  CHECK(oracle_quantize_weight_i8(wb, 0, 256, 256, qb, sb) == 0);

  /* rejected arguments leave the buffers alone */
  CHECK(oracle_rotate_quant(NULL, 1, 256, 256, qb, sb) != 0);
  CHECK(oracle_rotate_quant(xb, 1, 250, 256, qb, sb) != 0);
  CHECK(oracle_rotate_quant(xb, 1, 256, 3, qb, sb) != 0);
  CHECK(oracle_rotate_quant(xb, -1, 256, 256, qb, sb) != 0);
  CHECK(oracle_quantize_weight_i4(wb, 1, 255, 1, pb, sb, NULL) != 0);
  CHECK(oracle_unpack_i4(pb, 1, 7, qb) != 0);
  CHECK(oracle_rmsnorm_bf16(xb, wb, -1.0f, 1, 256, yb) != 0);
  CHECK(oracle_gemm_bf16(xb, xb, 1, 1, 0, yb) != 0);
  CHECK(oracle_dequantize_weight(qb, sb, 1, 256, 5, yb) != 0);

  if (failures) {
    fprintf(stderr, "%d oracle checks failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer checks passed\n");
  return 0;
}
