/*
 * Links against libconvrot.so from plain C (no C++, no Python) through
 * include/convrot.h and exercises the calls that need no GPU: the version,
 * the status strings, the workspace sizes, and argument validation (every
 * call below is rejected, or is an empty no-op, before anything would be
 * enqueued).  Exit status 0 when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "convrot.h"

static int failures = 0;

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                \
    }                                                            \
  } while (0)

int main(void) {
  /* fake, aligned, never dereferenced addresses */
  void *a = (void *)0x10000, *b = (void *)0x20000, *c = (void *)0x30000, *d = (void *)0x40000;
  void *mis = (void *)0x10008;
  hipStream_t s0 = 0;

  CHECK(convrot_version() >= 103);
  CHECK(strcmp(convrot_status_string(CONVROT_OK), "ok") == 0);
  for (int st = CONVROT_OK; st <= CONVROT_ERR_ARG; ++st) CHECK(convrot_status_string(st)[0] != '\0');
  CHECK(strstr(convrot_status_string(1000), "unknown") != NULL);

  CHECK(convrot_workspace_size(2048, 4096) == (size_t)2048 * 4096 + 2048 * 4);
  CHECK(convrot_workspace_size(0, 4096) == 0);
  CHECK(convrot_dequant_workspace_size(3, 64) == 512);

  CHECK(convrot_rotate_quant(NULL, 4, 256, 256, b, c, s0) == CONVROT_ERR_NULL);
  CHECK(convrot_rotate_quant(a, 4, 250, 256, b, c, s0) == CONVROT_ERR_SHAPE);
  CHECK(convrot_rotate_quant(a, 4, 256, 3, b, c, s0) == CONVROT_ERR_GROUP);
  CHECK(convrot_rotate_quant(mis, 4, 256, 256, b, c, s0) == CONVROT_ERR_ALIGN);
  CHECK(convrot_rotate_quant(NULL, 0, 256, 256, NULL, NULL, s0) == CONVROT_OK);
  CHECK(convrot_rmsnorm_rotate_quant(a, d, -1.0f, 4, 256, 256, b, c, NULL, s0) == CONVROT_ERR_ARG);
  CHECK(convrot_quantize_weight(a, 2, 8, 256, 256, 8, b, c, s0) == CONVROT_ERR_DTYPE);
  CHECK(convrot_w8a8_linear(a, 8, 512, b, c, 64, 256, d, a, 1, s0) == CONVROT_ERR_WORKSPACE);
  CHECK(convrot_w4a8_linear(a, 8, 528, b, c, 64, 16, d, a, 1 << 20, s0) == CONVROT_ERR_SHAPE);
  CHECK(convrot_gemm_i8(a, b, c, 3, d, 4, 4, 64, NULL, d, s0) == CONVROT_ERR_DTYPE);
  CHECK(convrot_gemm_bf16(a, b, 4, 4, 40, c, s0) == CONVROT_ERR_SHAPE);
  CHECK(convrot_dequantize_weight(a, 5, b, 4, 256, 256, c, s0) == CONVROT_ERR_DTYPE);
  CHECK(convrot_dequant_linear(a, 8, 512, b, 8, c, 64, 256, d, a, 1, s0) == CONVROT_ERR_WORKSPACE);

  convrot_linear_out outs[2];
  memset(outs, 0, sizeof outs);
  outs[0].wq = b; outs[0].w_scale = (const float *)c; outs[0].N = 64; outs[0].y = (uint16_t *)d;
  outs[1] = outs[0];
  outs[1].y = NULL; /* results asked for unevenly */
  CHECK(convrot_gemm_i8_multi(a, (const float *)b, 8, 4, 64, outs, 2, s0) == CONVROT_ERR_NULL);
  CHECK(convrot_gemm_i8_multi(a, (const float *)b, 8, 4, 64, outs, 0, s0) == CONVROT_ERR_ARG);
  CHECK(convrot_linear_multi(a, 8, 512, 256, 8, outs, 1, a, 1, s0) == CONVROT_ERR_WORKSPACE);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("C ABI checks passed\n");
  return 0;
}
