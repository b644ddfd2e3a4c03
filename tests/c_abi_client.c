/*
 * A plain C client of libfp8bw.so: includes fp8bw.h, links the library and
 * makes only calls that are answered on the host before any GPU work (the
 * ABI version, status strings, workspace queries and argument validation),
 * so it runs without a GPU.  Exit status 0 when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "fp8bw.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);  \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

int main(void) {
  CHECK(fp8bw_abi_version() >= 1);
  CHECK(strcmp(fp8bw_status_str(FP8BW_OK), "") != 0);
  CHECK(strcmp(fp8bw_status_str(FP8BW_ERR_SHAPE), fp8bw_status_str(FP8BW_ERR_NULL)) != 0);

  /* Workspace queries: split-K partials only when the plan splits. */
  CHECK(fp8bw_linear_ws_bytes(16640, 5120, 8192, 0) > 0);
  CHECK(fp8bw_linear_saved_bytes(16640, 5120, 8192) >= (size_t)8192 * 16640);
  CHECK(fp8bw_tensorwise_quant_ws_bytes(256, 1024) >= 4);

  /* Rejected before any launch: a null input, then K not a multiple of 128. */
  int st = fp8_blockwise_quant(NULL, 128, 128, 128, FP8BW_BLOCK_1x128, 0, NULL, 128, NULL, 1,
                               128, NULL);
  CHECK(st == FP8BW_ERR_NULL);
  CHECK(strlen(fp8bw_last_error()) > 0);
  static unsigned char dummy[256] __attribute__((aligned(256)));
  st = fp8_scaled_gemm_blockwise(dummy, 112, (const float*)dummy, 1, 64, dummy, 112,
                                 (const float*)dummy, 1, 1, FP8BW_BLOCK_128x128, 64, 64, 112,
                                 dummy, 64, FP8BW_OUT_BF16, NULL, 0, NULL);
  CHECK(st == FP8BW_ERR_SHAPE);
  /* Zero-sized problems succeed and enqueue nothing. */
  st = fp8_scaled_gemm_tensorwise(dummy, 16, (const float*)dummy, dummy, 16, (const float*)dummy,
                                  0, 32, 32, dummy, 32, FP8BW_OUT_F32, NULL);
  CHECK(st == FP8BW_OK);

  if (failures == 0) printf("c abi client ok\n");
  return failures == 0 ? 0 : 1;
}
