/* A plain C99 caller of the C ABI: the header compiles without HIP or torch,
 * the library links and resolves, and argument validation rejects bad calls
 * before anything reaches a device (so this runs without a GPU).  Prints one
 * line per check and exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "fp8sg.h"

static int failures = 0;

static void expect(const char* what, fp8_status_t got, fp8_status_t want) {
  const int ok = got == want;
  printf("%s %s: %s\n", ok ? "ok" : "FAIL", what, fp8_status_string(got));
  if (!ok) ++failures;
}

int main(void) {
  /* 16-byte aligned fake device addresses: never dereferenced, because each
   * call below fails validation first */
  void* p = (void*)(unsigned long)0x10000;
  float* f = (float*)p;
  uint8_t* q = (uint8_t*)p;
  fp8_operand_t a = {q, FP8_E4M3, FP8_SCALE_TENSOR, p};
  fp8_operand_t b = {q, FP8_E4M3, FP8_SCALE_BLOCK_1x128, p};

  expect("amax NULL x", fp8_amax(NULL, 4, 16, FP8_E4M3, f, NULL, NULL, p, NULL), FP8_ERR_NULL);
  expect("amax NULL workspace", fp8_amax(p, 4, 16, FP8_E4M3, f, NULL, NULL, NULL, NULL),
         FP8_ERR_NULL);
  expect("workspace init misaligned", fp8_workspace_init((char*)p + 128, 0, NULL),
         FP8_ERR_ALIGN);
  expect("cast cols % 16", fp8_quantize_tensor(p, 4, 24, FP8_E4M3, f, q, NULL, NULL, NULL, NULL),
         FP8_ERR_ALIGN);
  expect("block 1x96", fp8_quantize_block(p, 4, 128, FP8_E4M3, 1, 96, q, f, NULL),
         FP8_ERR_UNSUPPORTED);
  expect("block cols % 128", fp8_quantize_block(p, 4, 96, FP8_E4M3, 1, 128, q, f, NULL),
         FP8_ERR_SHAPE);
  expect("mx unknown format", fp8_quantize_mx(p, 4, 32, (fp8_format_t)7, q, q, NULL),
         FP8_ERR_UNSUPPORTED);
  expect("history length 0", fp8_amax_history_update(f, 0, 0, f, FP8_E4M3, f, f, NULL),
         FP8_ERR_SHAPE);
  expect("gemm mixed families", fp8_gemm_fprop(&a, &b, 256, 256, 256, p, NULL),
         FP8_ERR_UNSUPPORTED);
  expect("pair NULL b amax",
         fp8_quantize_pair_current(p, 4, 16, FP8_E4M3, q, f, NULL, f, p, 4, 16, FP8_E4M3, q, NULL,
                                   NULL, f, p, NULL),
         FP8_ERR_NULL);
  if (strncmp(fp8_status_string(FP8_OK), "FP8_OK", 6) != 0) ++failures;
  return failures != 0;
}
