/* The Q4_0 library's header used from plain C: compiled by the CPU test suite
 * with -std=c11 -Wall -Wextra -Werror -pedantic and linked against the
 * library.  Only calls that return before any HIP call (queries and argument
 * validation) are made, so no GPU is needed. */
#include <stdio.h>
#include <string.h>

#include "q4.h"

static int fail(const char* what) {
  fprintf(stderr, "FAIL: %s\n", what);
  return 1;
}

int main(void) {
  _Alignas(16) float buf[64];
  _Alignas(16) int32_t idx[4];
  q4_gguf* g = NULL;
  const char* missing = "/nonexistent/q4_abi_smoke.gguf";

  if (q4_abi_version() < 1) return fail("q4_abi_version");
  if (q4_row_bytes(3072) != 1728 || q4_row_bytes(48) != 0) return fail("q4_row_bytes");
  if (strcmp(q4_status_string(Q4_OK), "ok") != 0) return fail("q4_status_string");
  if (q4_matvec(NULL, buf, buf, 1, 1, 32, NULL) != Q4_ERR_NULL) return fail("matvec NULL");
  if (q4_matvec(buf, buf, buf, 1, 1, 48, NULL) != Q4_ERR_SHAPE) return fail("matvec K % 32");
  if (q4_matmul(buf, buf, buf, 0, 1, 32, NULL, 0, NULL) != Q4_ERR_SHAPE) return fail("matmul M = 0");
  if (q4_matmul_workspace_bytes(0, 1, 32) != 0) return fail("matmul workspace of a bad shape");
  if (q4_matmul_residual(buf, buf, NULL, buf, 1, 1, 32, NULL, 0, NULL) != Q4_ERR_NULL)
    return fail("matmul_residual NULL r");
  if (q4_matmul_residual(buf, buf, buf, buf, 2, 16, 64, NULL, 0, NULL) != Q4_ERR_WORKSPACE)
    return fail("matmul_residual in place without workspace");
  if (q4_matmul_residual_workspace_bytes(2, 16, 64) != 2 * 16 * 4)
    return fail("matmul_residual workspace size");
  if (q4_embed_rows(buf, NULL, buf, 1, 1, 32, NULL) != Q4_ERR_NULL) return fail("embed NULL ids");
  if (q4_lmhead_argmax(buf, buf, idx, NULL, 1, 4, 32, NULL, 0, NULL) != Q4_ERR_WORKSPACE)
    return fail("lmhead without workspace");
  if (q4_gguf_open(&missing, 1, &g) != Q4_ERR_IO || g != NULL) return fail("gguf open missing");
  q4_gguf_close(NULL);
  puts("abi_smoke ok");
  return 0;
}
