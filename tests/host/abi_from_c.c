/* abi_from_c.c -- the C ABI used from plain C99, with no HIP header:
 * include/fa_varlen.h and include/fa_probe.h must compile on their own, and
 * the calls below return their documented statuses before any device work
 * (built with gcc and run on the host by tests/test_c_abi.py). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa_probe.h"
#include "fa_varlen.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: status %d (%s), expected %d\n", what, got, fa_status_string(got), want);
    ++failures;
  }
}

/* A contiguous descriptor with no data: enough for host validation. */
static fa_tensor tensor(int32_t dtype, int32_t ndim, int64_t d0, int64_t d1, int64_t d2) {
  fa_tensor t;
  memset(&t, 0, sizeof t);
  t.dtype = dtype;
  t.ndim = ndim;
  t.shape[0] = d0;
  t.shape[1] = d1;
  t.shape[2] = d2;
  t.stride[ndim - 1] = 1;
  if (ndim >= 2) t.stride[ndim - 2] = t.shape[ndim - 1];
  if (ndim == 3) t.stride[0] = d1 * d2;
  return t;
}

int main(void) {
  int32_t bm = 0, bn = 0;
  size_t bytes = 0;
  expect(fa_varlen_block_sizes(128, FA_DTYPE_BF16, &bm, &bn), FA_OK, "block sizes");
  if (bm <= 0 || bn <= 0 || bm % 32 || bn % 32) {
    printf("FAIL block sizes %d x %d\n", (int)bm, (int)bn);
    ++failures;
  }
  expect(fa_varlen_block_sizes(100, FA_DTYPE_BF16, &bm, &bn), FA_ERR_HEAD_DIM, "block sizes, head_dim 100");
  expect(fa_varlen_bwd_workspace_size(2, 300, 4, 128, &bytes), FA_OK, "backward workspace");
  if (bytes < (size_t)300 * 4 * 128 * 4) {
    printf("FAIL backward workspace %zu bytes\n", bytes);
    ++failures;
  }
  expect(fa_varlen_kvcache_workspace_size(4, 8, 128, 3, &bytes), FA_OK, "cache workspace");
  expect(fa_varlen_kvcache_workspace_size(4, 8, 128, 65, &bytes), FA_ERR_ARG, "cache workspace, 65 splits");

  /* validation failures: nothing is launched */
  fa_tensor q = tensor(FA_DTYPE_BF16, 3, 0, 4, 128), k = tensor(FA_DTYPE_BF16, 3, 0, 2, 128);
  fa_tensor cu = tensor(FA_DTYPE_I32, 1, 1, 0, 0), out = tensor(FA_DTYPE_BF16, 3, 0, 4, 128);
  fa_tensor lse = tensor(FA_DTYPE_F32, 2, 4, 0, 0);
  expect(fa_varlen_fwd(NULL, &k, &k, &cu, &cu, 0, 0, 0.125f, 0, &out, &lse, NULL), FA_ERR_NULL, "NULL q");
  fa_tensor bad = q;
  bad.dtype = FA_DTYPE_I32;
  expect(fa_varlen_fwd(&bad, &k, &k, &cu, &cu, 0, 0, 0.125f, 0, &out, &lse, NULL), FA_ERR_DTYPE, "int32 q");
  fa_tensor q100 = tensor(FA_DTYPE_BF16, 3, 0, 4, 100), k100 = tensor(FA_DTYPE_BF16, 3, 0, 2, 100);
  fa_tensor out100 = tensor(FA_DTYPE_BF16, 3, 0, 4, 100);
  expect(fa_varlen_fwd(&q100, &k100, &k100, &cu, &cu, 0, 0, 0.125f, 0, &out100, &lse, NULL), FA_ERR_HEAD_DIM,
         "head_dim 100");
  /* the offsets need data (one entry); a host array suffices, as nothing
     past validation runs: the scale is rejected first */
  static int32_t cu_host[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  cu.data = cu_host;
  expect(fa_varlen_fwd(&q, &k, &k, &cu, &cu, 0, 0, -1.0f, 0, &out, &lse, NULL), FA_ERR_ARG, "negative scale");
  expect(fa_varlen_fwd(&q, &k, &k, &cu, &cu, 0, 0, 0.125f, 2, &out, &lse, NULL), FA_ERR_ARG, "causal 2");
  if (strcmp(fa_status_string(FA_OK), "ok") != 0) {
    printf("FAIL status string\n");
    ++failures;
  }
  /* the probe library's entry points exist with the declared types */
  int (*peak)(int32_t, double*, double*) = fa_probe_mfma_peak;
  int (*peak_random)(int32_t, uint32_t, double*, double*) = fa_probe_mfma_peak_random;
  if (!peak || !peak_random) ++failures;
  printf(failures ? "%d failures\n" : "C ABI checks passed\n", failures);
  return failures ? 1 : 0;
}
