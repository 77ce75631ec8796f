/*
 * A plain C99 caller of libsparse_ffn.so, built and run by tests/test_c_caller.py on
 * the CPU: the public header compiles as C (-std=c99 -pedantic -Werror), the library
 * links from C, and its host-side entry points behave as the header documents. Only the
 * size queries, the status strings and argument checks that reject a call before any HIP
 * call are exercised, so no kernel is launched and no GPU is needed. The device pointers
 * are fake, 256-byte aligned addresses that validation never dereferences.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sparse_ffn.h"

static int fails = 0;

#define CHECK(cond)                                          \
  do {                                                       \
    if (!(cond)) {                                           \
      printf("FAIL line %d: %s\n", __LINE__, #cond);         \
      ++fails;                                               \
    }                                                        \
  } while (0)

int main(void) {
  char* fake = (char*)(uintptr_t)0x100000;
  sfn_ffn ffn;
  sfn_ffn bad;
  sfn_ffn big;
  sfn_svd svd;
  size_t ws1, ws4, wsp;
  memset(&ffn, 0, sizeof ffn);
  ffn.d = 4096;
  ffn.f = 11008;
  ffn.wdtype = SFN_BF16;
  ffn.act = SFN_ACT_SILU;
  ffn.w_gate = fake;
  ffn.w_up = fake;
  ffn.w_down_t = fake;
  ffn.b_gate = NULL;

  /* size queries */
  ws1 = sparse_ffn_workspace_size(&ffn, 1);
  ws4 = sparse_ffn_workspace_size(&ffn, 4);
  CHECK(ws1 > SFN_WORKSPACE_HEADER_BYTES);
  CHECK(ws4 >= ws1);
  bad = ffn;
  bad.d = 4100; /* a bf16 row of 8200 bytes is not a multiple of 16 */
  CHECK(sparse_ffn_workspace_size(&bad, 1) == 0);
  CHECK(sparse_ffn_workspace_size(NULL, 1) == 0);
  memset(&svd, 0, sizeof svd);
  svd.d = 4096;
  svd.f = 11008;
  svd.r = 256;
  svd.q = fake;
  svd.l = fake;
  svd.tau = (const float*)fake;
  wsp = svd_predict_workspace_size(&svd);
  CHECK(wsp > 0);
  CHECK(sparse_ffn_svd_workspace_size(&ffn, &svd) > 0);
  svd.reserved = 1;
  CHECK(svd_predict_workspace_size(&svd) == 0);
  svd.reserved = 0;

  /* status strings */
  CHECK(strcmp(sparse_ffn_strerror(SFN_OK), "success") == 0);
  CHECK(strlen(sparse_ffn_strerror(SFN_EWORKSPACE)) > 0);
  CHECK(strcmp(sparse_ffn_strerror(12345), "unknown status") == 0);

  /* decode: each rejection comes before anything is enqueued */
  CHECK(sparse_ffn_decode(NULL, fake, 1, NULL, NULL, NULL, NULL, (float*)fake, NULL, NULL, fake, ws1, NULL) ==
        SFN_EINVAL);
  CHECK(sparse_ffn_decode(&ffn, fake, 5, NULL, NULL, NULL, NULL, (float*)fake, NULL, NULL, fake, ws4, NULL) ==
        SFN_ESHAPE);
  CHECK(sparse_ffn_decode(&ffn, fake + 4, 1, NULL, NULL, NULL, NULL, (float*)fake, NULL, NULL, fake, ws1, NULL) ==
        SFN_EALIGN);
  CHECK(sparse_ffn_decode(&ffn, fake, 1, NULL, NULL, NULL, NULL, (float*)fake, NULL, NULL, fake, 100, NULL) ==
        SFN_EWORKSPACE);
  CHECK(sparse_ffn_decode(&ffn, fake, 1, NULL, NULL, NULL, NULL, (float*)fake, NULL, NULL, fake + 16, ws1, NULL) ==
        SFN_EALIGN);
  CHECK(sparse_ffn_decode(&ffn, fake, 1, NULL, (const int32_t*)fake, NULL, NULL, (float*)fake, NULL, NULL, fake,
                          ws1, NULL) == SFN_EINVAL); /* cand without n_cand */
  CHECK(sparse_ffn_decode(&ffn, fake, 1, NULL, NULL, NULL, NULL, (float*)fake, (int32_t*)(fake + 2), NULL, fake,
                          ws1, NULL) == SFN_EALIGN);

  /* the allocation-free decode: beyond its fixed scratch array */
  big = ffn;
  big.d = 8192;
  big.f = 28672;
  CHECK(sparse_ffn_decode_noalloc(&big, fake, 4, NULL, NULL, NULL, NULL, (float*)fake, NULL, NULL, NULL) ==
        SFN_ETOOLARGE);

  /* the other calls */
  CHECK(sparse_ffn_calibrate(&ffn, fake, 256, 1.5f, (float*)fake, NULL, fake, ws4, NULL) == SFN_EINVAL);
  CHECK(sparse_ffn_calibrate(&ffn, fake, 0, 0.5f, (float*)fake, NULL, fake, ws4, NULL) == SFN_ESHAPE);
  CHECK(ffn_dense_chunk(&ffn, fake, 17, (float*)fake, fake, ws4, NULL) == SFN_ESHAPE);
  CHECK(sparse_ffn_decode_parallel(&ffn, fake, NULL, (const int32_t*)fake, (float*)fake, fake, ws1, NULL) ==
        SFN_EINVAL);
  CHECK(svd_predict(&svd, fake, (int32_t*)fake, (int32_t*)fake, NULL, fake, 16, NULL) == SFN_EWORKSPACE);
  CHECK(sparse_ffn_decode_svd(&ffn, &svd, fake, 7, (float*)fake, NULL, NULL, fake, wsp, NULL) == SFN_EINVAL);

  printf(fails ? "failed: %d\n" : "ok\n", fails);
  return fails != 0;
}
