/* Drives the argument checking of every libsparge entry point on the host
 * only: each call below must be refused before anything reaches HIP, so it
 * runs without a GPU. Built against a copy of the library whose host code is
 * compiled with AddressSanitizer and UndefinedBehaviorSanitizer, it also
 * exercises the size arithmetic (workspace sizes at extreme shapes) and the
 * per-thread error strings under the sanitizers. Exit status 0 = all refused
 * as expected. */
#include <limits.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sparge.h"

static int failures = 0;
#define A ((void*)0x10000)  /* aligned, never dereferenced */
#define M ((void*)0x10002)  /* misaligned */
#define I ((int32_t*)0x10000)
#define F ((float*)0x10000)

static void expect(int got, int want, const char* what) {
  const char* msg = sparge_last_error();
  if (got != want || msg == NULL || msg[0] == '\0') {
    fprintf(stderr, "FAIL %s: got %d want %d (%s)\n", what, got, want, msg ? msg : "(null)");
    ++failures;
  }
}

static void sizes(void) {
  /* every size query at shapes it rejects returns 0; extreme shapes must not
   * overflow (the sanitizers check the arithmetic) */
  const int bad[][6] = {{0, 1, 64, 64, 64, 64},   {1, 0, 64, 64, 64, 64},
                        {1, 1, 0, 64, 64, 64},    {1, 1, 64, 96, 64, 64},
                        {1, 1, 64, 64, 32, 64},   {1, 1, 64, 64, 64, 128},
                        {INT_MAX, INT_MAX, INT_MAX, 128, 64, 64},
                        {1, 1, INT_MAX, 128, 64, 64}, {-1, 1, 64, 64, 64, 64}};
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    const int* s = bad[i];
    if (sparge_mask_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]) != 0 ||
        sparge_mask_routed_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]) != 0 ||
        sparge_attn_lowbit_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]) != 0 ||
        sparge_attn_bwd_workspace_bytes(s[0], s[1], s[2], s[3], s[4], s[5]) != 0 ||
        (s[5] == 64 && svg2_attn_workspace_bytes(s[0], s[1], s[2], s[3], s[4], 8, 8) != 0)) {
      fprintf(stderr, "FAIL size query accepted bad shape %zu\n", i);
      ++failures;
    }
  }
  /* large but valid shapes: sizes are positive and consistent */
  const size_t m = sparge_mask_workspace_bytes(1, 40, 75600, 128, 128, 64);
  const size_t a = sparge_attn_workspace_bytes(64, 40, 262144, 128);
  const size_t l = sparse_linear_workspace_bytes(64, 40, 262144, 128);
  const size_t b = sparse_linear_bwd_workspace_bytes(8, 40, 262144, 128);
  if (m == 0 || a == 0 || l <= a || b == 0) {
    fprintf(stderr, "FAIL size query of a valid shape: %zu %zu %zu %zu\n", m, a, l, b);
    ++failures;
  }
  if (sparge_mask_noalloc_scratch_bytes() != ((size_t)64 << 20)) {
    fprintf(stderr, "FAIL scratch size\n");
    ++failures;
  }
}

static void masks(void) {
  const size_t W = (size_t)1 << 30;
  expect(sparge_mask_predict(NULL, A, 1, 2, 1024, 64, 64, 64, 0.1f, 0.9f, 0.125f, A, I, I, NULL,
                             A, W, NULL), SPARGE_ERR_INVALID_ARG, "mask null q");
  expect(sparge_mask_predict(M, A, 1, 2, 1024, 64, 64, 64, 0.1f, 0.9f, 0.125f, A, I, I, NULL, A,
                             W, NULL), SPARGE_ERR_INVALID_ARG, "mask misaligned q");
  expect(sparge_mask_predict(A, A, 1, 2, 1024, 64, 64, 64, NAN, 0.9f, 0.125f, A, I, I, NULL, A,
                             W, NULL), SPARGE_ERR_INVALID_ARG, "mask NaN k");
  expect(sparge_mask_predict(A, A, 1, 2, 1024, 64, 64, 64, 0.1f, INFINITY, 0.125f, A, I, I,
                             NULL, A, W, NULL), SPARGE_ERR_INVALID_ARG, "mask inf p");
  expect(sparge_mask_predict(A, A, 1, 2, 1024, 64, 64, 64, 0.1f, 0.9f, -1.0f, A, I, I, NULL, A,
                             W, NULL), SPARGE_ERR_INVALID_ARG, "mask negative scale");
  expect(sparge_mask_predict(A, A, 1, 2, 1024, 64, 64, 64, 0.1f, 0.9f, 0.125f, A, I, I, NULL, A,
                             16, NULL), SPARGE_ERR_INVALID_ARG, "mask small workspace");
  expect(sparge_mask_predict(A, A, 1, 2, 64 * 4097, 64, 64, 64, 0.1f, 0.9f, 0.125f, A, I, I,
                             NULL, A, W, NULL), SPARGE_ERR_UNSUPPORTED, "mask too many blocks");
  expect(sparge_mask_predict(A, A, INT_MAX, INT_MAX, INT_MAX, 64, 64, 64, 0.1f, 0.9f, 0.125f, A,
                             I, I, NULL, A, W, NULL), SPARGE_ERR_INVALID_ARG, "mask huge");
  expect(sparge_mask_predict_noalloc(A, A, 1, 40, 75600, 128, 128, 64, 0.1f, 0.9f, 0.125f, A, I,
                                     I, NULL, NULL), SPARGE_ERR_UNSUPPORTED, "noalloc too big");
  expect(sparge_mask_predict_noalloc(A, A, 1, 2, 1024, 64, 64, 64, 0.0f, 0.9f, 0.125f, A, I, I,
                                     NULL, NULL), SPARGE_ERR_INVALID_ARG, "noalloc k = 0");
  expect(sparge_mask_pool(A, NULL, 1, 2, 1024, 64, 64, 64, A, W, NULL), SPARGE_ERR_INVALID_ARG,
         "pool null k");
  expect(sparge_mask_select(1, 2, 1024, 64, 64, 64, 0.1f, 0.9f, 0.125f, NULL, I, I, NULL, A, W,
                            NULL), SPARGE_ERR_INVALID_ARG, "select null bits");
  expect(sparge_mask_predict_routed(A, A, NULL, F, 1, 2, 1024, 64, 64, 64, 0.1f, 0.0f, 0.125f, A,
                                    I, I, NULL, A, W, NULL), SPARGE_ERR_INVALID_ARG,
         "routed null w_q");
  expect(sparge_mask_pool_lowbit(A, A, 1, 2, 1024, 64, 64, 64, A, W, A, 16, NULL),
         SPARGE_ERR_INVALID_ARG, "pool lowbit small workspace");
}

static void attention(void) {
  const size_t W = (size_t)1 << 30;
  expect(sparge_attn_fwd(A, A, A, I, I, 1, 2, 1024, 64, 64, 64, 0.125f, NULL, A, W, NULL),
         SPARGE_ERR_INVALID_ARG, "fwd null o");
  expect(sparge_attn_fwd(A, A, A, I, I, 1, 2, 1024, 64, 48, 64, 0.125f, A, A, W, NULL),
         SPARGE_ERR_UNSUPPORTED, "fwd block_q 48");
  expect(sparge_attn_fwd(A, A, A, (int32_t*)M, I, 1, 2, 1024, 64, 64, 64, 0.125f, A, A, W, NULL),
         SPARGE_ERR_INVALID_ARG, "fwd misaligned idx");
  expect(sparge_attn_fwd(A, A, A, I, I, 1, 2, 1024, 64, 64, 64, 0.125f, A, A, 1, NULL),
         SPARGE_ERR_INVALID_ARG, "fwd small workspace");
  expect(sparge_attn_pack(NULL, 1, 2, 1024, 64, A, W, NULL), SPARGE_ERR_INVALID_ARG, "pack null");
  expect(sparge_attn_fwd_packed(A, A, I, I, 1, 2, 1024, 64, 64, 64, NAN, A, A, W, NULL),
         SPARGE_ERR_INVALID_ARG, "packed NaN scale");
  expect(sparge_attn_fwd_lse(A, A, A, I, I, 1, 2, 1024, 64, 64, 64, 0.125f, A, NULL, A, W, NULL),
         SPARGE_ERR_INVALID_ARG, "lse null");
  expect(sparge_attn_bwd(A, A, A, A, A, F, I, I, 1, 2, 1024, 64, 64, 64, 0.125f, A, A, NULL, A, W,
                         NULL), SPARGE_ERR_INVALID_ARG, "bwd null dv");
  expect(sparse_linear_attn_fwd(A, A, A, I, I, NULL, 1, 2, 1024, 64, 64, 64, 0.125f, 0.0f, A,
                                NULL, A, W, NULL), SPARGE_ERR_INVALID_ARG, "linear null alpha");
  expect(sparse_linear_attn_fwd(A, A, A, I, I, F, 1, 2, 1024, 128, 64, 64, 0.125f, 0.0f, A, NULL,
                                A, W, NULL), SPARGE_ERR_UNSUPPORTED, "linear block_q != d");
  expect(sla2_mix_attn_fwd(A, A, A, I, I, F, 1, 2, 1024, 64, 64, 64, NAN, 0.0f, A, NULL, A, W,
                           NULL), SPARGE_ERR_INVALID_ARG, "mix NaN scale");
  expect(sla2_mix_attn_fwd(A, A, A, I, I, (float*)M, 1, 2, 1024, 64, 64, 64, 0.125f, 0.0f, A,
                           NULL, A, W, NULL), SPARGE_ERR_INVALID_ARG, "mix misaligned alpha");
  expect(sparse_linear_attn_bwd(A, A, A, A, A, F, I, I, NULL, 1, 2, 1024, 64, 64, 64, 0.125f,
                                0.0f, A, A, A, A, W, NULL), SPARGE_ERR_INVALID_ARG,
         "linear bwd null alpha");
  expect(sla2_mix_attn_bwd(A, A, A, A, A, F, I, I, F, 1, 2, 1024, 64, 64, 64, 0.125f, 0.0f, A, A,
                           A, A, 1, NULL), SPARGE_ERR_INVALID_ARG, "mix bwd small workspace");
  expect(sparge_attn_fwd_lowbit(A, A, A, I, I, 1, 2, 1024, 64, 64, 64, 0.125f, A, M, W, NULL),
         SPARGE_ERR_INVALID_ARG, "lowbit misaligned workspace");
  expect(sparge_attn_lowbit_pack(A, 1, 2, 1024, 96, 64, A, W, NULL), SPARGE_ERR_UNSUPPORTED,
         "lowbit pack d 96");
  expect(sparge_attn_fwd_lowbit_packed(I, I, 1, 2, 1024, 64, 64, 64, 0.125f, NULL, A, W, NULL),
         SPARGE_ERR_INVALID_ARG, "lowbit packed null o");
  expect(svg2_attn_fwd(A, A, A, 1, 2, 1024, 64, 64, 0, 8, 3, 0.9f, 0.125f, A, A, W, NULL),
         SPARGE_ERR_INVALID_ARG, "svg2 zero clusters");
  expect(svg2_attn_fwd(A, A, A, 1, 2, 1024, 64, 64, 8, 8, -1, 0.9f, 0.125f, A, A, W, NULL),
         SPARGE_ERR_INVALID_ARG, "svg2 negative rounds");
}

static void* worker(void* arg) {
  (void)arg;
  for (int i = 0; i < 200; ++i) {
    masks();
    attention();
  }
  return NULL;
}

int main(void) {
  sizes();
  masks();
  attention();
  /* error strings are per thread: four threads refuse calls at once */
  pthread_t t[4];
  for (int i = 0; i < 4; ++i) pthread_create(&t[i], NULL, worker, NULL);
  for (int i = 0; i < 4; ++i) pthread_join(t[i], NULL);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("abi checks ok\n");
  return 0;
}
