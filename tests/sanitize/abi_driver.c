/*
 * Sanitizer driver for the host side of the C ABI (include/moe.h): linked by
 * tests/test_sanitizers.py against a host-only build of the library's
 * translation units under AddressSanitizer and UndefinedBehaviorSanitizer.
 * It calls the host-only helpers over a sweep of shapes and every
 * argument-validation path that returns before a launch (no device is
 * touched: the pointers below are never dereferenced).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

#define FAKE ((void*)0x10000)
#define FAKE_OFF(n) ((void*)(0x10000 + (n)))

static moe_fused_args_t base(void) {
  moe_fused_args_t a;
  memset(&a, 0, sizeof a);
  a.M = 4;
  a.E = 8;
  a.H = 256;
  a.I = 512;
  a.top_k = 2;
  a.dtype = MOE_DTYPE_BF16;
  a.x = FAKE;
  a.logits = (const float*)FAKE;
  a.w13 = FAKE;
  a.w2 = FAKE;
  a.y = FAKE;
  a.workspace = FAKE;
  a.workspace_bytes = (size_t)1 << 40;
  return a;
}

static void helpers(void) {
  const int Ms[] = {0, 1, 7, 63, 64, 65, 1023, 1024, 4096, 100000};
  const int Es[] = {1, 8, 128, 256, 257, 512, 513};
  const int ks[] = {1, 2, 8, 16, 17};
  const int HIs[] = {128, 256, 2048, 4096, 7168, 14336, 100};
  for (size_t a = 0; a < sizeof Ms / sizeof Ms[0]; ++a)
    for (size_t b = 0; b < sizeof Es / sizeof Es[0]; ++b)
      for (size_t c = 0; c < sizeof ks / sizeof ks[0]; ++c)
        for (size_t d = 0; d < sizeof HIs / sizeof HIs[0]; ++d)
          for (int dt = 0; dt < 3; ++dt) {
            const int M = Ms[a], E = Es[b], k = ks[c], H = HIs[d], I = HIs[(d + 3) % 7];
            (void)moe_fused_workspace_size(M, E, H, I, k, (moe_dtype_t)dt);
            for (int det = 0; det < 3; ++det)
              for (int ws = -1; ws < 5; ++ws) {
                int32_t blk = 0;
                int64_t cap = 0;
                moe_status_t rc = moe_fused_align_shape(M, E, H, I, k, (moe_dtype_t)dt, det, ws, &blk, &cap);
                if (rc == MOE_OK) CHECK(blk == 16 || blk == 128);
              }
            for (int B = 1; B <= 512; B *= 2) (void)moe_align_capacity(M, k, E, B);
          }
  for (int s = -1; s < 6; ++s) CHECK(moe_status_string((moe_status_t)s) != NULL);
  CHECK(moe_abi_version() > 0);
}

static void validation(void) {
  CHECK(moe_route_topk(FAKE, 4, 8, 9, FAKE, FAKE, NULL) == MOE_ERR_INVALID_ARG);
  CHECK(moe_route_topk(FAKE, 4, 600, 2, FAKE, FAKE, NULL) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_route_topk(NULL, 0, 8, 2, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_align(FAKE, 4, 2, 8, 24, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == MOE_ERR_INVALID_ARG);
  CHECK(moe_align(FAKE, 4, 2, 8, 512, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_quant_e4m3(FAKE, -1, FAKE, FAKE, NULL) == MOE_ERR_INVALID_ARG);
  CHECK(moe_quant_e4m3(NULL, 0, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_router_logits(FAKE, FAKE, 4, 8, 200, FAKE, NULL) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_router_logits(FAKE, FAKE_OFF(8), 4, 8, 256, FAKE, NULL) == MOE_ERR_INVALID_ARG);

  CHECK(moe_fused_forward(NULL, NULL) == MOE_ERR_INVALID_ARG);
  moe_fused_args_t a;
#define FUSED(field_setup, code)              \
  do {                                        \
    a = base();                               \
    field_setup;                              \
    CHECK(moe_fused_forward(&a, NULL) == (code)); \
  } while (0)
  FUSED(a.top_k = 9, MOE_ERR_INVALID_ARG);
  FUSED(a.M = -1, MOE_ERR_INVALID_ARG);
  FUSED(a.dtype = (moe_dtype_t)5, MOE_ERR_INVALID_ARG);
  FUSED(a.H = 200, MOE_ERR_UNSUPPORTED);
  FUSED(a.E = 1024, MOE_ERR_UNSUPPORTED);
  FUSED(a.x = NULL, MOE_ERR_INVALID_ARG);
  FUSED(a.workspace_bytes = 100, MOE_ERR_WORKSPACE_TOO_SMALL);
  FUSED(a.w13_scale = (const float*)FAKE, MOE_ERR_INVALID_ARG);
  FUSED(a.dtype = MOE_DTYPE_FP8_E4M3, MOE_ERR_INVALID_ARG);
  FUSED((a.dtype = MOE_DTYPE_FP8_E4M3, a.w13_scale = (const float*)FAKE, a.w2_scale = (const float*)FAKE,
         a.weight_scale_mode = 7),
        MOE_ERR_INVALID_ARG);
  FUSED((a.router_w = FAKE), MOE_ERR_INVALID_ARG);
  FUSED((a.n_shared = 15), MOE_ERR_UNSUPPORTED);
  FUSED((a.sorted_ids = (int32_t*)FAKE_OFF(2)), MOE_ERR_INVALID_ARG);
  FUSED((a.deterministic = 3), MOE_ERR_INVALID_ARG);
  FUSED((a.dtype = MOE_DTYPE_FP8_E4M3, a.w13_scale = (const float*)FAKE, a.w2_scale = (const float*)FAKE,
         a.deterministic = 1),
        MOE_ERR_INVALID_ARG);
  moe_tuning_t t;
  memset(&t, 0, sizeof t);
  t.gemm1_ksplit = 3;
  FUSED((a.tuning = &t), MOE_ERR_UNSUPPORTED);
  memset(&t, 0, sizeof t);
  t.gemm2_ksplit = 2;
  FUSED((a.tuning = &t, a.deterministic = 1), MOE_ERR_INVALID_ARG);
  FUSED((a.M = 0, a.x = NULL, a.workspace = NULL, a.workspace_bytes = 0), MOE_OK);
}

int main(void) {
  helpers();
  validation();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi sanitizer driver ok\n");
  return 0;
}
