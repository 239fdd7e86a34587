/*
 * Sanitizer driver for the CPU oracle (oracle/moe_oracle.c): built together
 * with it under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py and run on small inputs that reach every entry
 * point and every error path.  It checks only what needs no reference (return
 * codes, invariants); the oracle's values are pinned by the other tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_decode(uint16_t b);
uint16_t oracle_bf16_encode(float f);
double oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(float f);
float oracle_scale_from_amax(float amax);
int oracle_route(const float* logits, int64_t M, int32_t E, int32_t k, int32_t* ids, float* weights);
int oracle_align(const int32_t* ids, int64_t P, int32_t E, int32_t B, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_ids, int64_t sorted_len, int32_t* block_expert, int64_t n_blocks,
                 int32_t* num_padded);
int oracle_router_logits(const uint16_t* x, const uint16_t* w, int64_t M, int32_t E, int32_t H, float* logits);

/* mirrors oracle_layer_args in oracle/moe_oracle.c */
typedef struct {
  int64_t M;
  int32_t E, H, I, k, dtype;
  const uint16_t* x;
  const float* logits;
  const void* const* w13;
  const void* const* w2;
  float w13_scale, w2_scale;
  int32_t x_scale_static;
  float x_scale;
  int32_t h_scale_static;
  float h_scale;
  const int64_t* tokens;
  int64_t n_tokens;
  double* y;
  int32_t* ids;
  float* weights;
  float* s_x_out;
  float* s_h_out;
  int32_t all_pairs_h;
  const float* const* w13_scale_rows;
  const float* const* w2_scale_rows;
  int32_t n_shared;
  int32_t block_scaled;
  const uint8_t* const* w13_block;
  const uint8_t* const* w2_block;
} layer_args;
uint8_t oracle_block_quant(const float* v, int n, uint8_t* codes);
double oracle_e8m0_value(uint8_t c);
int oracle_layer(layer_args* A);

static int failures = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                             \
    }                                                         \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0;
}
static float normal(void) { return (float)(sqrt(-2.0 * log(uniform() + 1e-300)) * cos(6.283185307179586 * uniform())); }

static void codecs(void) {
  for (int c = 0; c < 256; ++c) {
    double v = oracle_e4m3_decode((uint8_t)c);
    if (!isnan(v)) CHECK(oracle_e4m3_encode((float)v) == (uint8_t)c || v == 0.0);
  }
  const float specials[] = {0.0f, -0.0f, 448.0f, 449.0f, 1e30f, -1e30f, NAN, INFINITY, -INFINITY, 1e-40f};
  for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
    (void)oracle_e4m3_encode(specials[i]);
    (void)oracle_bf16_encode(specials[i]);
  }
  for (int b = 0; b < 65536; b += 7) (void)oracle_bf16_decode((uint16_t)b);
  CHECK(oracle_scale_from_amax(0.0f) == 1.0f);
}

static void routing_and_align(void) {
  const int M = 37, E = 33;
  float* lg = malloc(sizeof(float) * M * E);
  for (int i = 0; i < M * E; ++i) lg[i] = (i % 5 == 0) ? 0.0f : normal();
  for (int k = 1; k <= E; k += 8) {
    int32_t* ids = malloc(sizeof(int32_t) * M * k);
    float* w = malloc(sizeof(float) * M * k);
    CHECK(oracle_route(lg, M, E, k, ids, w) == 0);
    for (int B = 1; B <= 256; B *= 4) {
      const int64_t P = (int64_t)M * k;
      const int64_t cap = ((P + (E < P ? E : P) * (B - 1)) + B - 1) / B * B;
      int32_t counts[33], offsets[34], num = 0;
      int32_t* sorted = malloc(sizeof(int32_t) * (size_t)(cap > 0 ? cap : 1));
      int32_t* blk = malloc(sizeof(int32_t) * (size_t)(cap / B > 0 ? cap / B : 1));
      CHECK(oracle_align(ids, P, E, B, counts, offsets, sorted, cap, blk, cap / B, &num) == 0);
      CHECK(num == offsets[E]);
      free(sorted);
      free(blk);
    }
    free(ids);
    free(w);
  }
  int32_t ids[4], cnt[2], off[3], srt[8], blk[8], num;
  float w[4];
  CHECK(oracle_route(lg, 2, E, 0, ids, w) != 0);     /* k < 1 */
  CHECK(oracle_route(lg, 2, 2, 3, ids, w) != 0);     /* k > E */
  lg[3] = NAN;
  CHECK(oracle_route(lg, 1, E, 2, ids, w) != 0);     /* non-finite logit */
  int32_t bad[3] = {0, 2, 1};
  CHECK(oracle_align(bad, 3, 2, 1, cnt, off, srt, 8, blk, 8, &num) != 0);  /* id out of range */
  int32_t ok[3] = {0, 1, 1};
  CHECK(oracle_align(ok, 3, 2, 4, cnt, off, srt, 4, blk, 1, &num) != 0);   /* capacity too small */
  free(lg);
}

static void layer(int fp8, int xs, int hs, int rows, int S, int subset, int blk) {
  const int M = 9, E = 5, H = blk ? 256 : 32, I = blk ? 128 : 48, k = 2, EW = E + S;
  uint16_t* x = malloc(sizeof(uint16_t) * M * H);
  float* lg = malloc(sizeof(float) * M * E);
  for (int i = 0; i < M * H; ++i) x[i] = oracle_bf16_encode(normal());
  for (int i = 0; i < M * E; ++i) lg[i] = normal();
  void* w13[8];
  void* w2[8];
  float* r13[8];
  float* r2[8];
  uint8_t* b13[8];
  uint8_t* b2[8];
  for (int e = 0; e < EW; ++e) {
    const size_t n13 = (size_t)2 * I * H, n2 = (size_t)H * I, esz = fp8 ? 1 : 2;
    w13[e] = malloc(n13 * esz);
    w2[e] = malloc(n2 * esz);
    for (size_t i = 0; i < n13; ++i) {
      float v = normal() * 0.2f;
      if (fp8) ((uint8_t*)w13[e])[i] = oracle_e4m3_encode(v * 100.0f);
      else ((uint16_t*)w13[e])[i] = oracle_bf16_encode(v);
    }
    for (size_t i = 0; i < n2; ++i) {
      float v = normal() * 0.2f;
      if (fp8) ((uint8_t*)w2[e])[i] = oracle_e4m3_encode(v * 100.0f);
      else ((uint16_t*)w2[e])[i] = oracle_bf16_encode(v);
    }
    r13[e] = malloc(sizeof(float) * 2 * I);
    r2[e] = malloc(sizeof(float) * H);
    for (int i = 0; i < 2 * I; ++i) r13[e][i] = 0.01f * (1 + i % 3);
    for (int i = 0; i < H; ++i) r2[e][i] = 0.01f * (1 + i % 4);
    b13[e] = malloc((size_t)(2 * I / 128) * (H / 128) + 1);
    b2[e] = malloc((size_t)(H / 128) * (I / 128) + 1);
    for (int i = 0; i < (2 * I / 128) * (H / 128); ++i) b13[e][i] = (uint8_t)(118 + i % 5);
    for (int i = 0; i < (H / 128) * (I / 128); ++i) b2[e][i] = (uint8_t)(119 + i % 3);
  }
  int64_t tokens[9];
  int64_t nt = 0;
  for (int m = 0; m < M; ++m)
    if (!subset || m % 3 == 0) tokens[nt++] = m;
  double* y = malloc(sizeof(double) * (size_t)nt * H);
  int32_t ids[18];
  float wts[18], sx = 0, sh = 0;
  layer_args A;
  memset(&A, 0, sizeof A);
  A.M = M; A.E = E; A.H = H; A.I = I; A.k = k; A.dtype = fp8;
  A.x = x; A.logits = lg; A.w13 = (const void* const*)w13; A.w2 = (const void* const*)w2;
  A.w13_scale = 0.01f; A.w2_scale = 0.01f;
  A.x_scale_static = xs; A.x_scale = 0.02f; A.h_scale_static = hs; A.h_scale = 0.01f;
  A.tokens = tokens; A.n_tokens = nt; A.y = y; A.ids = ids; A.weights = wts; A.s_x_out = &sx; A.s_h_out = &sh;
  A.all_pairs_h = fp8 && !hs;
  A.w13_scale_rows = rows ? (const float* const*)r13 : NULL;
  A.w2_scale_rows = rows ? (const float* const*)r2 : NULL;
  A.n_shared = S;
  A.block_scaled = blk;
  A.w13_block = (const uint8_t* const*)b13;
  A.w2_block = (const uint8_t* const*)b2;
  CHECK(oracle_layer(&A) == 0);
  for (int64_t i = 0; i < nt * H; ++i) CHECK(isfinite(y[i]));
  /* a missing expert is reported, not dereferenced */
  void* keep = w13[ids[0]];
  w13[ids[0]] = NULL;
  CHECK(oracle_layer(&A) != 0);
  w13[ids[0]] = keep;
  /* a token index out of range is reported */
  int64_t bad_tok = M;
  A.tokens = &bad_tok;
  A.n_tokens = 1;
  CHECK(oracle_layer(&A) != 0);
  for (int e = 0; e < EW; ++e) {
    free(w13[e]);
    free(w2[e]);
    free(r13[e]);
    free(r2[e]);
    free(b13[e]);
    free(b2[e]);
  }
  free(x);
  free(lg);
  free(y);
}

static void router(void) {
  const int M = 7, E = 9, H = 40;
  uint16_t* x = malloc(sizeof(uint16_t) * M * H);
  uint16_t* w = malloc(sizeof(uint16_t) * E * H);
  float* out = malloc(sizeof(float) * M * E);
  for (int i = 0; i < M * H; ++i) x[i] = oracle_bf16_encode(normal());
  for (int i = 0; i < E * H; ++i) w[i] = oracle_bf16_encode(normal());
  CHECK(oracle_router_logits(x, w, M, E, H, out) == 0);
  CHECK(oracle_router_logits(x, w, M, 0, H, out) != 0);
  free(x);
  free(w);
  free(out);
}

int main(void) {
  codecs();
  routing_and_align();
  for (int fp8 = 0; fp8 < 2; ++fp8)
    for (int xs = 0; xs < 2; ++xs)
      for (int hs = 0; hs < 2; ++hs)
        for (int rows = 0; rows < 2; ++rows)
          for (int S = 0; S < 3; S += 2)
            for (int subset = 0; subset < 2; ++subset) {
              if (!fp8 && (xs || hs || rows)) continue;
              layer(fp8, xs, hs, rows, S, subset, 0);
            }
  for (int S = 0; S < 3; S += 2)
    for (int subset = 0; subset < 2; ++subset) layer(1, 0, 0, 0, S, subset, 1);
  {
    float v[128];
    uint8_t q[128];
    for (int i = 0; i < 128; ++i) v[i] = normal() * 1e-39f;
    (void)oracle_block_quant(v, 128, q);
    for (int i = 0; i < 128; ++i) v[i] = normal() * 1e30f;
    (void)oracle_block_quant(v, 128, q);
    for (int c = 0; c < 256; ++c) (void)oracle_e8m0_value((uint8_t)c);
  }
  router();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver ok\n");
  return 0;
}
