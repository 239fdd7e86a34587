/*
 * CPU oracle for the fused Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library and must never be used as a
 * fallback for it.
 *
 * What it computes is the plain definition of the layer: for each token, the
 * selected experts are evaluated one after the other with dense loops, and
 * their outputs are summed with the routing weights.  The web pages on the
 * subject describe the fused layer only as token routing, data movement and
 * expert computation done as one batched GPU operation (wagnersolution,
 * "AWS describes a fused MoE optimization ...", body), with scaling, the
 * matrix product and expert aggregation fused into one pass (The Neural Net,
 * "AWS details MoE kernel fixes ...", body).  The swapped operand order the
 * pages discuss (computing B^T A^T, which yields the transposed product) only
 * changes how the product is evaluated, never its value, so the oracle does
 * no grouping, sorting, padding or operand swapping to compute y.
 *
 * Precision.  The pages fix no precision for the reference, so every sum and
 * every activation is evaluated in IEEE double, in the plain sequential order
 * written below (build with -ffp-contract=off, no fast-math).  Where floating
 * point decides an integer code (bf16 or e4m3 rounding of an activation, the
 * per-tensor scale that feeds it), the decision is taken in fp32, the
 * precision of the GPU path: value rounded to fp32, multiplied in fp32 by the
 * fp32 reciprocal of the scale, then rounded to the 8- or 16-bit code.
 *
 * Parity pins are in tests/test_oracle_*.py: brute-force sorts for routing
 * and alignment, closed forms for the softmax weights, the E=1/k=1 case
 * against a float64 library matmul, the all-equal-logit case against the mean
 * of expert outputs, the e4m3/bf16 codecs against the framework's casts, and
 * hand-derived fixtures in tests/golden/.  Block-scaled mode: block
 * quantisation by brute force over all E4M3 codes and by its exponent window
 * and shift invariance, the E=1/k=1 layer against float64 library matmuls of
 * the dequantised operands, and per-token independence (tests/
 * test_oracle_block.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_MISSING_EXPERT 2
#define ORC_ERR_NONFINITE 3

#define ORC_DTYPE_BF16 0
#define ORC_DTYPE_E4M3 1

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_bf16_decode(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Nearest bf16 to an fp32 value, ties to even mantissa.  NaN stays NaN. */
uint16_t oracle_bf16_encode(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t upper = u >> 16;
  uint32_t lower = u & 0xffffu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u; /* carries into exponent correctly */
  return (uint16_t)upper;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; largest finite 448 = 1.75 * 2^8; subnormals m/8 * 2^-6. */
double oracle_e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int ex = (c >> 3) & 0xf;
  int man = c & 0x7;
  double v;
  if (ex == 0xf && man == 0x7) return NAN;
  if (ex == 0)
    v = ldexp((double)man / 8.0, -6);
  else
    v = ldexp(1.0 + (double)man / 8.0, ex - 7);
  return sign ? -v : v;
}

/* Nearest e4m3 code to an fp32 value, ties to the even code, magnitudes
 * above 448 saturate to 448.  Non-negative codes 0x00..0x7e are ordered by
 * value, so a binary search finds the pair that brackets |v|. */
uint8_t oracle_e4m3_encode(float f) {
  if (isnan(f)) return 0x7f;
  uint8_t sign = signbit(f) ? 0x80 : 0x00;
  double a = fabs((double)f);
  if (a >= 448.0) return (uint8_t)(sign | 0x7e);
  int lo = 0, hi = 0x7e; /* invariant: decode(lo) <= a < decode(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_decode((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - oracle_e4m3_decode((uint8_t)lo);
  double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
  int code;
  if (dlo < dhi)
    code = lo;
  else if (dhi < dlo)
    code = hi;
  else
    code = (lo & 1) ? hi : lo;
  return (uint8_t)(sign | code);
}

/* Per-tensor scale of an fp8 activation from its largest magnitude:
 * amax/448 in fp32, 1.0 when the tensor is all zeros. */
float oracle_scale_from_amax(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  return amax / 448.0f;
}

/* ------------------------------------------------------------------------ */
/* Block-scaled FP8: power-of-two scales per block                           */
/* ------------------------------------------------------------------------ */

/* Value of an E8M0 scale code (OCP MX scale format: 2^(c-127); 255 is NaN). */
double oracle_e8m0_value(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* Block quantisation of n consecutive fp32 values (n <= 128) sharing one
 * scale, the OCP MX rule for an E4M3 element format: the shared exponent is
 * floor(log2(amax)) minus 8, the exponent of the format's largest power of
 * two (448 = 1.75 * 2^8), clamped to the code range; each element is
 * divided by the scale and rounded to E4M3 (nearest even, saturating at 448).
 * With amax read as a biased binary32 exponent field f, the scale code is
 * max(f - 8, 0) (the smallest scale, 2^-127, for amax below 2^-118: zero,
 * subnormal or tiny blocks).  Dividing by a power of two is exact here: the
 * quotients stay below 512.  Returns the scale code. */
uint8_t oracle_block_quant(const float* v, int n, uint8_t* codes) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i)
    if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
  uint32_t bits;
  memcpy(&bits, &amax, sizeof bits);
  const int f = (int)((bits >> 23) & 0xff);
  const int c = f > 8 ? f - 8 : 0;
  const float r = ldexpf(1.0f, 127 - c); /* 1/scale, a power of two between 2^-119 and 2^127 */
  for (int i = 0; i < n; ++i) codes[i] = oracle_e4m3_encode(v[i] * r);
  return (uint8_t)c;
}

/* Quantise an fp32 value with the fp32 reciprocal of the scale. */
static uint8_t quant_e4m3(float v, float recip) {
  float t = v * recip; /* fp32 product, rounded once */
  return oracle_e4m3_encode(t);
}

/* ------------------------------------------------------------------------ */
/* Routing: top-k over the router logits, softmax over the selected ones.   */
/* ------------------------------------------------------------------------ */

/* For every token m: repeatedly pick the largest logit not yet taken; a
 * strict '>' keeps the lower expert index on ties, and IEEE comparison makes
 * -0.0 equal to +0.0.  Slot j holds the j-th largest.  Weights are the
 * softmax over the k selected logits (the same as the softmax over all E
 * renormalised over the selected experts), in double, rounded to fp32. */
int oracle_route(const float* logits, int64_t M, int32_t E, int32_t k, int32_t* ids, float* weights) {
  if (E < 1 || k < 1 || k > E || M < 0) return ORC_ERR_ARG;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  double* ex = (double*)malloc(sizeof(double) * (size_t)k);
  for (int64_t m = 0; m < M; ++m) {
    const float* row = logits + m * E;
    for (int32_t e = 0; e < E; ++e) {
      if (!isfinite(row[e])) {
        free(taken);
        free(ex);
        return ORC_ERR_NONFINITE;
      }
    }
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || row[e] > row[best]) best = e;
      }
      taken[best] = 1;
      ids[m * k + j] = best;
    }
    double top = (double)row[ids[m * k + 0]];
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      ex[j] = exp((double)row[ids[m * k + j]] - top);
      sum += ex[j];
    }
    for (int32_t j = 0; j < k; ++j) weights[m * k + j] = (float)(ex[j] / sum);
  }
  free(taken);
  free(ex);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Alignment: group the (token, slot) pairs by expert and pad each group.    */
/* ------------------------------------------------------------------------ */

/* ids: [P] expert of flat pair f = m*k + j.  For block size B:
 *   counts[e]   = number of pairs routed to e
 *   offsets[e]  = sum over e' < e of ceil(counts[e']/B)*B, offsets[E] = total
 *   sorted_ids  = pair indices grouped by expert in increasing f (a counting
 *                 sort, hence stable), each group followed by the sentinel P
 *                 up to its padded length; entries at or after the total are
 *                 left untouched
 *   block_expert[b] = expert owning block b for b < total/B, -1 after, up to
 *                 n_blocks entries
 *   num_padded  = total */
int oracle_align(const int32_t* ids, int64_t P, int32_t E, int32_t B, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_ids, int64_t sorted_len, int32_t* block_expert, int64_t n_blocks,
                 int32_t* num_padded) {
  if (E < 1 || B < 1 || P < 0) return ORC_ERR_ARG;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < P; ++f) {
    if (ids[f] < 0 || ids[f] >= E) return ORC_ERR_ARG;
    counts[ids[f]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) {
    int32_t padded = ((counts[e] + B - 1) / B) * B;
    offsets[e + 1] = offsets[e] + padded;
  }
  int64_t total = offsets[E];
  if (total > sorted_len || total / B > n_blocks) return ORC_ERR_ARG;
  for (int64_t i = 0; i < total; ++i) sorted_ids[i] = (int32_t)P;
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t f = 0; f < P; ++f) sorted_ids[cursor[ids[f]]++] = (int32_t)f;
  free(cursor);
  for (int64_t b = 0; b < n_blocks; ++b) block_expert[b] = -1;
  for (int32_t e = 0; e < E; ++e)
    for (int64_t b = offsets[e] / B; b < offsets[e + 1] / B; ++b) block_expert[b] = e;
  *num_padded = (int32_t)total;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* The layer                                                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t M;
  int32_t E, H, I, k, dtype;
  const uint16_t* x;            /* [M,H] bf16 */
  const float* logits;          /* [M,E] */
  const void* const* w13;       /* E + n_shared pointers, each [2I,H] bf16|e4m3; NULL = not provided */
  const void* const* w2;        /* E pointers, each [H,I] */
  float w13_scale, w2_scale;    /* fp8 only */
  int32_t x_scale_static;       /* fp8: 1 = use x_scale, 0 = amax/448 */
  float x_scale;
  int32_t h_scale_static;
  float h_scale;
  const int64_t* tokens;        /* rows of y to produce */
  int64_t n_tokens;
  double* y;                    /* [n_tokens,H] out, before any output rounding */
  int32_t* ids;                 /* [M,k] out */
  float* weights;               /* [M,k] out */
  float* s_x_out;               /* fp8 out (may be NULL) */
  float* s_h_out;               /* fp8 out (may be NULL) */
  int32_t all_pairs_h;          /* 1: evaluate h for all pairs (needed for a dynamic h scale) */
  /* fp8, one scale per weight row (output channel) instead of w13_scale /
   * w2_scale: E pointers, each [2I] (row n of W13[e]) resp. [H] (row n of
   * W2[e]); NULL = one scale per tensor */
  const float* const* w13_scale_rows;
  const float* const* w2_scale_rows;
  /* shared experts: every token also passes through experts E..E+n_shared-1
   * (entries E.. of w13/w2 and of the row-scale arrays) with weight one */
  int32_t n_shared;
  /* fp8, block-scaled mode (1) instead of the scales above: weights carry one
   * power-of-two scale per 128 x 128 block (E pointers to uint8 E8M0 codes,
   * [2I/128][H/128] for W13[e], [H/128][I/128] for W2[e]); activations are
   * quantised per 128 consecutive elements of a token's x row or of a
   * pair's h row, each group with its own power-of-two scale
   * (oracle_block_quant).  H and I multiples of 128. */
  int32_t block_scaled;
  const uint8_t* const* w13_block;
  const uint8_t* const* w2_block;
} oracle_layer_args;

/* e4m3 code -> value, filled from oracle_e4m3_decode before any parallel
 * region so that the inner loops do not call ldexp per element. */
static double e4m3_value[256];
static int e4m3_value_ready = 0;
static void fill_e4m3_value(void) {
  if (e4m3_value_ready) return;
  for (int c = 0; c < 256; ++c) e4m3_value[c] = oracle_e4m3_decode((uint8_t)c);
  e4m3_value_ready = 1;
}

static double weight_at(int32_t dtype, const void* base, int64_t idx) {
  if (dtype == ORC_DTYPE_BF16) return oracle_bf16_decode(((const uint16_t*)base)[idx]);
  return e4m3_value[((const uint8_t*)base)[idx]];
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* Power-of-two scale of element (row, col) of W13[e] / W2[e] in block mode:
 * the code of its 128 x 128 block. */
static double w13_block_of(const oracle_layer_args* A, int32_t e, int64_t row, int64_t col) {
  return oracle_e8m0_value(A->w13_block[e][(row / 128) * (A->H / 128) + col / 128]);
}
static double w2_block_of(const oracle_layer_args* A, int32_t e, int64_t row, int64_t col) {
  return oracle_e8m0_value(A->w2_block[e][(row / 128) * (A->I / 128) + col / 128]);
}

/* Weight scale of row `row` of W13[e] / W2[e]: its own, or the tensor's. */
static double w13_scale_of(const oracle_layer_args* A, int32_t e, int64_t row) {
  return A->w13_scale_rows ? (double)A->w13_scale_rows[e][row] : (double)A->w13_scale;
}
static double w2_scale_of(const oracle_layer_args* A, int32_t e, int64_t row) {
  return A->w2_scale_rows ? (double)A->w2_scale_rows[e][row] : (double)A->w2_scale;
}

/* h for one pair (token m, expert e), in fp32 as the value the next step
 * rounds from.  a: the token's activation row in double (x, or its e4m3
 * codes decoded); s_a: the activation scale (fp8); the products of row n
 * are rescaled by s_a times that row's weight scale (fp8 only). */
static void expert_up(const oracle_layer_args* A, int32_t e, const double* a, double s_a, float* h) {
  const void* w = A->w13[e];
  const int fp8 = A->dtype == ORC_DTYPE_E4M3;
  int64_t H = A->H, I = A->I;
  for (int64_t n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    if (A->block_scaled) { /* a holds dequantised activations; each weight times its block's scale */
      for (int64_t t = 0; t < H; ++t) g += a[t] * (weight_at(A->dtype, w, n * H + t) * w13_block_of(A, e, n, t));
      for (int64_t t = 0; t < H; ++t)
        u += a[t] * (weight_at(A->dtype, w, (I + n) * H + t) * w13_block_of(A, e, I + n, t));
      h[n] = (float)(silu(g) * u);
      continue;
    }
    for (int64_t t = 0; t < H; ++t) g += a[t] * weight_at(A->dtype, w, n * H + t);
    for (int64_t t = 0; t < H; ++t) u += a[t] * weight_at(A->dtype, w, (I + n) * H + t);
    if (fp8) {
      g *= s_a * w13_scale_of(A, e, n);
      u *= s_a * w13_scale_of(A, e, I + n);
    }
    h[n] = (float)(silu(g) * u);
  }
}

int oracle_layer(oracle_layer_args* A) {
  const int64_t M = A->M;
  const int32_t E = A->E, H = A->H, I = A->I, k = A->k, S = A->n_shared;
  if (M < 0 || E < 1 || k < 1 || k > E || H < 1 || I < 1 || S < 0) return ORC_ERR_ARG;
  if (A->dtype != ORC_DTYPE_BF16 && A->dtype != ORC_DTYPE_E4M3) return ORC_ERR_ARG;
  const int fp8 = A->dtype == ORC_DTYPE_E4M3;
  const int blk = A->block_scaled != 0;
  if (blk && (!fp8 || H % 128 || I % 128 || !A->w13_block || !A->w2_block)) return ORC_ERR_ARG;
  fill_e4m3_value();

  int rc = oracle_route(A->logits, M, E, k, A->ids, A->weights);
  if (rc) return rc;
  if (M == 0) return ORC_OK;

  /* The pairs of token m: its k routed experts with their routing weights,
   * then each shared expert E+s (s < S) with weight one. */
  const int32_t kk = k + S;
  const int64_t P = M * kk;
  int32_t* pid = (int32_t*)malloc(sizeof(int32_t) * (size_t)P);
  double* pw = (double*)malloc(sizeof(double) * (size_t)P);
  for (int64_t m = 0; m < M; ++m) {
    for (int32_t j = 0; j < kk; ++j) {
      pid[m * kk + j] = j < k ? A->ids[m * k + j] : E + (j - k);
      pw[m * kk + j] = j < k ? (double)A->weights[m * k + j] : 1.0;
    }
  }

  /* which pairs need h */
  unsigned char* need = (unsigned char*)calloc((size_t)P, 1);
  for (int64_t i = 0; i < A->n_tokens; ++i) {
    int64_t m = A->tokens[i];
    if (m < 0 || m >= M) {
      free(need);
      free(pid);
      free(pw);
      return ORC_ERR_ARG;
    }
    for (int32_t j = 0; j < kk; ++j) need[m * kk + j] = 1;
  }
  if (A->all_pairs_h)
    for (int64_t p = 0; p < P; ++p) need[p] = 1;
  for (int64_t p = 0; p < P; ++p) {
    if (need[p] && (A->w13[pid[p]] == NULL || A->w2[pid[p]] == NULL)) {
      free(need);
      free(pid);
      free(pw);
      return ORC_ERR_MISSING_EXPERT;
    }
  }

  for (int64_t p = 0; blk && p < P; ++p) {
    if (need[p] && (A->w13_block[pid[p]] == NULL || A->w2_block[pid[p]] == NULL)) {
      free(need);
      free(pid);
      free(pw);
      return ORC_ERR_MISSING_EXPERT;
    }
  }

  /* activation operand of the first product (block mode: per 128-element
   * group of the token's row, below) */
  float s_x = 1.0f;
  if (blk) {
    if (A->s_x_out) *A->s_x_out = 0.0f;
  } else if (fp8) {
    if (A->x_scale_static) {
      s_x = A->x_scale;
    } else {
      float amax = 0.0f;
      for (int64_t i = 0; i < M * (int64_t)H; ++i) {
        float v = fabsf((float)oracle_bf16_decode(A->x[i]));
        if (v > amax) amax = v;
      }
      s_x = oracle_scale_from_amax(amax);
    }
    if (A->s_x_out) *A->s_x_out = s_x;
  }
  const float r_x = 1.0f / s_x;

  /* h for every needed pair, fp32 */
  float* h = (float*)malloc(sizeof(float) * (size_t)P * (size_t)I);
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < P; ++p) {
      if (!need[p]) continue;
      int64_t m = p / kk;
      if (blk) {
        float v[128];
        uint8_t q[128];
        for (int64_t g = 0; g < H; g += 128) {
          for (int i = 0; i < 128; ++i) v[i] = (float)oracle_bf16_decode(A->x[m * H + g + i]);
          const double sc = oracle_e8m0_value(oracle_block_quant(v, 128, q));
          for (int i = 0; i < 128; ++i) a[g + i] = oracle_e4m3_decode(q[i]) * sc;
        }
      } else {
        for (int64_t t = 0; t < H; ++t) {
          float xv = (float)oracle_bf16_decode(A->x[m * H + t]);
          a[t] = fp8 ? oracle_e4m3_decode(quant_e4m3(xv, r_x)) : (double)xv;
        }
      }
      expert_up(A, pid[p], a, (double)s_x, h + p * (int64_t)I);
    }
    free(a);
  }

  /* activation operand of the second product (block mode: per 128-element
   * group of each pair's h row) */
  float s_h = 1.0f;
  if (blk) {
    if (A->s_h_out) *A->s_h_out = 0.0f;
  } else if (fp8) {
    if (A->h_scale_static) {
      s_h = A->h_scale;
    } else {
      float amax = 0.0f;
      for (int64_t p = 0; p < P; ++p) {
        if (!need[p]) continue;
        for (int64_t n = 0; n < I; ++n) {
          float v = fabsf(h[p * I + n]);
          if (v > amax) amax = v;
        }
      }
      s_h = oracle_scale_from_amax(amax);
    }
    if (A->s_h_out) *A->s_h_out = s_h;
  }
  const float r_h = 1.0f / s_h;

  double* hq = (double*)malloc(sizeof(double) * (size_t)P * (size_t)I);
  for (int64_t p = 0; p < P; ++p) {
    if (!need[p]) continue;
    if (blk) {
      uint8_t q[128];
      for (int64_t g = 0; g < I; g += 128) {
        const double sc = oracle_e8m0_value(oracle_block_quant(h + p * I + g, 128, q));
        for (int i = 0; i < 128; ++i) hq[p * I + g + i] = oracle_e4m3_decode(q[i]) * sc;
      }
      continue;
    }
    for (int64_t n = 0; n < I; ++n) {
      float v = h[p * I + n];
      hq[p * I + n] = fp8 ? oracle_e4m3_decode(quant_e4m3(v, r_h)) : oracle_bf16_decode(oracle_bf16_encode(v));
    }
  }

  /* second product and the weighted combine, per requested token */
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < A->n_tokens; ++i) {
    for (int64_t n = 0; n < H; ++n) {
      int64_t m = A->tokens[i];
      double acc = 0.0;
      for (int32_t j = 0; j < kk; ++j) {
        int64_t p = m * kk + j;
        const void* w = A->w2[pid[p]];
        double o = 0.0;
        if (blk) {
          for (int64_t t = 0; t < I; ++t)
            o += hq[p * I + t] * (weight_at(A->dtype, w, n * (int64_t)I + t) * w2_block_of(A, pid[p], n, t));
        } else {
          for (int64_t t = 0; t < I; ++t) o += hq[p * I + t] * weight_at(A->dtype, w, n * (int64_t)I + t);
          if (fp8) o *= (double)s_h * w2_scale_of(A, pid[p], n);
        }
        acc += pw[p] * o;
      }
      A->y[i * H + n] = acc;
    }
  }
  free(hq);
  free(h);
  free(need);
  free(pid);
  free(pw);
  return ORC_OK;
}

/* Router logits, the step before routing: logits[m,e] = sum_t x[m,t] *
 * w[e,t] for bf16 x [M,H] and router weights w [E,H], summed in double with
 * t ascending and rounded once to fp32 (wagnersolution page, "AWS describes a
 * fused MoE optimization for the NVIDIA Hopper architecture", body: the fused
 * operation starts from the tokens' routing). */
int oracle_router_logits(const uint16_t* x, const uint16_t* w, int64_t M, int32_t E, int32_t H, float* logits) {
  if (M < 0 || E < 1 || H < 1) return ORC_ERR_ARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t t = 0; t < H; ++t)
        acc += oracle_bf16_decode(x[m * H + t]) * oracle_bf16_decode(w[(int64_t)e * H + t]);
      logits[m * E + e] = (float)acc;
    }
  }
  return ORC_OK;
}

/* Threads the parallel loops use (OpenMP's default team size). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif

int oracle_abi_version(void) { return 5; }
