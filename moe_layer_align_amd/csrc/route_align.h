// Router top-k and the sort-and-pad (align) kernels, plus the activation
// quantisation that rides along with the align launch in the fused path.
#pragma once

#include "moe_device.h"

namespace moe {

// --------------------------------------------------------------------------
// Router: four tokens per wavefront, one per 16-lane row.
//
// Lane l of a row holds the logits of experts l, l+16, ... of the row's
// token as 64-bit keys: high word = order-preserving image of the float (with
// -0.0 mapped to +0.0 first), low word = ~expert, so the largest key is the
// largest logit and, among equal logits, the lowest expert.  Each of the k
// rounds takes the row's largest key with four DPP steps that stay inside the
// row (every lane of the row ends with it), records it and clears it; k
// rounds give the top-k in decreasing order.  Keys of absent experts are 0,
// below every finite logit.  Rows serve independent tokens, so one wave
// routes four tokens with the instructions of one.
// --------------------------------------------------------------------------
__device__ __forceinline__ unsigned float_order_key(float v) {
  unsigned u = (v == 0.0f) ? 0u : __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_order_key (-0.0 comes back as +0.0).
__device__ __forceinline__ float float_from_order_key(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kRouteRows = 4;  // tokens per wave (16-lane rows)

struct RouteFusedArgs {
  const uint16_t* x;     // [M,H] bf16, for the activation amax (may be null)
  int H;
  float* x_amax_part;    // [gridDim.x] per-workgroup amax of |x| (may be null)
  unsigned* h_amax;      // global amax of |h| to clear (may be null)
  int32_t* hist;         // [ceil(M/16)][E] expert counts of each routing workgroup's pairs (may be null)
};

// Top-k of the token whose logits row is `row` (always a readable row; with
// have = false its keys are all 0 and its results are meaningless).  l16 is
// the lane's index in its row; lane j < K of the row returns the j-th expert
// in *e_out and its softmax weight (over the k selected logits) in *w_out.
// NPL = ceil(E/16) keys per lane.  All 64 lanes must be active.  The NPL
// loads are unconditional (clamped to the row), so they are all in flight
// at once: with a conditional load per key the compiler waited for each
// before issuing the next, which cost 2.4 us for E = 128 and 4.8 us for
// E = 256 at decode sizes.
template <int NPL>
__device__ __forceinline__ void route_row(const float* __restrict__ row, bool have, int E, int K, int l16,
                                          int* e_out, float* w_out) {
  float lv[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) lv[i] = row[min(l16 + 16 * i, E - 1)];
  unsigned long long key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = l16 + 16 * i;
    key[i] = (have && e < E) ? (((unsigned long long)float_order_key(lv[i]) << 32) | (unsigned)(~(unsigned)e)) : 0ull;
  }
  int my_e = 0;
  float my_v = 0.0f, top_v = 0.0f;
  for (int j = 0; j < K; ++j) {
    // the lane's largest key by a pairwise tree (depth log2 NPL, where a
    // running maximum would chain NPL-1 dependent 64-bit selects)
    unsigned long long t[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) t[i] = key[i];
#pragma unroll
    for (int w = NPL / 2; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) t[i] = t[i + w] > t[i] ? t[i + w] : t[i];
    unsigned long long best = t[0];
    best = max_dpp_u64<kDppXor1>(best);
    best = max_dpp_u64<kDppXor2>(best);
    best = max_dpp_u64<kDppHalfMirror>(best);
    best = max_dpp_u64<kDppMirror>(best);
    const int e = (int)(~(unsigned)best);
    const float val = float_from_order_key((unsigned)(best >> 32));  // no dependent memory access
    if (j == 0) top_v = val;
    if (l16 == j) {
      my_e = e;
      my_v = val;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (l16 + 16 * i == e) key[i] = 0ull;
  }
  float ex = (l16 < K) ? expf(my_v - top_v) : 0.0f;
  float sum = ex;
  sum += dpp_f32<kDppXor1>(sum);
  sum += dpp_f32<kDppXor2>(sum);
  sum += dpp_f32<kDppHalfMirror>(sum);
  sum += dpp_f32<kDppMirror>(sum);
  *e_out = my_e;
  *w_out = ex / sum;
}

// Workgroup b routes tokens [16b, 16b+16) (when below M) and, with
// fa.x_amax_part, takes the amax of |x| over elements
// [b*kRouteAmaxChunk, (b+1)*kRouteAmaxChunk) of x, eight 16-byte loads in
// flight per thread; the grid covers both ranges (route_grid).
constexpr int kRouteAmaxChunk = 256 * 8 * 8;

__host__ __device__ inline int route_grid(int M, int64_t x_elems) {
  const int64_t r = (M + 4 * kRouteRows - 1) / (4 * kRouteRows);
  const int64_t q = (x_elems + kRouteAmaxChunk - 1) / kRouteAmaxChunk;
  return (int)(r > q ? r : q);
}

// Router logits, the step before routing: logits[m][e] = sum_t x[m][t] *
// W_g[e][t] for bf16 hidden states x [M][H] and router weights W_g [E][H],
// fp32 accumulation.  The pages' fused operation starts from the tokens
// (routing, data movement and expert products in one batched GPU operation:
// wagnersolution page, "AWS describes a fused MoE optimization ...", body).
// A workgroup computes 16 experts x 16*T tokens with the 16x16x32 bf16 MFMA
// (router rows are the A operand, tokens the B operand, as in the expert
// products); its 16 waves take the 32-element K-steps s = wave, wave+16, ...
// and the wave sums are added in wave order through LDS.  Every 16 x 16 tile
// is summed in that same order whatever T is, so a token's logits are the
// same bits on every call and in every batch; T = 4 (large M) reads each
// router row once per 64 tokens instead of once per 16.
template <int T>
static __global__ __launch_bounds__(1024) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wg, int M, int E, int H,
                                                             float* __restrict__ logits) {
  __shared__ f32x4 s_part[16][T][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int e0 = blockIdx.x * 16, m0 = blockIdx.y * 16 * T;
  // rows past E or M read the last valid row (their results are not stored)
  const uint16_t* pa = wg + (int64_t)min(e0 + r16, E - 1) * H + kq * 8;
  const uint16_t* pb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) pb[t] = x + (int64_t)min(m0 + 16 * t + r16, M - 1) * H + kq * 8;
  const int nsteps = H >> 5;
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = wave;
  for (; s + 48 < nsteps; s += 64) {  // four steps of loads in flight
    u32x4 a[4], b[4][T];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = *(const u32x4*)(pa + (s + 16 * u) * 32);
#pragma unroll
      for (int t = 0; t < T; ++t) b[u][t] = *(const u32x4*)(pb[t] + (s + 16 * u) * 32);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] = mfma_bf16(a[u], b[u][t], acc[t]);
  }
  for (; s < nsteps; s += 16) {
    const u32x4 a = *(const u32x4*)(pa + s * 32);
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = mfma_bf16(a, *(const u32x4*)(pb[t] + s * 32), acc[t]);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) s_part[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave >= T) return;
  // wave t adds the 16 wave sums of token tile t, in wave order
  f32x4 sum = s_part[0][wave][lane];
#pragma unroll
  for (int w = 1; w < 16; ++w) sum += s_part[w][wave][lane];
  // lane holds experts e0 + 4*kq + 0..3 of token m0 + 16*wave + r16
  const int m = m0 + 16 * wave + r16;
  if (m < M) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + 4 * kq + r;
      if (e < E) logits[(int64_t)m * E + e] = sum[r];
    }
  }
}

// Slot l16 of token m (l16 < K: the j-th routed expert e with its weight w;
// K <= l16 < K+S: shared expert E + (l16 - K) with weight one) into ids/wts
// (row stride K+S); returns whether the lane holds a pair of a real token,
// and its expert in *e.
__device__ __forceinline__ bool route_store(int m, int M, int E, int K, int S, int l16, int* e, float w,
                                            int32_t* __restrict__ ids, float* __restrict__ wts) {
  if (l16 >= K) {  // a shared expert's slot
    *e = E + (l16 - K);
    w = 1.0f;
  }
  const int KS = K + S;
  const bool pair = m < M && l16 < KS;
  if (pair) {
    ids[(int64_t)m * KS + l16] = *e;
    wts[(int64_t)m * KS + l16] = w;
  }
  return pair;
}

// S shared experts follow the E routed ones: slots K..K+S-1 of each token's
// row of ids/wts (stride K+S) name experts E..E+S-1 with weight one, and the
// expert counts cover all E+S.
template <int NPL>
static __global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int M, int E, int K, int S,
                                                         int32_t* __restrict__ ids, float* __restrict__ wts,
                                                         RouteFusedArgs fa) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int m0 = blockIdx.x * (4 * kRouteRows);
  if (m0 < M) {  // uniform over the workgroup
    const int m = m0 + wave * kRouteRows + (lane >> 4);
    int e;
    float w;
    route_row<NPL>(logits + (int64_t)min(m, M - 1) * E, m < M, E, K, l16, &e, &w);
    const bool pair = route_store(m, M, E, K, S, l16, &e, w, ids, wts);
    if (fa.hist) {  // this workgroup's expert counts, for the align step
      const int ES = E + S;
      __shared__ int s_hist[kMaxExperts];
      for (int i = threadIdx.x; i < ES; i += 256) s_hist[i] = 0;
      __syncthreads();
      if (pair) atomicAdd(&s_hist[e], 1);
      __syncthreads();
      for (int i = threadIdx.x; i < ES; i += 256) fa.hist[(int64_t)blockIdx.x * ES + i] = s_hist[i];
    }
  }
  if (fa.x_amax_part) {
    __shared__ float s_amax[4];
    const int64_t n = (int64_t)M * fa.H;  // multiple of 8
    const int64_t base = (int64_t)blockIdx.x * kRouteAmaxChunk + threadIdx.x * 8;
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = base + u * 256 * 8;
      v[u] = *(const u32x4*)(fa.x + (i < n ? i : 0));  // in-range address; counted only when i < n
    }
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + u * 256 * 8 < n)
#pragma unroll
        for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[u][q])), fabsf(bf16_hi(v[u][q]))));
    amax = wave_max(amax);
    if (lane == 0) s_amax[wave] = amax;
    __syncthreads();
    if (threadIdx.x == 0)
      fa.x_amax_part[blockIdx.x] = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
  }
  if (fa.h_amax && blockIdx.x == 0 && threadIdx.x == 0) *fa.h_amax = 0u;
}

// --------------------------------------------------------------------------
// Align: counting sort of the P = M*K pairs by expert, stable in the pair
// index, each expert's group padded with the sentinel P to a multiple of B.
//
// Workgroup g owns the chunk [1024*g, 1024*g + 1024) of pairs (256 per wave).
// Every workgroup histograms all P ids in LDS (total per expert, the part
// before its chunk, and per wave inside its chunk), so no workgroup waits for
// another and the result does not depend on scheduling.  A parallel scan
// gives the padded offsets; each wave then places its pairs in rounds of 64:
// lanes with the same expert find their rank by a match over the bits of the
// expert id (ballots), so placement keeps the pair order.  Workgroup 0 also
// writes the counts, offsets, sentinels, block map and the list of experts
// that hold at least one pair.
// --------------------------------------------------------------------------
constexpr int kAlignChunk = 1024;

struct AlignOut {
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* sorted_ids;    // [capacity]
  int32_t* block_expert;  // [n_blocks]
  int32_t* num_padded;    // [1]
  int32_t* active;        // [E] experts with pairs, increasing (may be null)
  int32_t* num_active;    // [1] (may be null)
  int n_blocks;
};

struct QuantXArgs {
  const uint16_t* x;         // [n] bf16
  int64_t n;                 // elements, multiple of 16
  const float* amax_part;    // [n_part] or null when static
  int n_part;
  const float* static_scale; // device fp32 or null
  uint8_t* xq;               // [n] e4m3
  float* scale_slot;         // s_x used (0 in block mode)
  int first_wg;              // first workgroup index of the quantisation part
  uint8_t* xs;               // block mode: E8M0 code of each 128-element group [n/128]; null = per tensor
};

// Sixteen bf16 (two 16-byte words) -> sixteen e4m3 bytes, scaled by r.
__device__ __forceinline__ u32x4 quant16_e4m3(const u32x4& a0, const u32x4& a1, float r) {
  u32x4 o;
  o[0] = pack_e4m3x4(bf16_lo(a0[0]) * r, bf16_hi(a0[0]) * r, bf16_lo(a0[1]) * r, bf16_hi(a0[1]) * r);
  o[1] = pack_e4m3x4(bf16_lo(a0[2]) * r, bf16_hi(a0[2]) * r, bf16_lo(a0[3]) * r, bf16_hi(a0[3]) * r);
  o[2] = pack_e4m3x4(bf16_lo(a1[0]) * r, bf16_hi(a1[0]) * r, bf16_lo(a1[1]) * r, bf16_hi(a1[1]) * r);
  o[3] = pack_e4m3x4(bf16_lo(a1[2]) * r, bf16_hi(a1[2]) * r, bf16_lo(a1[3]) * r, bf16_hi(a1[3]) * r);
  return o;
}

// Sixteen bf16 of a 128-element group whose other 112 elements the seven
// neighbouring lanes of an aligned 8-lane group hold -> sixteen e4m3 bytes
// with the group's power-of-two scale (OCP MX rule, block_scale_code); the
// group's first lane stores the scale code.  Every lane of the wave takes part
// (live: this lane's group is in range; whole groups are live or not).
__device__ __forceinline__ void quant16_block(const u32x4& a0, const u32x4& a1, bool live, uint8_t* dst,
                                              uint8_t* scale_dst, bool store_scale) {
  unsigned m = 0;  // |bf16| order is the order of the low 15 bits
#pragma unroll
  for (int c = 0; c < 4; ++c)
    m = max(m, max(max(a0[c] & 0x7fffu, (a0[c] >> 16) & 0x7fffu), max(a1[c] & 0x7fffu, (a1[c] >> 16) & 0x7fffu)));
  const float amax = max8(live ? __uint_as_float(m << 16) : 0.0f);
  const int code = block_scale_code(amax);
  if (live) {
    *(u32x4*)dst = quant16_e4m3(a0, a1, block_scale_recip(code));
    if (store_scale) *scale_dst = (uint8_t)code;
  }
}

// x -> e4m3 with the per-tensor scale (static, or amax/448 from the router's
// per-workgroup partial maxima), by a workgroup of NT threads, PER groups of
// 16 elements per thread (NT*16 apart, all loads issued before the first
// conversion): every workgroup first reduces the partial maxima, so a
// workgroup quantises enough elements to amortise that.
template <int NT, int PER = 1>
__device__ void quant_x_part(const QuantXArgs& q, int wg) {
  __shared__ float s_red[NT / 64];
  if (q.xs) {  // block mode: each 128-element group with its own scale, eight consecutive threads per group
    if (wg == 0 && threadIdx.x == 0) *q.scale_slot = 0.0f;
    const int64_t i0 = ((int64_t)wg * NT * PER + threadIdx.x) * 16;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int64_t i = i0 + (int64_t)p * NT * 16;
      const bool live = i < q.n;
      const int64_t src = live ? i : 0;
      quant16_block(*(const u32x4*)(q.x + src), *(const u32x4*)(q.x + src + 8), live, q.xq + i, q.xs + (i >> 7),
                    (threadIdx.x & 7) == 0);
    }
    return;
  }
  float s;
  if (q.static_scale) {
    s = *q.static_scale;
  } else {
    float a = 0.0f;
    for (int i = threadIdx.x; i < q.n_part; i += NT) a = fmaxf(a, q.amax_part[i]);
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) a = fmaxf(a, s_red[w]);
    s = scale_from_amax(a);
  }
  if (wg == 0 && threadIdx.x == 0) *q.scale_slot = s;
  const float r = 1.0f / s;
  const int64_t i0 = ((int64_t)wg * NT * PER + threadIdx.x) * 16;
  u32x4 lo[PER], hi[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int64_t i = i0 + (int64_t)p * NT * 16;
    if (i < q.n) {
      lo[p] = *(const u32x4*)(q.x + i);
      hi[p] = *(const u32x4*)(q.x + i + 8);
    }
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int64_t i = i0 + (int64_t)p * NT * 16;
    if (i < q.n) *(u32x4*)(q.xq + i) = quant16_e4m3(lo[p], hi[p], r);
  }
}

// elements quantised by one quantising workgroup of align_kernel
constexpr int kAlignQuantPer = 4;
constexpr int kAlignQuantPerWg = 256 * 16 * kAlignQuantPer;

// Exclusive scan of v over up to 512 entries held two per thread (256 threads).
// Returns the exclusive prefix for entry 2t; *total receives the sum.
__device__ __forceinline__ int block_excl_scan_pair(int v0, int v1, int* s_wtot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v0 + v1);
  if (lane == 63) s_wtot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wtot[w];
  *total = s_wtot[0] + s_wtot[1] + s_wtot[2] + s_wtot[3];
  __syncthreads();
  return before + incl - (v0 + v1);
}

// Per-routing-workgroup expert counts (from route_topk_kernel), usable when
// a routing workgroup's 16 tokens hold a whole number of pairs per 256 (k a
// power of two up to 16): rows r cover pairs [16k*r, 16k*(r+1)).
struct AlignHist {
  const int32_t* counts;  // [rows][E], or null: count the ids themselves
  int rows;
  int rows_per_wave;      // 256 / (16 k)
};

static __global__ __launch_bounds__(256) void align_kernel(const int32_t* __restrict__ ids, int P, int E, int B,
                                                    int log2B, int id_bits, int n_align_wgs, AlignOut o,
                                                    QuantXArgs q, AlignHist hist) {
  if ((int)blockIdx.x >= n_align_wgs) {
    quant_x_part<256, kAlignQuantPer>(q, blockIdx.x - n_align_wgs);
    return;
  }
  __shared__ int s_total[kMaxExperts];
  __shared__ int s_before[kMaxExperts];
  __shared__ int s_wave[4][kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_act[kMaxExperts + 1];
  __shared__ int s_wtot[4];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cb = blockIdx.x * kAlignChunk;
  const int ce = min(cb + kAlignChunk, P);

  for (int e = tid; e < E; e += 256) {
    s_total[e] = 0;
    s_before[e] = 0;
    s_wave[0][e] = s_wave[1][e] = s_wave[2][e] = s_wave[3][e] = 0;
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();

  constexpr int kHistBatch = 16;
  if (hist.counts) {
    // the routing workgroups' counts: every row adds to the totals, rows
    // before the chunk to s_before, the chunk's rows to their wave
    // thread t sums column e = t % E of rows t/E, t/E + rstep, ... in
    // registers (no division in the loop, one LDS atomic per column and
    // thread at the end)
    const int rw = hist.rows_per_wave;
    const int r0 = blockIdx.x * 4 * rw;
    const int rstep = E < 256 ? 256 / E : 1;
    for (int e0 = 0; e0 < E; e0 += 256) {
      const int e = e0 + (E < 256 ? tid % E : tid);
      const int rfirst = E < 256 ? tid / E : 0;
      if (e < E && rfirst < rstep) {
        int tot = 0, before = 0, wv[4] = {0, 0, 0, 0};
        for (int rb = rfirst; rb < hist.rows; rb += rstep * kHistBatch) {
          int cv[kHistBatch];
#pragma unroll
          for (int u = 0; u < kHistBatch; ++u) {
            const int r = rb + rstep * u;
            cv[u] = r < hist.rows ? hist.counts[(int64_t)r * E + e] : 0;
          }
#pragma unroll
          for (int u = 0; u < kHistBatch; ++u) {
            const int r = rb + rstep * u;
            tot += cv[u];
            if (r < r0) before += cv[u];
#pragma unroll
            for (int w = 0; w < 4; ++w)
              if (r >= r0 + w * rw && r < r0 + (w + 1) * rw) wv[w] += cv[u];
          }
        }
        atomicAdd(&s_total[e], tot);
        atomicAdd(&s_before[e], before);
#pragma unroll
        for (int w = 0; w < 4; ++w) atomicAdd(&s_wave[w][e], wv[w]);
      }
    }
  } else {
  // histogram of all P ids, 16 loads in flight per thread
  for (int f0 = tid; f0 < P; f0 += 256 * kHistBatch) {
    int ev[kHistBatch];
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
      const int f = f0 + 256 * u;
      ev[u] = f < P ? ids[f] : 0;
    }
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
      const int f = f0 + 256 * u;
      const int e = ev[u];
      if (f >= P) break;
      if ((unsigned)e >= (unsigned)E) {
        s_bad = 1;
        continue;
      }
      atomicAdd(&s_total[e], 1);
      if (f < cb)
        atomicAdd(&s_before[e], 1);
      else if (f < ce)
        atomicAdd(&s_wave[(f - cb) >> 8][e], 1);
    }
  }
  }
  __syncthreads();

  // padded sizes and active flags, two experts per thread
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  const int c0 = e0 < E ? s_total[e0] : 0, c1 = e1 < E ? s_total[e1] : 0;
  const int p0 = ((c0 + B - 1) >> log2B) << log2B, p1 = ((c1 + B - 1) >> log2B) << log2B;
  int tot_pad, tot_act;
  const int x0 = block_excl_scan_pair(p0, p1, s_wtot, &tot_pad);
  const int a0 = block_excl_scan_pair(c0 > 0, c1 > 0, s_wtot, &tot_act);
  if (e0 < E) {
    s_off[e0] = x0;
    s_act[e0] = a0;
  }
  if (e1 < E) {
    s_off[e1] = x0 + p0;
    s_act[e1] = a0 + (c0 > 0);
  }
  if (tid == 0) {
    s_off[E] = tot_pad;
    s_act[E] = tot_act;
  }
  __syncthreads();

  // starting position of each wave's pairs of expert e
  for (int e = tid; e < E; e += 256) {
    int run = s_off[e] + s_before[e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = s_wave[w][e];
      s_wave[w][e] = run;
      run += c;
    }
  }
  __syncthreads();

  // stable placement, 64 pairs per round
  const int wb = cb + wave * (kAlignChunk / 4);
  const int we = min(wb + kAlignChunk / 4, ce);
  for (int base = wb; base < we; base += 64) {
    const int f = base + lane;
    int e = (f < we) ? ids[f] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    unsigned long long match = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const unsigned long long m1 = __ballot(bit);
      match &= bit ? m1 : ~m1;
    }
    if (valid) {
      const int rank = __popcll(match & lanemask_lt(lane));
      const int grp = __popcll(match);
      const int pos = s_wave[wave][e] + rank;
      o.sorted_ids[pos] = f;
      if (rank == grp - 1) s_wave[wave][e] = pos + 1;
    }
  }

  if (blockIdx.x != 0) return;
  const int total = s_off[E];
  for (int e = tid; e < E; e += 256) {
    o.counts[e] = s_total[e];
    o.offsets[e] = s_off[e];
    if (o.active && s_total[e] > 0) o.active[s_act[e]] = e;
  }
  for (int e = wave; e < E; e += 4)  // sentinels: the lanes of a wave fill one expert's padding
    for (int p = s_off[e] + s_total[e] + lane; p < s_off[e + 1]; p += 64) o.sorted_ids[p] = P;
  if (tid == 0) {
    o.offsets[E] = total;
    *o.num_padded = s_bad ? -1 : total;
    if (o.num_active) *o.num_active = s_act[E];
  }
  for (int b = tid; b < o.n_blocks; b += 256) {
    const int pos = b << log2B;
    int ex = -1;
    if (pos < total) {
      int lo = 0, hi = E - 1;  // largest e with s_off[e] <= pos
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= pos)
          lo = mid;
        else
          hi = mid - 1;
      }
      ex = lo;
    }
    o.block_expert[b] = ex;
  }
}


// --------------------------------------------------------------------------
// Decode prologue: one launch of 1024-thread workgroups for token counts
// whose pairs fit one workgroup (M*K <= 1024) and at most 256 experts.  Workgroup 0 routes the tokens
// and does the stable sort-and-pad by expert (block 16); in fp8 mode
// workgroups 1..Q quantise x to e4m3, 16K elements each.  Each quantising
// workgroup first takes the per-tensor amax over all of x by itself (packed
// 16-bit maxima of the bf16 magnitudes, a short read of at most
// kSmallQuantElems elements that the first workgroup brings into L2), so no
// workgroup waits for another.
//
// Align here: wave w owns the pairs [64w, 64w+64).  A match over the bits of
// the expert id gives each pair its rank among the wave's pairs of the same
// expert and each (wave, expert) group its size; a prefix over waves and a
// scan over experts of the padded counts give every pair its position.
// --------------------------------------------------------------------------
constexpr int kSmallPairs = 1024;
constexpr int kSmallMaxExperts = 256;            // 16 keys per lane of the 1024-thread workgroup
constexpr int kSmallQuantPerWg = 1024 * 16;        // elements quantised per workgroup
constexpr int64_t kSmallQuantElems = 1LL << 17;    // largest M*H of this path (amax read per workgroup)

struct SmallQuant {
  const uint16_t* x;          // [M,H] bf16
  int H;
  const float* static_scale;  // device fp32 or null (dynamic amax/448)
  uint8_t* xq;                // [M,H] e4m3, null in bf16 mode
  float* scale_slot;          // s_x used (0 in block mode)
  unsigned* h_amax;           // cleared when non-null
  uint8_t* xs;                // block mode: E8M0 codes [M*H/128]; null = per tensor
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Quantising workgroup qb of the prologue (1024 threads).
__device__ __forceinline__ void prologue_quant(const SmallQuant& q, int64_t nx, int qb) {
  __shared__ float s_red[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (q.xs) {  // block mode: each 128-element group with its own scale
    if (qb == 0 && tid == 0) *q.scale_slot = 0.0f;
    const int64_t i = (int64_t)qb * kSmallQuantPerWg + (int64_t)tid * 16;
    const bool live = i < nx;
    const int64_t src = live ? i : 0;
    quant16_block(*(const u32x4*)(q.x + src), *(const u32x4*)(q.x + src + 8), live, q.xq + i, q.xs + (i >> 7),
                  (tid & 7) == 0);
    return;
  }
  float s;
  if (q.static_scale) {
    s = *q.static_scale;
  } else {
    // |bf16| ordering is the ordering of the low 15 bits as integers
    u16x2 m2 = {0, 0};
    for (int64_t i0 = (int64_t)tid * 8; i0 < nx; i0 += 4 * 8192) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * 8192;
        v[u] = *(const u32x4*)(q.x + (i < nx ? i : 0));  // in-range address; counted only when i < nx
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const unsigned keep = (i0 + u * 8192 < nx) ? 0x7fff7fffu : 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, v[u][c] & keep));
      }
    }
    float a = __uint_as_float((unsigned)max(m2[0], m2[1]) << 16);
    a = wave_max(a);
    if (lane == 0) s_red[wave] = a;
    __syncthreads();
    a = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w) a = fmaxf(a, s_red[w]);
    s = scale_from_amax(a);
  }
  if (qb == 0 && tid == 0) *q.scale_slot = s;
  const float r = 1.0f / s;
  const int64_t i = (int64_t)qb * kSmallQuantPerWg + (int64_t)tid * 16;
  if (i >= nx) return;
  *(u32x4*)(q.xq + i) = quant16_e4m3(*(const u32x4*)(q.x + i), *(const u32x4*)(q.x + i + 8), r);
}

// LDS of the one-wave align alone (wave_align).
struct WaveAlignLds {
  int tot[kMaxExperts];
  int off[kMaxExperts + 1];
  int act[kMaxExperts + 1];
};

// LDS of the one-workgroup align.
struct SmallAlignLds {
  int wc[16][kMaxExperts];  // per (wave, expert): group size, then start within the expert
  int tot[kMaxExperts];
  int off[kMaxExperts + 1];
  int act[kMaxExperts + 1];
  int scan[16];
};

// Stable sort-and-pad of P <= 1024 pairs with valid expert ids by one
// 1024-thread workgroup.  Requires L.wc zeroed and ids[0..P) in LDS, both
// before a barrier.
__device__ __forceinline__ void small_align(const int* s_ids, int P, int E, int log2B, int id_bits, const AlignOut& o,
                                            SmallAlignLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = 1 << log2B;
  // rank of each pair among its wave's pairs of the same expert
  const int f = tid;
  const bool valid = f < P;
  const int e = valid ? s_ids[f] : 0;
  unsigned long long match = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const unsigned long long m1 = __ballot(bit);
    match &= bit ? m1 : ~m1;
  }
  const int rank = valid ? __popcll(match & lanemask_lt(lane)) : 0;
  if (valid && rank == __popcll(match) - 1) L.wc[wave][e] = rank + 1;
  __syncthreads();
  // per expert: total, and the start of each wave's group within the expert
  for (int x = tid; x < E; x += 1024) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = L.wc[w][x];
      L.wc[w][x] = run;
      run += c;
    }
    L.tot[x] = run;
  }
  __syncthreads();
  // exclusive scan over experts of the padded sizes and of the active flags
  {
    const int x = tid;
    const int c = x < E ? L.tot[x] : 0;
    const int pad = ((c + B - 1) >> log2B) << log2B;
    const int v = pad | ((c > 0) << 20);  // padded size < 2^20 (P <= 1024, B <= 256)
    const int incl = wave_incl_scan(v);
    if (lane == 63) L.scan[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += L.scan[w];
    const int excl = before + incl - v;
    if (x < E) {
      L.off[x] = excl & 0xfffff;
      L.act[x] = excl >> 20;
    }
    if (x == E - 1) {
      L.off[E] = (excl + v) & 0xfffff;
      L.act[E] = (excl + v) >> 20;
    }
  }
  __syncthreads();
  if (valid) o.sorted_ids[L.off[e] + L.wc[wave][e] + rank] = f;
  const int total = L.off[E];
  for (int x = tid; x < E; x += 1024) {
    const int beg = L.off[x], end = L.off[x + 1];
    o.counts[x] = L.tot[x];
    o.offsets[x] = beg;
    for (int p = beg + L.tot[x]; p < end; ++p) o.sorted_ids[p] = P;
    for (int p = beg; p < end; p += B) o.block_expert[p >> log2B] = x;  // the expert's blocks
    if (o.active && L.tot[x] > 0) o.active[L.act[x]] = x;
  }
  for (int b = (total >> log2B) + tid; b < o.n_blocks; b += 1024) o.block_expert[b] = -1;  // blocks past the end
  if (tid == 0) {
    o.offsets[E] = total;
    *o.num_padded = total;
    if (o.num_active) *o.num_active = L.act[E];
  }
}

// The same sort-and-pad for P <= 64 pairs by one wave (wave 0 of the
// workgroup): a pair per lane, per-expert sums and the scan over experts in
// the wave's own LDS, so no workgroup barrier follows the routing barrier.
// The outputs are those of small_align bit for bit.  Requires ids[0..P) in
// LDS before a barrier.
template <class Lds>  // SmallAlignLds, or any LDS struct with the same tot, off and act arrays
__device__ __forceinline__ void wave_align(const int* s_ids, int P, int E, int log2B, int id_bits, const AlignOut& o,
                                           Lds& L) {
  const int lane = threadIdx.x & 63;
  const int B = 1 << log2B;
  const bool valid = lane < P;
  const int e = valid ? s_ids[lane] : 0;
  unsigned long long match = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const unsigned long long m1 = __ballot(bit);
    match &= bit ? m1 : ~m1;
  }
  const int rank = valid ? __popcll(match & lanemask_lt(lane)) : 0;
  for (int x = lane; x < E; x += 64) L.tot[x] = 0;
  if (valid && rank == 0) L.tot[e] = __popcll(match);
  // exclusive scan over experts of the padded sizes and active flags: lane
  // l takes experts [l*npe, (l+1)*npe)
  const int npe = (E + 63) >> 6;
  const int x0 = lane * npe;
  int pad_sum = 0, act_sum = 0;
  for (int x = x0; x < min(x0 + npe, E); ++x) {
    const int c = L.tot[x];
    pad_sum += ((c + B - 1) >> log2B) << log2B;
    act_sum += c > 0;
  }
  const int v = pad_sum | (act_sum << 20);  // padded total < 2^20 (P <= 64)
  int run = wave_incl_scan(v) - v;
  for (int x = x0; x < min(x0 + npe, E); ++x) {
    const int c = L.tot[x];
    L.off[x] = run & 0xfffff;
    L.act[x] = run >> 20;
    run += (((c + B - 1) >> log2B) << log2B) | ((c > 0) << 20);
  }
  if (x0 < E && x0 + npe >= E) {  // the lane holding the last expert
    L.off[E] = run & 0xfffff;
    L.act[E] = run >> 20;
  }
  if (valid) o.sorted_ids[L.off[e] + rank] = lane;
  const int total = L.off[E];
  for (int x = lane; x < E; x += 64) {
    const int beg = L.off[x], end = L.off[x + 1];
    o.counts[x] = L.tot[x];
    o.offsets[x] = beg;
    for (int p = beg + L.tot[x]; p < end; ++p) o.sorted_ids[p] = P;
    for (int p = beg; p < end; p += B) o.block_expert[p >> log2B] = x;
    if (o.active && L.tot[x] > 0) o.active[L.act[x]] = x;
  }
  for (int b = (total >> log2B) + lane; b < o.n_blocks; b += 64) o.block_expert[b] = -1;
  if (lane == 0) {
    o.offsets[E] = total;
    *o.num_padded = total;
    if (o.num_active) *o.num_active = L.act[E];
  }
}

template <int NPL>
static __global__ __launch_bounds__(1024) void prologue_small_kernel(const float* __restrict__ logits, int M, int E, int K,
                                                              int S, int32_t* __restrict__ ids, float* __restrict__ wts,
                                                              int log2B, int id_bits, AlignOut o, SmallQuant q) {
  if (blockIdx.x > 0) {
    prologue_quant(q, (int64_t)M * q.H, blockIdx.x - 1);
    return;
  }
  __shared__ int s_ids[kSmallPairs];
  __shared__ SmallAlignLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15;
  const int KS = K + S, P = M * KS;  // routed slots, then the shared experts' (as in route_topk_kernel)
  if (P > 64)  // the per-wave tables of small_align (wave_align needs none)
    for (int i = tid; i < 16 * kMaxExperts; i += 1024) (&L.wc[0][0])[i] = 0;
  // routing: four tokens per wave, 64 per pass of the 16 waves
  for (int mb = wave * kRouteRows; mb < M; mb += 16 * kRouteRows) {
    const int m = mb + (lane >> 4);
    int e;
    float w;
    route_row<NPL>(logits + (int64_t)min(m, M - 1) * E, m < M, E, K, l16, &e, &w);
    if (l16 >= K) {
      e = E + (l16 - K);
      w = 1.0f;
    }
    if (m < M && l16 < KS) {
      ids[m * KS + l16] = e;
      wts[m * KS + l16] = w;
      s_ids[m * KS + l16] = e;
    }
  }
  if (q.h_amax && tid == 0) *q.h_amax = 0u;
  __syncthreads();
  if (P <= 64) {
    if (wave == 0) wave_align(s_ids, P, E + S, log2B, id_bits, o, L);
    return;
  }
  small_align(s_ids, P, E + S, log2B, id_bits, o, L);
}

// Align of P <= 1024 router-produced pairs (valid ids) in workgroup 0 of
// 1024 threads; workgroups 1.. quantise x (16K elements each) from the
// router's partial maxima.
static __global__ __launch_bounds__(1024) void align_small_kernel(const int32_t* __restrict__ ids, int P, int E, int log2B,
                                                           int id_bits, AlignOut o, QuantXArgs q) {
  if (blockIdx.x > 0) {
    quant_x_part<1024>(q, blockIdx.x - 1);
    return;
  }
  __shared__ int s_ids[kSmallPairs];
  __shared__ SmallAlignLds L;
  const int tid = threadIdx.x;
  for (int i = tid; i < 16 * kMaxExperts; i += 1024) (&L.wc[0][0])[i] = 0;
  if (tid < P) s_ids[tid] = ids[tid];
  __syncthreads();
  small_align(s_ids, P, E, log2B, id_bits, o, L);
}

}  // namespace moe
