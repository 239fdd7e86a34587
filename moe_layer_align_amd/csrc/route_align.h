// Router top-k and the sort-and-pad (align) kernels, plus the activation
// quantisation that rides along with the align launch in the fused path.
#pragma once

#include "moe_device.h"

namespace moe {

// --------------------------------------------------------------------------
// Router: one wavefront per token.
//
// Each lane holds NPL logits (experts lane, lane+64, ...).  A logit becomes a
// 64-bit key: high word = order-preserving image of the float (with -0.0
// mapped to +0.0 first), low word = ~expert, so the largest key is the
// largest logit and, among equal logits, the lowest expert.  k rounds of a
// wavefront max-reduction pick the top-k in decreasing order; the winner's
// key is cleared after each round.  Keys of absent experts are 0, below every
// finite logit.
// --------------------------------------------------------------------------
__device__ __forceinline__ unsigned float_order_key(float v) {
  unsigned u = (v == 0.0f) ? 0u : __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_order_key (-0.0 comes back as +0.0).
__device__ __forceinline__ float float_from_order_key(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct RouteFusedArgs {
  const uint16_t* x;     // [M,H] bf16, for the activation amax (may be null)
  int H;
  float* x_amax_part;    // [gridDim.x] per-workgroup amax of |x| (may be null)
  unsigned* h_amax;      // global amax of |h| to clear (may be null)
};

// Top-k of one token by the 64 lanes of a wave, from the lane's NPL logits
// (experts lane, lane+64, ...; absent experts hold any value and are masked
// by E); lane j < K returns the j-th expert in *e_out and its softmax weight
// in *w_out.
template <int NPL>
__device__ __forceinline__ void route_select(const float (&v)[NPL], int E, int K, int lane, int* e_out, float* w_out) {
  unsigned long long key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((unsigned long long)float_order_key(v[i]) << 32) | (unsigned)(~(unsigned)e)) : 0ull;
  }
  int my_e = 0;
  float my_v = 0.0f;
  float top_v = 0.0f;
  for (int j = 0; j < K; ++j) {
    unsigned long long best = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(~(unsigned)best);
    const float val = float_from_order_key((unsigned)(best >> 32));  // no dependent memory access
    if (j == 0) top_v = val;
    if (lane == j) {
      my_e = e;
      my_v = val;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
  }
  const float ex = (lane < K) ? expf(my_v - top_v) : 0.0f;
  const float sum = wave_sum(ex);
  *e_out = my_e;
  *w_out = ex / sum;
}

template <int NPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, int lane, float (&v)[NPL]) {
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = (lane + 64 * i < E) ? row[lane + 64 * i] : 0.0f;
}

template <int NPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int K, int lane, int* e_out,
                                            float* w_out) {
  float v[NPL];
  load_logits<NPL>(row, E, lane, v);
  route_select<NPL>(v, E, K, lane, e_out, w_out);
}

template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int M, int E, int K,
                                                         int32_t* __restrict__ ids, float* __restrict__ wts,
                                                         RouteFusedArgs fa) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = blockIdx.x * 4 + wave;
  __shared__ float s_amax[4];
  float amax = 0.0f;
  if (m < M) {
    int e;
    float w;
    route_token<NPL>(logits + (int64_t)m * E, E, K, lane, &e, &w);
    if (lane < K) {
      ids[(int64_t)m * K + lane] = e;
      wts[(int64_t)m * K + lane] = w;
    }
    if (fa.x_amax_part) {
      const uint16_t* xr = fa.x + (int64_t)m * fa.H;
      for (int t = lane * 8; t < fa.H; t += 64 * 8) {
        u32x4 v = *(const u32x4*)(xr + t);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          amax = fmaxf(amax, fabsf(bf16_lo(v[q])));
          amax = fmaxf(amax, fabsf(bf16_hi(v[q])));
        }
      }
    }
  }
  if (fa.x_amax_part) {
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
  float* scale_slot;         // s_x used
  int first_wg;              // first workgroup index of the quantisation part
};

// x -> e4m3 with the per-tensor scale (static, or amax/448 from the router's
// per-workgroup partial maxima).  16 elements per thread.
__device__ void quant_x_part(const QuantXArgs& q, int wg) {
  __shared__ float s_red[4];
  float s;
  if (q.static_scale) {
    s = *q.static_scale;
  } else {
    float a = 0.0f;
    for (int i = threadIdx.x; i < q.n_part; i += 256) a = fmaxf(a, q.amax_part[i]);
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    s = scale_from_amax(a);
  }
  if (wg == 0 && threadIdx.x == 0) *q.scale_slot = s;
  const float r = 1.0f / s;
  const int64_t i = ((int64_t)wg * 256 + threadIdx.x) * 16;
  if (i >= q.n) return;
  u32x4 a0 = *(const u32x4*)(q.x + i);
  u32x4 a1 = *(const u32x4*)(q.x + i + 8);
  u32x4 o;
  o[0] = pack_e4m3x4(bf16_lo(a0[0]) * r, bf16_hi(a0[0]) * r, bf16_lo(a0[1]) * r, bf16_hi(a0[1]) * r);
  o[1] = pack_e4m3x4(bf16_lo(a0[2]) * r, bf16_hi(a0[2]) * r, bf16_lo(a0[3]) * r, bf16_hi(a0[3]) * r);
  o[2] = pack_e4m3x4(bf16_lo(a1[0]) * r, bf16_hi(a1[0]) * r, bf16_lo(a1[1]) * r, bf16_hi(a1[1]) * r);
  o[3] = pack_e4m3x4(bf16_lo(a1[2]) * r, bf16_hi(a1[2]) * r, bf16_lo(a1[3]) * r, bf16_hi(a1[3]) * r);
  *(u32x4*)(q.xq + i) = o;
}

// Exclusive scan of v over up to 512 entries held two per thread (256 threads).
// Returns the exclusive prefix for entry 2t; *total receives the sum.
__device__ __forceinline__ int block_excl_scan_pair(int v0, int v1, int* s_wtot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v0 + v1, lane);
  if (lane == 63) s_wtot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wtot[w];
  *total = s_wtot[0] + s_wtot[1] + s_wtot[2] + s_wtot[3];
  __syncthreads();
  return before + incl - (v0 + v1);
}

__global__ __launch_bounds__(256) void align_kernel(const int32_t* __restrict__ ids, int P, int E, int B,
                                                    int log2B, int id_bits, int n_align_wgs, AlignOut o,
                                                    QuantXArgs q) {
  if ((int)blockIdx.x >= n_align_wgs) {
    quant_x_part(q, blockIdx.x - n_align_wgs);
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

  for (int f = tid; f < P; f += 256) {
    const int e = ids[f];
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
    for (int p = s_off[e] + s_total[e]; p < s_off[e + 1]; ++p) o.sorted_ids[p] = P;
    if (o.active && s_total[e] > 0) o.active[s_act[e]] = e;
  }
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
// Decode prologue in one workgroup of 1024 threads (16 waves), for token
// counts whose pairs fit one workgroup (M*K <= 1024): routing, the stable
// sort-and-pad by expert (block 16) and, in fp8 mode, the per-tensor
// activation scale and the e4m3 quantisation of x.  One launch replaces the
// router and align launches; no workgroup waits for another.
//
// Align here: wave w owns the pairs [64w, 64w+64).  A match over the bits of
// the expert id gives each pair its rank among the wave's pairs of the same
// expert and each (wave, expert) group its size; a prefix over waves and a
// scan over experts of the padded counts give every pair its position.
// --------------------------------------------------------------------------
constexpr int kSmallPairs = 1024;
constexpr int kSmallQuantChunks = 8;                                 // 8-element chunks of x per thread
constexpr int64_t kSmallQuantElems = 1024LL * 8 * kSmallQuantChunks;  // largest M*H quantised here

struct SmallQuant {
  const uint16_t* x;          // [M,H] bf16
  int H;
  const float* static_scale;  // device fp32 or null (dynamic amax/448)
  uint8_t* xq;                // [M,H] e4m3, null in bf16 mode
  float* scale_slot;          // s_x used
  unsigned* h_amax;           // cleared when non-null
};

template <int NPL>
__global__ __launch_bounds__(1024) void prologue_small_kernel(const float* __restrict__ logits, int M, int E, int K,
                                                              int32_t* __restrict__ ids, float* __restrict__ wts,
                                                              int log2B, int id_bits, AlignOut o, SmallQuant q) {
  __shared__ int s_ids[kSmallPairs];
  __shared__ int s_wc[16][kMaxExperts];   // per (wave, expert): group size, then start within the expert
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_act[kMaxExperts + 1];
  __shared__ int s_scan[16];
  __shared__ float s_red[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = M * K;
  const int B = 1 << log2B;

  // fp8: x is read once into registers (at most kSmallQuantChunks 8-element
  // chunks per thread), before the routing so that the loads overlap it
  constexpr int QC = kSmallQuantChunks;
  u32x4 xv[QC];
  const int64_t nx = q.xq ? (int64_t)M * q.H : 0;
#pragma unroll
  for (int c = 0; c < QC; ++c) {
    const int64_t i = ((int64_t)c * 1024 + tid) * 8;
    xv[c] = i < nx ? *(const u32x4*)(q.x + i) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int i = tid; i < 16 * kMaxExperts; i += 1024) (&s_wc[0][0])[i] = 0;
  // routing: all of the wave's logits rows are loaded before the first top-k
  {
    for (int m0 = wave; m0 < M; m0 += 16 * 4) {
      float rows[4][NPL];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + 16 * t;
        if (m < M) load_logits<NPL>(logits + (int64_t)m * E, E, lane, rows[t]);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + 16 * t;
        if (m < M) {
          int e;
          float w;
          route_select<NPL>(rows[t], E, K, lane, &e, &w);
          if (lane < K) {
            ids[m * K + lane] = e;
            wts[m * K + lane] = w;
            s_ids[m * K + lane] = e;
          }
        }
      }
    }
  }
  if (q.xq) {
    float s;
    if (q.static_scale) {
      s = *q.static_scale;
    } else {
      float a = 0.0f;
#pragma unroll
      for (int c = 0; c < QC; ++c)
#pragma unroll
        for (int h = 0; h < 4; ++h) a = fmaxf(a, fmaxf(fabsf(bf16_lo(xv[c][h])), fabsf(bf16_hi(xv[c][h]))));
      a = wave_max(a);
      if (lane == 0) s_red[wave] = a;
      __syncthreads();
      a = 0.0f;
#pragma unroll
      for (int w = 0; w < 16; ++w) a = fmaxf(a, s_red[w]);
      s = scale_from_amax(a);
    }
    if (tid == 0) *q.scale_slot = s;
    const float r = 1.0f / s;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const int64_t i = ((int64_t)c * 1024 + tid) * 8;
      if (i < nx) {
        const u32x4 v = xv[c];
        u32x2 out = {pack_e4m3x4(bf16_lo(v[0]) * r, bf16_hi(v[0]) * r, bf16_lo(v[1]) * r, bf16_hi(v[1]) * r),
                     pack_e4m3x4(bf16_lo(v[2]) * r, bf16_hi(v[2]) * r, bf16_lo(v[3]) * r, bf16_hi(v[3]) * r)};
        *(u32x2*)(q.xq + i) = out;
      }
    }
  }
  if (q.h_amax && tid == 0) *q.h_amax = 0u;
  __syncthreads();

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
  if (valid && rank == __popcll(match) - 1) s_wc[wave][e] = rank + 1;
  __syncthreads();
  // per expert: total, and the start of each wave's group within the expert
  for (int x = tid; x < E; x += 1024) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = s_wc[w][x];
      s_wc[w][x] = run;
      run += c;
    }
    s_tot[x] = run;
  }
  __syncthreads();
  // exclusive scan over experts of the padded sizes and of the active flags
  {
    const int x = tid;
    const int c = x < E ? s_tot[x] : 0;
    const int pad = ((c + B - 1) >> log2B) << log2B;
    const int v = pad | ((c > 0) << 20);  // padded size < 2^20 (P <= 1024, B <= 256)
    const int incl = wave_incl_scan(v, lane);
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_scan[w];
    const int excl = before + incl - v;
    if (x < E) {
      s_off[x] = excl & 0xfffff;
      s_act[x] = excl >> 20;
    }
    if (x == E - 1) {
      s_off[E] = (excl + v) & 0xfffff;
      s_act[E] = (excl + v) >> 20;
    }
  }
  __syncthreads();
  if (valid) o.sorted_ids[s_off[e] + s_wc[wave][e] + rank] = f;
  for (int x = tid; x < E; x += 1024) {
    o.counts[x] = s_tot[x];
    o.offsets[x] = s_off[x];
    for (int p = s_off[x] + s_tot[x]; p < s_off[x + 1]; ++p) o.sorted_ids[p] = P;
    if (o.active && s_tot[x] > 0) o.active[s_act[x]] = x;
  }
  if (tid == 0) {
    o.offsets[E] = s_off[E];
    *o.num_padded = s_off[E];
    if (o.num_active) *o.num_active = s_act[E];
  }
  for (int b = tid; b < o.n_blocks; b += 1024) {
    const int pos = b << log2B;
    int ex = -1;
    if (pos < s_off[E]) {
      int lo = 0, hi = E - 1;  // largest x with s_off[x] <= pos
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

}  // namespace moe
