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

struct RouteFusedArgs {
  const uint16_t* x;     // [M,H] bf16, for the activation amax (may be null)
  int H;
  float* x_amax_part;    // [gridDim.x] per-workgroup amax of |x| (may be null)
  float* y_acc;          // [M,H] fp32 accumulator to clear (may be null)
  unsigned* h_amax;      // global amax of |h| to clear (may be null)
};

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
    const float* row = logits + (int64_t)m * E;
    unsigned long long key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      key[i] = (e < E) ? (((unsigned long long)float_order_key(row[e]) << 32) | (unsigned)(~(unsigned)e)) : 0ull;
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
      const float v = row[e];
      if (j == 0) top_v = v;
      if (lane == j) {
        my_e = e;
        my_v = v;
      }
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (lane + 64 * i == e) key[i] = 0ull;
    }
    const float ex = (lane < K) ? expf(my_v - top_v) : 0.0f;
    const float sum = wave_sum(ex);
    if (lane < K) {
      ids[(int64_t)m * K + lane] = my_e;
      wts[(int64_t)m * K + lane] = ex / sum;
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
    if (fa.y_acc) {
      float* yr = fa.y_acc + (int64_t)m * fa.H;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int t = lane * 4; t < fa.H; t += 64 * 4) *(f32x4*)(yr + t) = z;
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

}  // namespace moe
