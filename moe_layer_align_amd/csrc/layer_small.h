// The whole layer in one launch for tiny token counts (at most 64 pairs).
//
// The pages' point is one pass over the data with no round trips between
// separately launched steps: scaling, the products and the aggregation of the
// experts' outputs fused into one operation (The Neural Net, "AWS details MoE
// kernel fixes for SageMaker ...", body; ZICQ, "AWS Unveils MoE Kernel
// Optimizations ...", §Triton Backend Routing for FP8 Quantization).  At
// decode sizes the layer's launches, not its arithmetic, set the floor: the
// Qwen3-shaped layer at M = 1 streams 38 MB of weights (about 5 us) in four
// launches that take 30 us.
//
// One launch of at most one workgroup per CU (all co-resident: the host
// checks the kernel's occupancy), in four phases:
//  0. every workgroup routes all tokens, sorts and pads the pairs by expert in
//     its own LDS (one wave, as wave_align) and, in fp8, quantises x into the
//     workspace; no workgroup waits for another (the results are the same
//     bits everywhere, and the duplicated xq stores write the same bytes);
//  1. gate/up items (active expert x 16-feature tile, K split over the four
//     waves) walked round robin, h to the workspace; each workgroup records
//     its largest |h|;
//  -- grid barrier (layer1_barrier) --
//  2. down items (active expert x row tile of 32*(4/WKS) rows, K = I split
//     over WKS waves): per-pair fp32 partial outputs; with a dynamic h scale
//     every workgroup first reduces the recorded maxima;
//  -- grid barrier --
//  3. the weighted top-k combine: y[m] = bf16(sum_j w[m,j] * o_(m,j)), slots
//     in order, spread over all workgroups.
// The expert products are the decode bodies of gemm_decode.h (weight rows in
// the wide MFMA operand, tokens in the narrow one), fed with the LDS copy of
// the sort-and-pad result.
//
// Measured on MI355X (probe kernels, 256 workgroups): a kernel boundary costs
// about 6 us, a grid barrier 4.5 us at best (two-level counters below; one
// counter 9 us, per-workgroup flags 12 us, the cooperative-groups grid sync
// 60 us, and a cooperative launch 14 us more than a plain one).  So this
// layer saves little over the multi-launch path and is taken only on request
// (tuning single_launch = 1).
#pragma once

#include "gemm_decode.h"
#include "route_align.h"

namespace moe {

// ---------------------------------------------------------------- grid barrier
// Two-level counter barrier over the launch's workgroups: workgroup b arrives
// at the counter of group b % 8 (arrivals at one address serialise, about
// 12 ns each); the last of a group arrives at the top counter; the last of
// those advances the epoch that every workgroup waits for.  Counters return to
// zero as each barrier completes (the last arriver of a counter resets it,
// after every other arrival and before the epoch advances), so they are zero
// before every barrier: they live in a device array that the loader zeroes
// and that only this barrier touches.  A workgroup reads the epoch before it
// arrives (it cannot advance before that arrival) and waits for any other
// value.  Release/acquire at device scope around the arrivals carries each
// workgroup's global stores to the workgroups after the barrier.  The wait is
// bounded; a wait that runs out (which needs workgroups that never become
// resident, excluded by the host) raises *err and lets the kernel finish.
// Two launches of this layer on one GPU must not overlap (they would share
// the counters).
constexpr int kL1SyncStride = 32;               // words between counters (one 128-byte line each)
constexpr int kL1SyncGroups = 8;
constexpr int kL1SyncWords = kL1SyncStride * (kL1SyncGroups + 3);  // groups, top, epoch, error
constexpr int kL1SpinLimit = 1 << 22;           // about 0.1 s of s_sleep(1)

__device__ __forceinline__ void layer1_barrier(unsigned* sync) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int G = gridDim.x, ng = min(G, kL1SyncGroups), g = blockIdx.x % kL1SyncGroups;
    unsigned* top = sync + kL1SyncStride * kL1SyncGroups;
    unsigned* epoch = top + kL1SyncStride;
    unsigned* err = epoch + kL1SyncStride;
    const unsigned e0 = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned* grp = sync + kL1SyncStride * g;
    const unsigned gsize = (unsigned)((G - g + kL1SyncGroups - 1) / kL1SyncGroups);
    if (__hip_atomic_fetch_add(grp, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1 == gsize) {
      __hip_atomic_store(grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1 == (unsigned)ng) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(epoch, e0 + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    int spin = 0;
    while (__hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == e0) {
      __builtin_amdgcn_s_sleep(1);
      if (++spin > kL1SpinLimit) {
        __hip_atomic_fetch_add(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

constexpr int kLayer1Pairs = 64;       // pairs M*(k+S) of the single-launch layer (one-wave align)
constexpr int kLayer1Tokens = 16;      // four tokens per wave, four waves
constexpr int kLayer1Experts = 256;    // routed experts: 16 keys per lane
constexpr int kLayer1NPL = 16;
constexpr int kLayer1Sorted = kLayer1Pairs * 16;  // align capacity bound: P + min(E,P)*15 <= 64*16
constexpr int kLayer1LdsMax = 65536;   // LDS of one workgroup (static + the dynamic token slice)
constexpr int kLayer1MaxGrid = 1024;   // slots of the per-workgroup |h| maxima
constexpr int kTinyXElems = 16384;     // fp8 x of the two-launch layer: every gate/up workgroup's LDS copy

struct Layer1Args {
  const float* logits;   // [M][E] routed experts' logits
  const uint16_t* x;     // [M][H] bf16
  int M, E, K, S;        // tokens, routed experts, routed slots per token, shared experts
  int H, I;
  const uint8_t* w13;    // [E+S][2I][H]
  const uint8_t* w2;     // [E+S][H][I]
  const float* w13_scale;
  const float* w2_scale;
  int w_cs, w_es;        // weight scale per row / per expert (as Gemm1Args)
  const float* x_scale;  // fp8: static s_x, or null (dynamic)
  const float* h_scale;  // fp8: static s_h, or null (dynamic)
  uint8_t* xq;           // [M][H] e4m3 (fp8)
  uint8_t* h;            // [P][I] in the kernel's h format
  float* part;           // [P][H] fp32 partial outputs
  float* wg_hmax;        // [gridDim.x] largest |h| of each workgroup (dynamic h scale)
  uint16_t* y;           // [M][H] bf16
  int n_blocks;          // block_expert entries of the call's align layout (block 16)
  // optional outputs, written by workgroup 0 (null: not wanted)
  int32_t* ids_out;
  float* wts_out;
  AlignOut align_out;    // counts, offsets, sorted_ids, block_expert, num_padded (each may be null)
  float* scales_out;     // fp32[2]: s_x, s_h
  unsigned* sync;        // the barrier's counters (kL1SyncWords, zero between launches)
  float* sx_out;         // fp8: s_x in effect, for a later launch (may be null)
};

// Largest |x| over n bf16 elements by the whole workgroup (every thread gets it).
__device__ __forceinline__ float layer1_amax_bf16(const uint16_t* x, int64_t n, float* s_red4) {
  const int tid = threadIdx.x;
  unsigned m = 0;  // |bf16| order is the order of the low 15 bits
  for (int64_t i = (int64_t)tid * 8; i < n; i += 256 * 8) {
    const u32x4 v = *(const u32x4*)(x + i);
#pragma unroll
    for (int c = 0; c < 4; ++c) m = max(m, max(v[c] & 0x7fffu, (v[c] >> 16) & 0x7fffu));
  }
  float a = wave_max(__uint_as_float(m << 16));
  if ((tid & 63) == 0) s_red4[tid >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(s_red4[0], s_red4[1]), fmaxf(s_red4[2], s_red4[3]));
  __syncthreads();
  return a;
}

// The routing and sort-and-pad state every workgroup of the small layers
// keeps in LDS.
struct Layer1Lds {
  int ids[kLayer1Pairs];
  float wts[kLayer1Pairs];
  int counts[kMaxExperts], offsets[kMaxExperts + 1], active[kMaxExperts];
  int sorted[kLayer1Sorted];
  int block_expert[kLayer1Sorted / 16];
  int num_padded, num_active;
  WaveAlignLds al;
  float red4[4];
  float sx;
};

// Phase 0 of the small layers, in every workgroup: routing (token
// 4*wave + lane/16), the activation scale and quantisation into xq (fp8:
// a.xq, which every workgroup writes with the same bytes, or the workgroup's
// own LDS copy), and the one-wave sort-and-pad into LDS.  The lead workgroup
// also writes the routing, the sort-and-pad outputs that were asked for, and
// s_x.  An fp8 x of at most XC*4096 elements (XC 16-element chunks per
// thread) is loaded into registers before the routing, so that its loads are
// in flight with the logits' and x is read once.  Ends with the workgroup
// synchronised.
template <bool FP8, int XC = 2>
__device__ __forceinline__ void layer1_prologue(const Layer1Args& a, Layer1Lds& s, bool lead, uint8_t* xq) {
  constexpr int kXChunks = XC, kX2Reg = XC * 256 * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15;
  const int M = a.M, E = a.E, K = a.K, S = a.S, H = a.H;
  const int KS = K + S, ES = E + S, P = M * KS;
  const int64_t nx = (int64_t)M * H;
  const bool xreg = FP8 && nx <= kX2Reg;  // H is a multiple of 16
  // chunk c: elements 16*(tid + 256c) .. +16, loaded from the last chunk
  // where that is past x (no branch around the loads, so no wait for them
  // here; a repeated chunk leaves the largest |x| unchanged)
  u32x4 xr[2 * kXChunks];
  // a static s_x is read here too, beside the other loads
  const float sx_given = (xreg && a.x_scale) ? *a.x_scale : 0.0f;
  if (xreg) {
#pragma unroll
    for (int c = 0; c < kXChunks; ++c) {
      const int64_t i = min((int64_t)(tid + 256 * c) * 16, nx - 16);
      xr[2 * c] = *(const u32x4*)(a.x + i);
      xr[2 * c + 1] = *(const u32x4*)(a.x + i + 8);
    }
  }
  {
    const int m = wave * kRouteRows + (lane >> 4);
    int e;
    float w;
    route_row<kLayer1NPL>(a.logits + (int64_t)min(m, M - 1) * E, m < M, E, K, l16, &e, &w);
    if (l16 >= K) {  // a shared expert's slot
      e = E + (l16 - K);
      w = 1.0f;
    }
    if (m < M && l16 < KS) {
      s.ids[m * KS + l16] = e;
      s.wts[m * KS + l16] = w;
      if (lead && a.ids_out) a.ids_out[m * KS + l16] = e;
      if (lead && a.wts_out) a.wts_out[m * KS + l16] = w;
    }
  }
  if constexpr (FP8) {
    float sx;
    if (xreg) {
      if (a.x_scale) {
        sx = sx_given;
      } else {  // largest |x| as layer1_amax_bf16 takes it, from the registers
        unsigned m = 0;
#pragma unroll
        for (int c = 0; c < 2 * kXChunks; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) m = max(m, max(xr[c][q] & 0x7fffu, (xr[c][q] >> 16) & 0x7fffu));
        float am = wave_max(__uint_as_float(m << 16));
        if (lane == 0) s.red4[wave] = am;
        __syncthreads();
        am = fmaxf(fmaxf(s.red4[0], s.red4[1]), fmaxf(s.red4[2], s.red4[3]));
        sx = scale_from_amax(am);
      }
      const float r = 1.0f / sx;
#pragma unroll
      for (int c = 0; c < kXChunks; ++c) {
        const int64_t i = (int64_t)(tid + 256 * c) * 16;
        if (i < nx) *(u32x4*)(xq + i) = quant16_e4m3(xr[2 * c], xr[2 * c + 1], r);
      }
    } else {
      sx = a.x_scale ? *a.x_scale : scale_from_amax(layer1_amax_bf16(a.x, nx, s.red4));
      const float r = 1.0f / sx;
      for (int64_t i = (int64_t)tid * 16; i < nx; i += 256 * 16)
        *(u32x4*)(xq + i) = quant16_e4m3(*(const u32x4*)(a.x + i), *(const u32x4*)(a.x + i + 8), r);
    }
    if (tid == 0) s.sx = sx;
    if (lead && tid == 0 && a.scales_out) a.scales_out[0] = sx;
    if (lead && tid == 0 && a.sx_out) *a.sx_out = sx;
  }
  __syncthreads();
  if (wave == 0) {
    int bits = 0;
    while ((1 << bits) < ES) ++bits;
    const AlignOut lo{s.counts, s.offsets, s.sorted, s.block_expert, &s.num_padded, s.active, &s.num_active,
                      a.n_blocks};
    wave_align(s.ids, P, ES, 4, bits, lo, s.al);
  }
  __syncthreads();
  if (lead) {  // the call's sort-and-pad outputs, when asked for
    const AlignOut& o = a.align_out;
    for (int x = tid; x < ES; x += 256) {
      if (o.counts) o.counts[x] = s.counts[x];
      if (o.offsets) o.offsets[x] = s.offsets[x];
    }
    if (o.offsets && tid == 0) o.offsets[ES] = s.offsets[ES];
    if (o.num_padded && tid == 0) *o.num_padded = s.num_padded;
    if (o.sorted_ids)
      for (int p = tid; p < s.num_padded; p += 256) o.sorted_ids[p] = s.sorted[p];
    if (o.block_expert)
      for (int b = tid; b < a.n_blocks; b += 256) o.block_expert[b] = s.block_expert[b];
  }
}

template <bool FP8, int HFMT, int WKS>
static __global__ __launch_bounds__(256) void layer1_kernel(Layer1Args a) {
  constexpr int U1 = FP8 ? 2 : 4, U2 = FP8 ? 1 : 4;
  constexpr int TPW2 = 4 / WKS;  // row tiles of 32 per down item
  __shared__ Layer1Lds s;
  __shared__ f32x4 s_red[3 * 2 * 64];  // three waves' partial tiles (K split over four waves, one token tile)
  __shared__ unsigned s_hamax;
  extern __shared__ __align__(16) uint8_t s_tok[];  // down product's token slice (dynamic h scale)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = a.M, K = a.K, S = a.S, H = a.H, I = a.I;
  const int KS = K + S, P = M * KS;
  const bool lead = blockIdx.x == 0;
  float* const s_red4 = s.red4;
  const int* const s_active = s.active;
  const int* const s_offsets = s.offsets;
  const int* const s_counts = s.counts;
  const float* const s_wts = s.wts;

  // ---- phase 0: routing, activation scale and quantisation, sort and pad
  layer1_prologue<FP8>(a, s, lead, a.xq);

  const Segments seg{s.sorted, s.offsets, s.counts, s.active, &s.num_active, 0};
  const int nact = s.num_active;
  auto grid_barrier = [&] { layer1_barrier(a.sync); };

  auto layer = [&](auto pc_tag) {
    constexpr int WS = decltype(pc_tag)::value ? kWsRow : kWsTensor;
    // ---- phase 1: gate/up items (expert, 16-feature tile)
    Gemm1Args g1{a.w13, FP8 ? a.xq : (const uint8_t*)a.x, seg, H, I, KS, a.w13_scale, &s.sx, a.h_scale, a.h,
                 nullptr};
    g1.w_cs = a.w_cs;
    g1.w_es = a.w_es;
    const int t1 = I / 16;
    float hmax = 0.0f;
    for (int it = blockIdx.x; it < nact * t1; it += gridDim.x) {
      __syncthreads();  // the previous item's reduction tiles are consumed
      const int e = s_active[it / t1];
      hmax = fmaxf(hmax, gemm1_body<FP8, HFMT, 1, 1, U1, 4, WS>(g1, s_red, e, s_offsets[e], s_counts[e], 0,
                                                                 it % t1));
    }
    if constexpr (HFMT == H_F32) {
      hmax = wave_max(hmax);
      if (lane == 0) s_red4[wave] = hmax;
      __syncthreads();
      if (tid == 0) a.wg_hmax[blockIdx.x] = fmaxf(fmaxf(s_red4[0], s_red4[1]), fmaxf(s_red4[2], s_red4[3]));
    }
    grid_barrier();

    // ---- phase 2: down items (expert, 32*TPW2-row tile), one K slice
    float sh = 1.0f;
    if constexpr (HFMT == H_F32) {
      float m = 0.0f;
      for (int i = tid; i < (int)gridDim.x; i += 256) m = fmaxf(m, a.wg_hmax[i]);
      m = wave_max(m);
      __syncthreads();
      if (lane == 0) s_red4[wave] = m;
      __syncthreads();
      if (tid == 0) s_hamax = __float_as_uint(fmaxf(fmaxf(s_red4[0], s_red4[1]), fmaxf(s_red4[2], s_red4[3])));
      __syncthreads();
      sh = scale_from_amax(__uint_as_float(s_hamax));
    } else if constexpr (FP8) {
      sh = *a.h_scale;
    }
    if (FP8 && lead && tid == 0 && a.scales_out) a.scales_out[1] = sh;
    Gemm2Args g2{a.w2, a.h, seg, nullptr, H, I, KS, 1, a.w2_scale, a.h_scale, &s_hamax, a.part, P};
    g2.w_cs = a.w_cs;
    g2.w_es = a.w_es;
    const int t2 = H / (32 * TPW2);
    for (int it = blockIdx.x; it < nact * t2; it += gridDim.x) {
      __syncthreads();  // the previous item's token slice and reduction tiles are consumed
      const int e = s_active[it / t2];
      gemm2_body<FP8, HFMT, 1, 1, U2, WKS, WS>(g2, s_tok, s_red, e, s_offsets[e], s_counts[e], 0, 0, it % t2);
    }
    grid_barrier();
  };
  if constexpr (FP8) {
    if (a.w_cs)
      layer(std::true_type{});
    else
      layer(std::false_type{});
  } else {
    layer(std::false_type{});
  }

  // ---- phase 3: y[m, n..n+3] = bf16(sum_j w[m,j] * part[m*KS+j][n..n+3]), j ascending
  const int64_t groups = (int64_t)M * H / 4;
  for (int64_t g = (int64_t)blockIdx.x * 256 + tid; g < groups; g += (int64_t)gridDim.x * 256) {
    const int m = (int)(g * 4 / H), n = (int)(g * 4 - (int64_t)m * H);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < KS; ++j) acc += s_wts[m * KS + j] * *(const f32x4*)(a.part + (int64_t)(m * KS + j) * H + n);
    *(uint2*)(a.y + (int64_t)m * H + n) = uint2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  }
}

// ---------------------------------------------------------------- two launches for tiny M
// The layer in two launches where it fits the single-launch layer's limits:
//   1. tiny_gate_up_kernel: every workgroup runs phase 0 above (the routing,
//      quantisation and sort-and-pad of a few tokens cost less than a launch;
//      fp8 x is quantised into the workgroup's LDS, where its gate/up product
//      reads it) and then takes gate/up items it = blockIdx.x, + gridDim.x, ... exactly
//      as the single-launch layer's phase 1 does; with a dynamic h scale it
//      writes its largest |h| to wg_hmax[blockIdx.x] (no counter to clear);
//   2. down_token_kernel (gemm_decode.h): the down product and the weighted
//      combine per token, reducing those maxima for s_h.
// The kernel boundary orders the two launches, so no grid barrier is needed;
// the arithmetic is the multi-launch path's, bit for bit.
template <bool FP8, int HFMT, int XC>
static __global__ __launch_bounds__(256) void tiny_gate_up_kernel(Layer1Args a) {
  constexpr int U1 = FP8 ? 2 : 4;
  __shared__ Layer1Lds s;
  __shared__ f32x4 s_red[3 * 2 * 64];  // three waves' partial tiles (K split over four waves, one token tile)
  __shared__ __align__(16) uint8_t s_xq[FP8 ? kTinyXElems : 16];  // this workgroup's e4m3 copy of x
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  layer1_prologue<FP8, XC>(a, s, blockIdx.x == 0, s_xq);
  const Segments seg{s.sorted, s.offsets, s.counts, s.active, &s.num_active, 0};
  const int KS = a.K + a.S, t1 = a.I / 16, nact = s.num_active;
  auto run = [&](auto pc_tag) {
    constexpr int WS = decltype(pc_tag)::value ? kWsRow : kWsTensor;
    Gemm1Args g1{a.w13, FP8 ? s_xq : (const uint8_t*)a.x, seg, a.H, a.I, KS, a.w13_scale, &s.sx, a.h_scale, a.h,
                 nullptr};
    g1.w_cs = a.w_cs;
    g1.w_es = a.w_es;
    float hmax = 0.0f;
    for (int it = blockIdx.x; it < nact * t1; it += gridDim.x) {
      __syncthreads();  // the previous item's reduction tiles are consumed
      const int e = s.active[it / t1];
      hmax = fmaxf(hmax, gemm1_body<FP8, HFMT, 1, 1, U1, 4, WS>(g1, s_red, e, s.offsets[e], s.counts[e], 0,
                                                                 it % t1));
    }
    return hmax;
  };
  float hmax;
  if constexpr (FP8)
    hmax = a.w_cs ? run(std::true_type{}) : run(std::false_type{});
  else
    hmax = run(std::false_type{});
  if constexpr (HFMT == H_F32) {
    hmax = wave_max(hmax);
    __syncthreads();
    if (lane == 0) s.red4[wave] = hmax;
    __syncthreads();
    if (tid == 0) a.wg_hmax[blockIdx.x] = fmaxf(fmaxf(s.red4[0], s.red4[1]), fmaxf(s.red4[2], s.red4[3]));
  }
}

}  // namespace moe
