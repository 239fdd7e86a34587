// Grouped expert products for large token counts (prefill), gfx950 fp8 MFMA.
//
// At prefill every active expert holds hundreds to thousands of tokens, so the
// products are compute-bound and both operands are reused: a workgroup
// computes a 256 x 128 tile (256 weight rows x 128 tokens of one expert) and
// stages both operands through LDS, K-step by K-step.  The token dimension is
// grouped by the align step with a block of 128: block b holds tokens of
// expert block_expert[b] only, padded with the sentinel, so a workgroup's
// tokens share one expert.  Weight rows stay the MFMA's A operand and tokens
// the B operand, as in the decode kernels; the 32x32x64 fp8 MFMA is used,
// each of the eight waves owning a 64 x 64 sub-tile (2 x 2 MFMA tiles).
//
// Grid: one dimension, mapped to (weight tile, token block) so that each
// weight tile stays on one XCD (pf_map), where its reuse across the token
// blocks of one expert hits that XCD's L2.
//
// Pipeline: both operand tiles of each 128-byte K-step are loaded from global
// memory straight into a three-deep LDS ring (direct-to-LDS loads, no staging
// registers), two steps ahead of the MFMAs, with one barrier per step.
#pragma once

#include <type_traits>

#include "moe_device.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// 32x32x64 OCP e4m3 x e4m3 -> fp32, unit block scales.  A: lane l holds 32
// bytes of row l%32; B: 32 bytes of column l%32, at the same k positions.
// C: lane l holds column l%32, rows 8*(v/4) + 4*(l/32) + v%4, v = 0..15.
__device__ __forceinline__ f32x16 mfma32_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Wait until at most N vector-memory operations of this wave are
// outstanding (the LDS-DMA loads below are vector-memory operations whose
// destination the compiler does not track).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt[3:0] | expcnt 7 [6:4] | lgkmcnt 15 [11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the LDS ring: waits for this wave's own LDS reads
// only (lgkmcnt 0), not for its outstanding global-to-LDS loads, whose
// completion the K-loop waits for explicitly; the memory clobber keeps the
// compiler from moving LDS accesses across it.  (__syncthreads() would also
// wait for every vector-memory operation, draining the prefetch queue.)
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int kPfTok = 128;                          // tokens per workgroup (the align block)
constexpr int kPfRows = 256;                         // weight rows per workgroup
constexpr int kPfBK = 128;                           // K bytes per step (fp8): two MFMA k-steps
constexpr int kPfStages = 3;                         // LDS ring depth
constexpr int kPfStageA = kPfRows * kPfBK;           // 32 KB
constexpr int kPfStageB = kPfTok * kPfBK;            // 16 KB
constexpr int kPfStage = kPfStageA + kPfStageB;      // 48 KB
constexpr int kPfLds = kPfStages * kPfStage;         // 144 KB: one workgroup of 8 waves per CU
constexpr int kPfThreads = 512;

struct PrefillSeg {
  const int32_t* sorted_ids;    // [capacity] pair ids grouped by expert, block 128
  const int32_t* block_expert;  // [capacity/128]
  const int32_t* offsets;       // [E+1]
  const int32_t* counts;        // [E]
  const int32_t* num_padded;    // [1]
};

// LDS layout of an operand tile in one stage: rows of 128 bytes, the eight
// 16-byte chunks of row r stored at chunk position c ^ (r & 7), so the MFMA
// fragment reads (32 rows, same chunk) spread over all banks.
__device__ __forceinline__ int pf_swz(int row, int chunk) { return row * kPfBK + ((chunk ^ (row & 7)) << 4); }

// Workgroup -> (weight tile, token block), XCD-aware.  Workgroups are handed
// to the eight XCDs round robin by linear id; XCD c owns weight tiles c, c+8,
// ... for every block, and the T % 8 tiles left over are shared out as
// contiguous (tile, block) ranges, so each weight tile is read by as few XCDs
// (L2s) as possible.  nblk must be a multiple of 8.
__device__ __forceinline__ void pf_map(int L, int T, int nblk, int* tile, int* blk) {
  const int c = L & 7, j = L >> 3;
  const int full = T >> 3, rem = T & 7;
  if (j < full * nblk) {
    *blk = j / full;
    *tile = c + 8 * (j - *blk * full);
  } else {
    const int per = rem * nblk / 8;
    const int p = c * per + (j - full * nblk);
    *tile = 8 * full + p / nblk;
    *blk = p - (p / nblk) * nblk;
  }
}

// ---------------------------------------------------------------- products
struct PrefillArgs {
  const uint8_t* w;        // W13 [E][2I][H] or W2 [E][H][I], e4m3
  const uint8_t* act;      // gate/up: xq [M][H]; down: hq [P][I], e4m3
  PrefillSeg seg;
  const float* topk_w;     // [P] (down)
  int H, I, top_k, P;
  int tiles, nblk;         // weight tiles (2I/256 or H/256) and token blocks (rounded up to 8)
  const float* w_scale;    // s_w13 or s_w2
  const float* a_scale;    // gate/up: s_x in effect; down: static s_h (null = dynamic)
  const unsigned* h_amax;  // down with dynamic scale: max |h| (float bits)
  const float* h_scale;    // gate/up: static s_h (null = dynamic: h written as bf16)
  uint8_t* out;            // gate/up: h; down: part [P][H] bf16
  unsigned* h_amax_out;    // gate/up with dynamic scale
};

// MODE 0: gate/up product, tile rows = 128 gate + 128 up rows of the same 128
//   features, epilogue SiLU(g)*u -> h.  HDYN: h stored as bf16 with a running
//   amax (quantised by prefill_quant_h_kernel), else as e4m3 with the static
//   scale.
// MODE 1: down product, tile rows = 256 output features, epilogue
//   w[pair] * s_h * s_w2 * acc -> bf16 part[pair][feature].
//
// Eight waves: wave (wr = 0..3, wc = 0..1) owns 64 weight rows x 64 tokens
// (2 x 2 MFMA tiles; in MODE 0 the 32 gate and the 32 up rows of the same 32
// features).  Each 128-byte K-step: every wave DMA-loads 32 rows of the A
// tile and 16 rows of the B tile (six 1 KB load instructions, lane i filling
// bytes 16i..16i+15 of an 8-row block) into a three-deep LDS ring two steps
// ahead; one barrier per step; 8 MFMAs per wave per step.
template <int MODE, bool HDYN>
__global__ __launch_bounds__(kPfThreads) void prefill_gemm_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  int tile, blk;
  pf_map(blockIdx.x, a.tiles, a.nblk, &tile, &blk);
  const int npad = *a.seg.num_padded;
  if (blk * kPfTok >= npad) return;
  const int e = a.seg.block_expert[blk];
  if (e < 0) return;
  const int seg_end = a.seg.offsets[e] + a.seg.counts[e];  // first padding slot of the expert
  const int tok0 = blk * kPfTok;
  const int ntok = min(kPfTok, seg_end - tok0);            // valid tokens of the block (>= 1)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the wave's branches scalar
  const int K = MODE == 0 ? a.H : a.I;                        // contraction length (bytes)
  const int64_t wrows = MODE == 0 ? 2 * a.I : a.H;            // rows of one expert's weight

  // DMA sources of this lane: A rows 32*wave + 8*q + lane/8 (q < 4), B rows
  // 16*wave + 8*q + lane/8 (q < 2), logical chunk (lane%8) ^ (row & 7)
  const int lrow = lane >> 3, lchunk = lane & 7;
  const uint8_t* srcA[4];
  const uint8_t* srcB[2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 32 * wave + 8 * q + lrow;
    int64_t wrow;
    if (MODE == 0) {
      const int f0 = tile * 128;
      wrow = row < 128 ? f0 + row : a.I + f0 + (row - 128);
    } else {
      wrow = (int64_t)tile * kPfRows + row;
    }
    srcA[q] = a.w + ((int64_t)e * wrows + wrow) * K + ((lchunk ^ (row & 7)) << 4);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * wave + 8 * q + lrow;
    // padding slots read the first token of the block (their results are dropped)
    const int f = a.seg.sorted_ids[tok0 + (row < ntok ? row : 0)];
    const int64_t brow = MODE == 0 ? f / a.top_k : f;
    srcB[q] = a.act + brow * K + ((lchunk ^ (row & 7)) << 4);
  }
  auto issue = [&](int s) {  // DMA of K-step s into ring slot s % kPfStages
    lds_u8* base = smem + (s % kPfStages) * kPfStage;
    const int kb = s * kPfBK;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(srcA[q] + kb),
                                       (void __attribute__((address_space(3)))*)(base + (32 * wave + 8 * q) * kPfBK),
                                       16, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcB[q] + kb),
          (void __attribute__((address_space(3)))*)(base + kPfStageA + (16 * wave + 8 * q) * kPfBK), 16, 0, 0);
  };

  // wave sub-tile: two 32-row A tiles and 64 tokens
  const int wr = wave & 3, wc = wave >> 2;
  const int arow0 = MODE == 0 ? 32 * wr : 64 * wr;             // gate rows (MODE 0)
  const int arow1 = MODE == 0 ? 128 + 32 * wr : 64 * wr + 32;  // up rows of the same features (MODE 0)
  const int brow0 = 64 * wc;
  const bool live0 = brow0 < ntok, live1 = brow0 + 32 < ntok;  // 32-token sub-tiles that hold tokens
  // fragment addresses within a stage: row l%32 of each tile, k-step ks uses
  // chunks 4*ks + 2*(l/32) and +1
  const int fr = lane & 31, fc = (lane >> 5) * 2;
  int offA0[2][2], offA1[2][2], offB0[2][2], offB1[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      offA0[ks][c] = pf_swz(arow0 + fr, 4 * ks + fc + c);
      offA1[ks][c] = pf_swz(arow1 + fr, 4 * ks + fc + c);
      offB0[ks][c] = kPfStageA + pf_swz(brow0 + fr, 4 * ks + fc + c);
      offB1[ks][c] = kPfStageA + pf_swz(brow0 + 32 + fr, 4 * ks + fc + c);
    }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / kPfBK;
  // K-loop with NJ (0, 1 or 2) of the wave's 32-token sub-tiles multiplied;
  // one version per NJ so that the loop body has no branches
  auto kloop = [&](auto nj_tag) {
    constexpr int NJ = decltype(nj_tag)::value;
    issue(0);
    if (nk > 1) issue(1);
    for (int s = 0; s < nk; ++s) {
      // this wave's DMA of step s is complete once at most the next step's six loads are in flight
      if (s + 1 < nk)
        wait_vm<6>();
      else
        wait_vm<0>();
      ring_barrier();  // every wave's step-s data is in LDS; slot (s+2)%3 is no longer read
      if (s + 2 < nk) issue(s + 2);
      if constexpr (NJ > 0) {
        const lds_u8* st = smem + (s % kPfStages) * kPfStage;
        u32x4 a0[2][2], a1[2][2], b0[2][2], b1[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            a0[ks][c] = *(const __attribute__((address_space(3))) u32x4*)(st + offA0[ks][c]);
            a1[ks][c] = *(const __attribute__((address_space(3))) u32x4*)(st + offA1[ks][c]);
            b0[ks][c] = *(const __attribute__((address_space(3))) u32x4*)(st + offB0[ks][c]);
            if constexpr (NJ > 1) b1[ks][c] = *(const __attribute__((address_space(3))) u32x4*)(st + offB1[ks][c]);
          }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          acc[0][0] = mfma32_fp8(a0[ks][0], a0[ks][1], b0[ks][0], b0[ks][1], acc[0][0]);
          acc[1][0] = mfma32_fp8(a1[ks][0], a1[ks][1], b0[ks][0], b0[ks][1], acc[1][0]);
          if constexpr (NJ > 1) {
            acc[0][1] = mfma32_fp8(a0[ks][0], a0[ks][1], b1[ks][0], b1[ks][1], acc[0][1]);
            acc[1][1] = mfma32_fp8(a1[ks][0], a1[ks][1], b1[ks][0], b1[ks][1], acc[1][1]);
          }
        }
      }
    }
  };
  if (live1)
    kloop(std::integral_constant<int, 2>{});
  else if (live0)
    kloop(std::integral_constant<int, 1>{});
  else
    kloop(std::integral_constant<int, 0>{});

  // epilogue
  const int col = lane & 31, rq = (lane >> 5) * 4;
  if (MODE == 0) {
    const float deq = (*a.a_scale) * (*a.w_scale);
    const float rhs = HDYN ? 1.0f : 1.0f / *a.h_scale;
    float hmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = brow0 + 32 * j + col;
      if (t < ntok) {
        const int f = a.seg.sorted_ids[tok0 + t];
        const int fbase = tile * 128 + 32 * wr;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gt = acc[0][j][4 * g + q] * deq;
            const float up = acc[1][j][4 * g + q] * deq;
            hv[q] = gt / (1.0f + expf(-gt)) * up;
            hmax = fmaxf(hmax, fabsf(hv[q]));
          }
          const int64_t idx = (int64_t)f * a.I + fbase + 8 * g + rq;
          if (HDYN) {
            u32x2 o = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            *(u32x2*)(a.out + idx * 2) = o;
          } else {
            *(unsigned*)(a.out + idx) = pack_e4m3x4(hv[0] * rhs, hv[1] * rhs, hv[2] * rhs, hv[3] * rhs);
          }
        }
      }
    }
    if (HDYN) {
      hmax = wave_max(hmax);
      if (lane == 0) atomicMax(a.h_amax_out, __float_as_uint(hmax));
    }
  } else {
    const float sh = HDYN ? scale_from_amax(__uint_as_float(*a.h_amax)) : *a.a_scale;
    const float deq = sh * (*a.w_scale);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = brow0 + 32 * j + col;
      if (t < ntok) {
        const int f = a.seg.sorted_ids[tok0 + t];
        const float w = a.topk_w[f] * deq;
        uint16_t* dst = (uint16_t*)a.out + (int64_t)f * a.H + (int64_t)tile * kPfRows + 64 * wr;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& c = acc[i][j];
            u32x2 o = {pack_bf16x2(c[4 * g] * w, c[4 * g + 1] * w), pack_bf16x2(c[4 * g + 2] * w, c[4 * g + 3] * w)};
            *(u32x2*)(dst + 32 * i + 8 * g + rq) = o;
          }
      }
    }
  }
}

// h (bf16, [P][I]) -> e4m3 with the dynamic scale amax/448; 16 per thread.
__global__ __launch_bounds__(256) void prefill_quant_h_kernel(const uint16_t* __restrict__ h, int64_t n,
                                                              const unsigned* __restrict__ h_amax,
                                                              uint8_t* __restrict__ hq) {
  const float r = 1.0f / scale_from_amax(__uint_as_float(*h_amax));
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (i >= n) return;
  const u32x4 v0 = *(const u32x4*)(h + i), v1 = *(const u32x4*)(h + i + 8);
  u32x4 o = {pack_e4m3x4(bf16_lo(v0[0]) * r, bf16_hi(v0[0]) * r, bf16_lo(v0[1]) * r, bf16_hi(v0[1]) * r),
             pack_e4m3x4(bf16_lo(v0[2]) * r, bf16_hi(v0[2]) * r, bf16_lo(v0[3]) * r, bf16_hi(v0[3]) * r),
             pack_e4m3x4(bf16_lo(v1[0]) * r, bf16_hi(v1[0]) * r, bf16_lo(v1[1]) * r, bf16_hi(v1[1]) * r),
             pack_e4m3x4(bf16_lo(v1[2]) * r, bf16_hi(v1[2]) * r, bf16_lo(v1[3]) * r, bf16_hi(v1[3]) * r)};
  *(u32x4*)(hq + i) = o;
}

// y[m,n] = bf16( sum_j part[m*k+j][n] ), j ascending, fp32 sum; 8 outputs per
// thread.
__global__ __launch_bounds__(256) void prefill_finalize_kernel(const uint16_t* __restrict__ part,
                                                               uint16_t* __restrict__ y, int M, int H, int top_k,
                                                               const float* x_scale, const unsigned* h_amax,
                                                               const float* h_scale, float* scales_out) {
  if (scales_out && blockIdx.x == 0 && threadIdx.x == 0) {
    scales_out[0] = *x_scale;
    scales_out[1] = h_scale ? *h_scale : scale_from_amax(__uint_as_float(*h_amax));
  }
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= (int64_t)M * H) return;
  const int64_t m = i / H, n = i - m * H;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const u32x4 v = *(const u32x4*)(part + (m * top_k + j) * H + n);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_lo(v[q]);
      acc[2 * q + 1] += bf16_hi(v[q]);
    }
  }
  u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
             pack_bf16x2(acc[6], acc[7])};
  *(u32x4*)(y + i) = o;
}

}  // namespace moe
