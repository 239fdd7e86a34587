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
// Work items (weight tile, token block) are numbered so that each XCD works
// on its own range of token blocks, rasterised so that concurrent workgroups
// share operands in that XCD's L2 (pf_map); one persistent workgroup per CU
// walks them.
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
// third descriptor word of a raw byte buffer resource on CDNA (32-bit data
// format, no swizzle, no index stride)
constexpr int kBufferWord3 = 0x00020000;

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
// to the eight XCDs round robin by linear id.  XCD c takes a contiguous eighth
// of the token blocks that hold tokens (blocks are ordered by expert, so an
// XCD's range covers a few experts; only experts cut by a range boundary have
// their weights read by two XCDs) and all weight tiles for them.  Inside an
// XCD the work is rasterised in groups of kPfGT tiles x kPfGB blocks, about
// one workgroup per CU, so the workgroups running together share weight
// tiles and token blocks in that XCD's L2.  Returns false for surplus
// workgroups (the grid is sized for the largest possible block count).
constexpr int kPfGT = 4;  // weight tiles per raster group
constexpr int kPfGB = 8;  // token blocks per raster group

__device__ __forceinline__ bool pf_map(int L, int T, int nb, int* tile, int* blk) {
  const int c = L & 7, j = L >> 3;
  const int nbx = (nb + 7) >> 3;                     // blocks per XCD
  const int ntg = (T + kPfGT - 1) / kPfGT;           // tile groups
  const int g = j / (kPfGT * kPfGB), r = j - g * (kPfGT * kPfGB);
  const int bg = g / ntg, tg = g - bg * ntg;
  const int t = tg * kPfGT + r / kPfGB, b = bg * kPfGB + (r % kPfGB);
  if (t >= T || b >= nbx) return false;
  *tile = t;
  *blk = c * nbx + b;
  return *blk < nb;
}

// ---------------------------------------------------------------- products
struct PrefillArgs {
  const uint8_t* w;        // W13 [E][2I][H] or W2 [E][H][I], e4m3
  const uint8_t* act;      // gate/up: xq [M][H]; down: hq [P][I], e4m3
  PrefillSeg seg;
  int H, I, top_k, P;
  int tiles;               // weight tiles: 2I/256 or H/256
  int items;               // linear work items covered by pf_map (>= tiles x blocks)
  const float* w_scale;    // s_w13 or s_w2
  const float* a_scale;    // gate/up: s_x in effect; down: static s_h (null = dynamic)
  const unsigned* h_amax;  // down with dynamic scale: max |h| (float bits)
  const float* h_scale;    // gate/up: static s_h (null = dynamic: h written as bf16)
  uint8_t* out;            // gate/up: h; down: part [P][H] bf16
  unsigned* h_amax_out;    // gate/up with dynamic scale
};

// DMA sources of one work item for one lane (see prefill_gemm_kernel).  At
// namespace scope: with the struct local to the kernel, the host compilation
// pass silently drops the kernel's launch stub.
struct PfSrc {
  const uint8_t* wa;  // the expert's weight matrix (a buffer resource is made from it at issue)
  int offA[4], offB[2];
  int fb[2];  // pair ids of this lane's B rows, until finish_src turns them into offB
  int f[2];   // pair ids of this lane's epilogue tokens brow0 + 32*j + lane%32 (clamped)
};

// One work item: weight tile x token block of one expert.
struct PfItem {
  int tile, blk, e;
  int ntok;  // tokens of the block that belong to the expert (1..128)
};

// The next work item at or after linear index L (stepping by `stride`), or
// false when none is left.  Uniform across the workgroup; the skip over
// surplus indices is arithmetic only, so the loads are issued once and
// waited for where their values are first used.
__device__ __forceinline__ bool pf_next(const PrefillArgs& a, int nb, int& L, int stride, PfItem& it) {
  int tile = 0, blk = 0;
  for (; L < a.items; L += stride)
    if (pf_map(L, a.tiles, nb, &tile, &blk)) break;
  if (L >= a.items) return false;
  const int e = a.seg.block_expert[blk];  // every block below num_padded belongs to an expert
  it.tile = tile;
  it.blk = blk;
  it.e = e;
  it.ntok = min(kPfTok, a.seg.offsets[e] + a.seg.counts[e] - blk * kPfTok);
  return true;
}

// MODE 0: gate/up product, tile rows = 128 gate + 128 up rows of the same 128
//   features, epilogue SiLU(g)*u -> h.  HDYN: h stored as bf16 with a running
//   amax (quantised by prefill_quant_h_kernel), else as e4m3 with the static
//   scale.
// MODE 1: down product, tile rows = 256 output features, epilogue
//   s_h * s_w2 * acc -> bf16 part[pair][feature] (the routing weight is
//   applied when the pairs of a token are summed).
//
// Persistent: one workgroup per CU walks the work items L = blockIdx.x,
// blockIdx.x + gridDim.x, ... (gridDim.x a multiple of 8 keeps every
// workgroup on the XCD that pf_map assigns its items to).  The LDS ring runs
// on across items: the last two K-steps of an item load the first two of the
// next, whose metadata was fetched one item earlier, so an item's epilogue
// overlaps the next item's first loads and no workgroup start or metadata
// latency sits between items.
//
// Eight waves: wave (wr = 0..3, wc = 0..1) owns 64 weight rows x 64 tokens
// (2 x 2 MFMA tiles; in MODE 0 the 32 gate and the 32 up rows of the same 32
// features).  Each 128-byte K-step: every wave DMA-loads 32 rows of the A
// tile and 16 rows of the B tile (six 1 KB load instructions, lane i filling
// bytes 16i..16i+15 of an 8-row block) into a three-deep LDS ring two steps
// ahead; one barrier per step; 8 MFMAs per wave per step, issued in the same
// window as the LDS reads of the next step.
//
// Wait accounting: the waits count vector-memory operations, which complete
// in issue order.  Before the barrier of step s a wave waits until at most
// six are outstanding, the six loads of step s+1 issued after step s's: any
// other vector-memory operation (token ids, epilogue stores) only makes that
// wait stricter.  When no load follows step s (the last step of the last
// item) the wait is for zero.
template <int MODE, bool HDYN>
__global__ __launch_bounds__(kPfThreads) void prefill_gemm_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int nb = *a.seg.num_padded / kPfTok;
  const int stride = gridDim.x;
  int L = blockIdx.x;
  PfItem cur;
  if (!pf_next(a, nb, L, stride, cur)) return;
  PfItem nxt = cur;  // stays a valid item when there is no next one (its loads are then unused)
  L += stride;
  bool has_next = pf_next(a, nb, L, stride, nxt);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the wave's branches scalar
  const int K = MODE == 0 ? a.H : a.I;                        // contraction length (bytes)
  const int nk = K / kPfBK;                                   // >= 2 (host)
  const int wrows = MODE == 0 ? 2 * a.I : a.H;                // rows of one expert's weight
  const int lrow = lane >> 3, lchunk = lane & 7;
  // wave sub-tile: two 32-row A tiles and 64 tokens
  const int wr = wave & 3, wc = wave >> 2;
  const int arow0 = MODE == 0 ? 32 * wr : 64 * wr;             // gate rows (MODE 0)
  const int arow1 = MODE == 0 ? 128 + 32 * wr : 64 * wr + 32;  // up rows of the same features (MODE 0)
  const int brow0 = 64 * wc;
  const int col = lane & 31, rq = (lane >> 5) * 4;

  // DMA sources of an item for this lane: A rows 32*wave + 8*q + lane/8
  // (q < 4), B rows 16*wave + 8*q + lane/8 (q < 2), logical chunk
  // (lane%8) ^ (row & 7).  The loads go through buffer resources (the
  // expert's weight matrix and the activation matrix, byte offsets below
  // 2^31, checked by the host) rather than flat-global addresses: the
  // compiler's wait-count model treats a flat-global load into LDS as a
  // possible LDS access for as long as it is in flight, which would turn
  // every wait for LDS reads into a full drain.

  const __amdgpu_buffer_rsrc_t rsrcB =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.act, (short)0, 0x7fffffff, kBufferWord3);
  auto make_src = [&](const PfItem& it, PfSrc& sr) {
    sr.wa = a.w + (int64_t)it.e * wrows * K;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 32 * wave + 8 * q + lrow;
      int wrow;
      if (MODE == 0) {
        const int f0 = it.tile * 128;
        wrow = row < 128 ? f0 + row : a.I + f0 + (row - 128);
      } else {
        wrow = it.tile * kPfRows + row;
      }
      sr.offA[q] = wrow * K + ((lchunk ^ (row & 7)) << 4);
    }
    // token ids: padding slots read the block's last token (their results are dropped)
    const int32_t* ids = a.seg.sorted_ids + it.blk * kPfTok;
#pragma unroll
    for (int q = 0; q < 2; ++q) sr.fb[q] = ids[min(16 * wave + 8 * q + lrow, it.ntok - 1)];
#pragma unroll
    for (int j = 0; j < 2; ++j) sr.f[j] = ids[min(brow0 + 32 * j + col, it.ntok - 1)];
  };
  // B-row offsets from the token ids: kept apart from make_src so that the
  // wait for the ids falls where the offsets are first needed (the empty asm
  // pins the conversion here; otherwise the compiler hoists it next to the
  // loads, waiting for them there)
  auto finish_src = [&](PfSrc& sr) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 16 * wave + 8 * q + lrow;
      int f = sr.fb[q];
      asm volatile("" : "+v"(f));
      const int brow = MODE == 0 ? f / a.top_k : f;
      sr.offB[q] = brow * K + ((lchunk ^ (row & 7)) << 4);
    }
  };
  // element-wise choice between two sources (a choice of struct address
  // would force both structs into scratch memory)
  auto pick = [](bool first, const PfSrc& x, const PfSrc& y) {
    PfSrc r;
    r.wa = first ? x.wa : y.wa;
#pragma unroll
    for (int q = 0; q < 4; ++q) r.offA[q] = first ? x.offA[q] : y.offA[q];
#pragma unroll
    for (int q = 0; q < 2; ++q) r.offB[q] = first ? x.offB[q] : y.offB[q];
#pragma unroll
    for (int j = 0; j < 2; ++j) r.f[j] = 0;
    return r;
  };
  auto issue = [&](const PfSrc& sr, int kstep, int slot) {  // DMA of one K-step into ring slot `slot`
    lds_u8* base = smem + slot * kPfStage;
    const int kb = kstep * kPfBK;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)sr.wa, (short)0, wrows * K, kBufferWord3);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (void __attribute__((address_space(3)))*)(base + (32 * wave + 8 * q) * kPfBK),
                                               16, sr.offA[q], kb, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrcB, (void __attribute__((address_space(3)))*)(base + kPfStageA + (16 * wave + 8 * q) * kPfBK), 16, sr.offB[q],
          kb, 0, 0);
  };

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

  // epilogue constants
  const float deq = MODE == 0 ? (*a.a_scale) * (*a.w_scale)
                              : (HDYN ? scale_from_amax(__uint_as_float(*a.h_amax)) : *a.a_scale) * (*a.w_scale);
  const float rhs = (MODE == 0 && !HDYN) ? 1.0f / *a.h_scale : 1.0f;
  float hmax = 0.0f;

  PfSrc cs, ns;
  make_src(cur, cs);
  finish_src(cs);
  int slot0 = 0;  // ring slot of the current item's first K-step
  issue(cs, 0, 0);
  issue(cs, 1, 1);

  // Fragments of one 64-byte MFMA k-step for up to two token sub-tiles.
  struct Frags {
    u32x4 a0[2], a1[2], b0[2], b1[2];
  };
  // K-loop of the current item with NJ (0, 1 or 2) of the wave's 32-token
  // sub-tiles multiplied; one version per NJ so that the loop body has no
  // branches.  Software pipelined by half K-steps over two register sets:
  // the LDS reads of one MFMA k-step are in flight while the MFMAs of the
  // previous one run, so the LDS and matrix pipes overlap.
  auto kloop = [&](auto nj_tag) {
    constexpr int NJ = decltype(nj_tag)::value;
    auto slot = [&](int s) { return (slot0 + s) % kPfStages; };
    auto read = [&](Frags& F, int s, int ks) {
      const lds_u8* st = smem + slot(s) * kPfStage;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        F.a0[c] = *(const __attribute__((address_space(3))) u32x4*)(st + offA0[ks][c]);
        F.a1[c] = *(const __attribute__((address_space(3))) u32x4*)(st + offA1[ks][c]);
        F.b0[c] = *(const __attribute__((address_space(3))) u32x4*)(st + offB0[ks][c]);
        if constexpr (NJ > 1) F.b1[c] = *(const __attribute__((address_space(3))) u32x4*)(st + offB1[ks][c]);
      }
    };
    auto mma = [&](const Frags& F) {
      acc[0][0] = mfma32_fp8(F.a0[0], F.a0[1], F.b0[0], F.b0[1], acc[0][0]);
      acc[1][0] = mfma32_fp8(F.a1[0], F.a1[1], F.b0[0], F.b0[1], acc[1][0]);
      if constexpr (NJ > 1) {
        acc[0][1] = mfma32_fp8(F.a0[0], F.a0[1], F.b1[0], F.b1[1], acc[0][1]);
        acc[1][1] = mfma32_fp8(F.a1[0], F.a1[1], F.b1[0], F.b1[1], acc[1][1]);
      }
    };
    // step s >= 1: wait for this wave's DMA of step s, barrier, DMA of step
    // s+2 (of this item, else of the next)
    auto sync = [&](int s) {
      if (s + 1 < nk || has_next)
        wait_vm<6>();
      else
        wait_vm<0>();
      ring_barrier();  // every wave's step-s data is in LDS; slot (s+2)%3 is no longer read
      const bool own = s + 2 < nk;
      if (own || has_next) issue(pick(own, cs, ns), own ? s + 2 : s + 2 - nk, slot(s + 2));
    };
    // step 0 also loads the next item's token ids, ahead of the step-2 DMA
    auto sync0 = [&]() {
      wait_vm<6>();  // nk >= 2: step 1's loads follow step 0's
      ring_barrier();
      make_src(nxt, ns);  // unconditional: a conditional load would be copied at the join, waiting for it
      if (2 < nk) {
        issue(cs, 2, slot(2));  // independent of the token ids just requested
      } else {
        finish_src(ns);
        if (has_next) issue(ns, 0, slot(2));
      }
    };
    if constexpr (NJ == 0) {
      sync0();
      int s = 1;
      for (; s + 2 < nk; ++s) {
        wait_vm<6>();
        ring_barrier();
        issue(cs, s + 2, slot(s + 2));
      }
      if (nk > 2) finish_src(ns);
      for (; s < nk; ++s) sync(s);
    } else {
      Frags F0, F1;
      sync0();
      read(F0, 0, 0);
      // The scheduling barriers keep each MFMA batch between the reads it is
      // meant to overlap; the steady-state body is branch-free so that the
      // compiler cannot sink the first batch into a join block.
      int s = 0;
      for (; s + 3 < nk; ++s) {
        read(F1, s, 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(F0);  // k-step 0 of step s
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<6>();    // this wave's DMA of step s+1 has landed
        ring_barrier();  // also waits for the reads into F1
        issue(cs, s + 3, slot(s + 3));
        read(F0, s + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        mma(F1);  // k-step 1 of step s
        __builtin_amdgcn_sched_barrier(0);
      }
      if (nk > 2) finish_src(ns);
      for (; s < nk; ++s) {  // the last (up to three) steps
        read(F1, s, 1);
        mma(F0);
        if (s + 1 < nk) {
          sync(s + 1);
          read(F0, s + 1, 0);
        }
        mma(F1);
      }
    }
  };

  while (true) {
    const bool live0 = brow0 < cur.ntok, live1 = brow0 + 32 < cur.ntok;  // 32-token sub-tiles that hold tokens
    if (live1)
      kloop(std::integral_constant<int, 2>{});
    else if (live0)
      kloop(std::integral_constant<int, 1>{});
    else
      kloop(std::integral_constant<int, 0>{});

    // metadata of the item after the next, waited for at its first use
    PfItem nn = nxt;
    bool has_nn = false;
    if (has_next) {
      L += stride;
      has_nn = pf_next(a, nb, L, stride, nn);
    }

    // epilogue (no LDS: the next item's first loads are landing in the ring)
    if (MODE == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = brow0 + 32 * j + col;
        if (t < cur.ntok) {
          const int f = cs.f[j];
          const int fbase = cur.tile * 128 + 32 * wr;
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
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = brow0 + 32 * j + col;
        if (t < cur.ntok) {
          uint16_t* dst = (uint16_t*)a.out + (int64_t)cs.f[j] * a.H + (int64_t)cur.tile * kPfRows + 64 * wr;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x16& c = acc[i][j];
              u32x2 o = {pack_bf16x2(c[4 * g] * deq, c[4 * g + 1] * deq), pack_bf16x2(c[4 * g + 2] * deq, c[4 * g + 3] * deq)};
              *(u32x2*)(dst + 32 * i + 8 * g + rq) = o;
            }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    if (!has_next) break;
    cur = nxt;
    cs = ns;
    nxt = nn;
    has_next = has_nn;
    slot0 = (slot0 + nk) % kPfStages;
  }
  if (MODE == 0 && HDYN) {
    hmax = wave_max(hmax);
    if (lane == 0) atomicMax(a.h_amax_out, __float_as_uint(hmax));
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

// y[m,n] = bf16( sum_j w[m*k+j] * part[m*k+j][n] ), j ascending, fp32 sum;
// 8 outputs per thread.
__global__ __launch_bounds__(256) void prefill_finalize_kernel(const uint16_t* __restrict__ part,
                                                               const float* __restrict__ topk_w,
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
    const float w = topk_w[m * top_k + j];
    const u32x4 v = *(const u32x4*)(part + (m * top_k + j) * H + n);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += w * bf16_lo(v[q]);
      acc[2 * q + 1] += w * bf16_hi(v[q]);
    }
  }
  u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
             pack_bf16x2(acc[6], acc[7])};
  *(u32x4*)(y + i) = o;
}

}  // namespace moe
