// Grouped expert products for large token counts (prefill), gfx950 MFMA: fp8
// (32x32x64) and bf16 (32x32x16) layers.
//
// At prefill every active expert holds hundreds to thousands of tokens, so the
// products are compute-bound and both operands are reused: a work item is a
// 256 x 128 tile (256 weight rows x 128 tokens of one expert) whose operands
// are staged through LDS, K-step by K-step.  The token dimension is grouped by
// the align step with a block of 128: block b holds tokens of expert
// block_expert[b] only, padded with the sentinel, so an item's tokens share
// one expert.  Weight rows stay the MFMA's A operand and tokens the B operand,
// as in the decode kernels; the 32x32x64 fp8 MFMA is used, or for bf16
// layers four 32x32x16 bf16 MFMAs per 128-byte K-step (the tiles, the LDS
// ring and its byte layout are the same).
//
// Four waves, one per SIMD, each own 64 weight rows x all 128 tokens (2 x 4
// MFMA tiles, accumulators in AGPRs).  A K-step is 128 bytes (two MFMA
// k-steps), so every 1 KB direct-to-LDS load covers eight whole cache lines of
// eight rows: the texture units, not the LDS port or the matrix pipes, are the
// busiest part of the CU here, and a load of sixteen half lines costs them
// twice as much.  Per K-step a CU reads 96 KB of fragments and writes 48 KB of
// operands into LDS against 16 MFMAs per SIMD.  With one wave per SIMD there is
// no second wave to fill the matrix pipe, so every LDS read and DMA is
// interleaved between MFMAs (sched_group_barrier) instead of being issued as a
// block.
//
// Work items (weight tile, token block) are numbered so that each XCD works
// on its own range of token blocks, rasterised so that concurrent workgroups
// share operands in that XCD's L2 (pf_map); one persistent workgroup per CU
// walks them.
//
// Pipeline: both operand tiles of each K-step are loaded from global memory
// straight into a three-deep LDS ring (direct-to-LDS loads, no staging
// registers), two steps ahead of the MFMAs, with one barrier per step.
//
// Down-product epilogue: a wave's 64 bf16 partial sums for each of 32 tokens
// are 32 token rows of 128 bytes in the output.  In the MFMA result layout a
// lane holds 8 bytes of one token, so storing straight from it makes every
// store touch 32 cache lines; the tile is instead transposed through the
// wave's own 4 KB of LDS past the ring, and each store then writes 8 whole
// lines with half as many store instructions (the down product ran 5 %
// faster).  The gate/up epilogue stores 16 bytes per lane, two lanes filling
// 32 contiguous bytes of a token; the same transposition made that product
// 2 % slower, so it stores directly.
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

// 32x32x16 bf16 -> fp32.  A: lane l holds 8 bf16 (16 bytes) of row l%32 at
// k = 8*(l/32); B: the same k of column l%32.  C as for mfma32_fp8.
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
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
// wait for every vector-memory operation, draining the prefetch queue.)  The
// leading builtin repeats the LDS wait where the compiler's counter model
// sees it, so that it does not wait again for reads that already completed.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int kPfTok = 128;                      // tokens per work item (the align block)
constexpr int kPfRows = 256;                     // weight rows per work item
constexpr int kPfBK = 128;                       // K bytes per step: two MFMA k-steps, one cache line per row
constexpr int kPfStages = 3;                     // LDS ring depth: loads run two steps ahead
constexpr int kPfStageA = kPfRows * kPfBK;       // 32 KB
constexpr int kPfStageB = kPfTok * kPfBK;        // 16 KB
constexpr int kPfStage = kPfStageA + kPfStageB;  // 48 KB
constexpr int kPfRing = kPfStages * kPfStage;    // 144 KB
constexpr int kPfEpiWave = 32 * 128;             // a wave's epilogue tile: 32 token rows of 128 bytes
constexpr int kPfLds = kPfRing + 4 * kPfEpiWave;  // 160 KB, all of a CU's LDS: one workgroup per CU
constexpr int kPfThreads = 256;                  // four waves
static_assert(kPfLds <= 160 * 1024, "LDS of one gfx950 CU");
constexpr int kPfDma = 12;                       // DMA instructions per wave per step: 8 A + 4 B
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

// LDS layout of an operand tile in one stage: rows of 128 bytes (a whole
// cache line of the row per step, so a 1 KB load covers 8 lines rather than
// 16 half lines, which halves its texture-address work), the eight 16-byte
// chunks of row r stored at chunk position c ^ pf_mix(r).  A 16-byte LDS read
// is served 16 lanes at a time over 64 four-byte banks (256 bytes); a 128-byte
// row covers half of them, even rows one half and odd rows the other.  The
// MFMA fragment reads take one logical chunk of 16 consecutive rows, so the
// eight rows of each parity must land on eight different chunk positions:
// pf_mix(r) = (r & 7) ^ ((r >> 3) & 1) does that (r & 7 alone repeats every
// eight rows, a two-way conflict on every such read).  pf_mix depends on the
// row's low four bits only, so tiles 32 rows apart share one pattern.
__device__ __forceinline__ int pf_mix(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int pf_swz(int row, int chunk) { return row * kPfBK + ((chunk ^ pf_mix(row)) << 4); }

// Work item -> (weight tile, token block), XCD-aware.  Workgroups are handed
// to the eight XCDs round robin by linear id, and item L belongs to XCD L % 8.
// XCD c takes a contiguous eighth of the token blocks that hold tokens
// (blocks are ordered by expert, so an XCD's range covers a few experts; only
// experts cut by a range boundary have their weights read by two XCDs) and
// all weight tiles for them.  Inside an XCD the items are numbered densely
// (no holes, so the workgroups walking them round robin get equal shares):
// by groups of GB blocks, within a block group by groups of GT tiles, the
// last group of either kind possibly smaller.  A full group of GT x GB items
// is about one per CU of an XCD, so workgroups running together share weight
// tiles and token blocks in that XCD's L2.  Returns false past the XCD's last
// item (all later indices of that XCD are past it too).  Group shapes, from a
// sweep of (GT, GB) over {2,4,8} x {4,8,16} on the E=128 top-8 H=4096 I=1536
// M=4096 layer: 2 x 16 for the gate/up product (12 tiles of 128 features,
// 2 % faster than 4 x 8), 8 x 4 for the down product (16 tiles of 256 output
// rows, 3 % faster).
template <int MODE>
struct PfRaster {
  static constexpr int GT = MODE == 0 ? 2 : 8;   // weight tiles per raster group
  static constexpr int GB = MODE == 0 ? 16 : 4;  // token blocks per raster group
};

template <int MODE>
__device__ __forceinline__ bool pf_map(int L, int T, int nb, int* tile, int* blk) {
  constexpr int kPfGT = PfRaster<MODE>::GT, kPfGB = PfRaster<MODE>::GB;
  const int c = L & 7, j = L >> 3;
  const int nbx = (nb + 7) >> 3;                    // blocks per XCD
  const int nbc = max(0, min(nbx, nb - c * nbx));  // blocks of XCD c
  if (j >= T * nbc) return false;
  const int bg = j / (T * kPfGB), r = j - bg * (T * kPfGB);
  const int gb = min(kPfGB, nbc - bg * kPfGB);       // blocks in this block group
  const int tg = r / (kPfGT * gb), rr = r - tg * (kPfGT * gb);
  *tile = tg * kPfGT + rr / gb;
  *blk = c * nbx + bg * kPfGB + rr % gb;
  return true;
}

// ---------------------------------------------------------------- products
struct PrefillArgs {
  const uint8_t* w;        // W13 [E][2I][H] or W2 [E][H][I], e4m3
  const uint8_t* act;      // gate/up: xq [M][H]; down: hq [P][I], e4m3 (bf16 layers: x and h, bf16)
  PrefillSeg seg;
  int H, I, top_k, P;
  int tiles;               // weight tiles: I/128 (128 gate + 128 up rows each) or H/256
  int items;               // bound on the linear item index: 8 x tiles x blocks per XCD (largest case)
  const float* w_scale;    // s_w13 or s_w2: one per tensor, per expert ([E], w_es = 1) or per weight row
                           // ([E][2I] / [E][H], PC)
  const float* a_scale;    // gate/up: s_x in effect; down: static s_h (null = dynamic)
  const unsigned* h_amax;  // down with dynamic scale: max |h| (float bits)
  const float* h_scale;    // gate/up: static s_h (null = dynamic: h written as bf16)
  uint8_t* out;            // gate/up: h (fp32 or e4m3); down: part [P][H] bf16
  unsigned* h_amax_out;    // gate/up with dynamic scale
  int w_es = 0;            // without PC: 1 = one weight scale per expert (w_scale[e]), 0 = w_scale[0]
};

// DMA sources of one work item for one lane (see prefill_gemm_kernel).  At
// namespace scope: with the struct local to the kernel, the host compilation
// pass silently drops the kernel's launch stub.
struct PfSrc {
  const uint8_t* wa;  // the expert's weight matrix (a buffer resource is made from it at issue)
  int offA;     // byte offset of this lane's first A row (load q adds 8*q rows)
  int offB[4];  // byte offsets of this lane's four B rows
  int fb[4];    // pair ids of this lane's B rows, until finish_src turns them into offB
  int f[4];     // pair ids of this lane's epilogue tokens 32*j + lane%32 (clamped)
};

// One work item: weight tile x token block of one expert.
struct PfItem {
  int tile, blk, e;
  int ntok;  // tokens of the block that belong to the expert (1..128)
};

// The work item at linear index L, or false when the workgroup has none left
// (stride, a multiple of 8, keeps L on one XCD).  Uniform across the
// workgroup; the loads are waited for where their values are first used.
template <int MODE>
__device__ __forceinline__ bool pf_next(const PrefillArgs& a, int nb, int& L, int stride, PfItem& it) {
  int tile = 0, blk = 0;
  if (L >= a.items || !pf_map<MODE>(L, a.tiles, nb, &tile, &blk)) return false;  // later indices of this XCD are past its items too
  const int e = a.seg.block_expert[blk];  // every block below num_padded belongs to an expert
  it.tile = tile;
  it.blk = blk;
  it.e = e;
  it.ntok = min(kPfTok, a.seg.offsets[e] + a.seg.counts[e] - blk * kPfTok);
  return true;
}

// The same lookup in three phases for use inside the K-loop, each phase's
// loads issued before a K-step's loads and consumed after the next K-step's
// wait (which covers them), so that no wait of its own drains the ring.
// Loads are unconditional, at index 0 when there is no item.
struct PfFetch {
  bool ok;
  int tile, blk, e, off, cnt;
};
template <int MODE>
__device__ __forceinline__ void pf_fetch_a(const PrefillArgs& a, int nb, int L, bool want, PfFetch& f) {
  f.tile = 0;
  f.blk = 0;
  f.ok = want && L < a.items && pf_map<MODE>(L, a.tiles, nb, &f.tile, &f.blk);
  f.e = a.seg.block_expert[f.ok ? f.blk : 0];
}
__device__ __forceinline__ void pf_fetch_b(const PrefillArgs& a, PfFetch& f) {
  const int e = f.ok ? __builtin_amdgcn_readfirstlane(f.e) : 0;
  f.e = e;
  f.off = a.seg.offsets[e];
  f.cnt = a.seg.counts[e];
}
__device__ __forceinline__ bool pf_fetch_c(const PfFetch& f, PfItem& it) {
  if (!f.ok) return false;
  it.tile = f.tile;
  it.blk = f.blk;
  it.e = f.e;
  it.ntok = min(kPfTok, __builtin_amdgcn_readfirstlane(f.off + f.cnt) - f.blk * kPfTok);
  return true;
}

// SiLU(x) = x / (1 + e^-x) with the hardware exp2 and reciprocal (about one
// ulp each in fp32, far below the e4m3 / bf16 rounding that follows): the
// libm exp and the IEEE division cost several times more, and with one wave
// per SIMD nothing hides the epilogue.  Large |x| behave: e^-x overflows to
// inf for x << 0 (result -0), and underflows to 0 for x >> 0 (result x).
__device__ __forceinline__ float silu_fast(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Scheduling pattern of one K-step with NMF MFMAs: the step's NDS LDS
// fragment reads follow the MFMAs of the first half, its NVM DMA loads those
// of the second half, spread as evenly as the counts allow.
template <int K, int NMF, int NDS, int NVM, int ID>
__device__ __forceinline__ void pf_interleave() {
  if constexpr (K < NMF) {
    constexpr int H = NMF / 2;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);  // one MFMA
    if constexpr (K < H) {
      constexpr int n = NDS * (K + 1) / H - NDS * K / H;
      if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, ID);  // LDS reads
    } else {
      constexpr int n = NVM * (K - H + 1) / (NMF - H) - NVM * (K - H) / (NMF - H);
      if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x020, n, ID);  // vector-memory loads
    }
    pf_interleave<K + 1, NMF, NDS, NVM, ID>();
  }
}

// MODE 0: gate/up product, tile rows = 128 gate + 128 up rows of the same 128
//   features, epilogue SiLU(g)*u -> h.  HDYN: h stored as fp32 with a running
//   amax (quantised by prefill_quant_h_kernel), else as e4m3 with the static
//   scale.
// PC: the weight scale is one fp32 per weight row (output channel) instead of
//   one per tensor; the epilogue reads the lane's 16 (MODE 0: 16 gate + 16 up)
//   row scales once per item.
// MODE 1: down product, tile rows = 256 output features, epilogue
//   s_h * s_w2 * acc -> bf16 part[pair][feature] (the routing weight is
//   applied when the pairs of a token are summed).
//
// Persistent: one workgroup per CU walks the work items L = blockIdx.x,
// blockIdx.x + gridDim.x, ... (gridDim.x a multiple of 8 keeps every
// workgroup on the XCD that pf_map assigns its items to).  The LDS ring runs
// on across items: the last two K-steps of an item that load anything load
// the first two of the next, whose metadata was fetched one item earlier, so
// an item's epilogue overlaps the next item's first loads and no workgroup
// start or metadata latency sits between items.
//
// Wave w multiplies 64 weight rows of the tile (MODE 0: gate rows 32w.. and
// the up rows of the same 32 features; MODE 1: rows 64w..64w+63) by all 128
// tokens.  Each 128-byte K-step (two MFMA k-steps) every wave DMA-loads rows
// 64w..64w+63 of the A tile and 32w..32w+31 of the B tile (twelve 1 KB load
// instructions, lane i filling bytes 16i..16i+15 of an 8-row block).
//
// Wait accounting: the waits count vector-memory operations, which complete
// in issue order.  Before the barrier that precedes the reads of step s+1 a
// wave waits until at most twelve are outstanding: the loads of step s+2,
// issued after those of step s+1.  Any other vector-memory operation (token
// ids, epilogue stores) only makes that wait stricter.
// BF: bf16 layers (weights, x and h bf16, no scales; HDYN and PC false):
//   a 128-byte K-step holds 64 elements, four 32x32x16 bf16 MFMA k-steps, and
//   the gate/up epilogue stores h as bf16 for the down product.
template <int MODE, bool HDYN, bool PC, bool BF = false>
static __global__ __launch_bounds__(kPfThreads) void prefill_gemm_kernel(PrefillArgs a) {
  static_assert(!BF || (!HDYN && !PC), "bf16 layers have no scales");
  extern __shared__ __align__(16) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int nb = *a.seg.num_padded / kPfTok;
  const int stride = gridDim.x;
  int L = blockIdx.x;
  PfItem cur;
  if (!pf_next<MODE>(a, nb, L, stride, cur)) return;
  PfItem nxt = cur;  // stays a valid item when there is no next one (its loads are then unused)
  L += stride;
  bool has_next = pf_next<MODE>(a, nb, L, stride, nxt);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the wave's branches scalar
  const int K = (MODE == 0 ? a.H : a.I) * (BF ? 2 : 1);       // contraction length (bytes)
  const int nk = K / kPfBK;                                   // even, >= 4 (host)
  const int wrows = MODE == 0 ? 2 * a.I : a.H;                // rows of one expert's weight
  const int drow = lane >> 3, dchunk = lane & 7;              // DMA: row in an 8-row block, chunk position
  const int col = lane & 31, rq = (lane >> 5) * 4;

  // DMA sources of an item for this lane: A rows 64*wave + 8*q + lane/8
  // (q < 8), B rows 32*wave + 8*q + lane/8 (q < 4), logical chunk
  // (lane%8) ^ pf_mix(row) = (lane%8) ^ (lane/8) ^ (q & 1): offA holds the
  // chunk for even q, odd q flip its lowest bit (byte offset bit 4).  The loads go through buffer resources (the
  // expert's weight matrix and the activation matrix, byte offsets below
  // 2^31, checked by the host) rather than flat-global addresses: the
  // compiler's wait-count model treats a flat-global load into LDS as a
  // possible LDS access for as long as it is in flight, which would turn
  // every wait for LDS reads into a full drain.
  auto make_src = [&](const PfItem& it, PfSrc& sr) {
    sr.wa = a.w + (int64_t)it.e * wrows * K;
    {
      // rows 64*wave + 8*q + lane/8: in MODE 0 waves 0, 1 load gate rows and
      // waves 2, 3 the up rows of the same features
      const int row = 64 * wave + drow;
      int wrow;
      if (MODE == 0) {
        const int f0 = it.tile * (kPfRows / 2);
        wrow = row < kPfRows / 2 ? f0 + row : a.I + f0 + (row - kPfRows / 2);
      } else {
        wrow = it.tile * kPfRows + row;
      }
      sr.offA = wrow * K + ((dchunk ^ drow) << 4);
    }
    // token ids: padding slots read the block's last token (their results are dropped)
    const int32_t* ids = a.seg.sorted_ids + it.blk * kPfTok;
#pragma unroll
    for (int q = 0; q < 4; ++q) sr.fb[q] = ids[min(32 * wave + 8 * q + drow, it.ntok - 1)];
#pragma unroll
    for (int j = 0; j < 4; ++j) sr.f[j] = ids[min(32 * j + col, it.ntok - 1)];
  };
  // B-row offsets from the token ids: kept apart from make_src so that the
  // wait for the ids falls where the offsets are first needed (the empty asm
  // pins the conversion here; otherwise the compiler hoists it next to the
  // loads, waiting for them there)
  auto finish_src = [&](PfSrc& sr) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int f = sr.fb[q];
      asm volatile("" : "+v"(f));
      const int brow = MODE == 0 ? f / a.top_k : f;
      sr.offB[q] = brow * K + ((dchunk ^ drow ^ (q & 1)) << 4);  // row 32*wave + 8*q + drow
    }
  };
  const __amdgpu_buffer_rsrc_t rsrcB =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.act, (short)0, 0x7fffffff, kBufferWord3);
  auto issue = [&](const PfSrc& sr, int kstep, int slot) {  // DMA of one K-step into ring slot `slot`
    lds_u8* base = smem + slot * kPfStage;
    const int kb = kstep * kPfBK;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)sr.wa, (short)0, wrows * K, kBufferWord3);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (void __attribute__((address_space(3)))*)(base + (64 * wave + 8 * q) * kPfBK), 16,
          (q & 1) ? (sr.offA ^ 16) : sr.offA,
          kb + 8 * q * K, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrcB, (void __attribute__((address_space(3)))*)(base + kPfStageA + (32 * wave + 8 * q) * kPfBK), 16,
          sr.offB[q], kb, 0, 0);
  };

  // fragment addresses within a stage: A tile i rows arow0 + arow_off(i) +
  // lane%32, B tile j rows 32*j + lane%32.  fp8: MFMA k-step ks (64 bytes)
  // of the step uses chunks 4*ks + 2*(lane/32) + c, c = 0, 1 (32 bytes per
  // lane); bf16: MFMA k-step 2*ks + c (32 bytes) uses chunk 4*ks + 2*c +
  // lane/32 (16 bytes per lane).  Tiles differ by whole 32-row multiples,
  // which leave pf_mix unchanged, so a tile is a constant byte
  // offset from the (ks, c) base.
  const int fr = lane & 31, hl = lane >> 5;
  const int arow0 = MODE == 0 ? 32 * wave : 64 * wave;
  int baseA[2][2], baseB[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = BF ? 4 * ks + 2 * c + hl : 4 * ks + 2 * hl + c;
      baseA[ks][c] = pf_swz(arow0 + fr, chunk);
      baseB[ks][c] = kPfStageA + pf_swz(fr, chunk);
    }
  // row offset of A tile i from arow0 (MODE 0: tile 0 gate, tile 1 the up
  // rows of the same features)
  auto arow_off = [](int i) { return MODE == 0 ? i * (kPfRows / 2) : 32 * i; };

  // epilogue constants
  const float sa = BF ? 1.0f
                      : (MODE == 0 ? *a.a_scale : (HDYN ? scale_from_amax(__uint_as_float(*a.h_amax)) : *a.a_scale));
  const float rhs = (MODE == 0 && !HDYN && !BF) ? 1.0f / *a.h_scale : 1.0f;
  float hmax = 0.0f;

  PfSrc cs, ns;
  make_src(cur, cs);
  finish_src(cs);
  int slot0 = 0;  // ring slot of the current item's first K-step
  issue(cs, 0, 0);  // steps 0, 1 (each item's start issues its step 2)
  issue(cs, 1, 1);

  // Fragments of one K-step (two MFMA k-steps): the wave's two A tiles and up
  // to four B tiles.
  struct Frags {
    u32x4 a[2][2][2], b[2][4][2];  // [k-step][tile][chunk]
  };
  PfItem nn = nxt;  // the item after the next (fetched during each item)
  bool has_nn = false;
  // One item with its NJ (1..4) 32-token tiles multiplied; one version per NJ
  // so that the K-step body has no branches, each with its own accumulators
  // and epilogue (a join of the versions' accumulators would be copied out of
  // AGPRs).  Fragments are double-buffered: the reads of step k+1 run while
  // the MFMAs of step k do.  Each step's barrier follows this wave's wait for
  // its loads of step k+1 (those of k+2 may still be in flight); then step
  // k+3 is loaded into the slot of step k, whose reads the barrier has just
  // drained.
  auto item = [&](auto nj_tag) {
    constexpr int NJ = decltype(nj_tag)::value;
    constexpr int NMF = (BF ? 8 : 4) * NJ, NDS = 8 + 4 * NJ;
    f32x16 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    auto slot = [&](int k) { return (slot0 + k) % kPfStages; };
    auto read = [&](Frags& F, int k) {
      const lds_u8* st = smem + slot(k) * kPfStage;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
            F.a[ks][i][c] =
                *(const __attribute__((address_space(3))) u32x4*)(st + baseA[ks][c] + arow_off(i) * kPfBK);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            F.b[ks][j][c] = *(const __attribute__((address_space(3))) u32x4*)(st + baseB[ks][c] + 32 * j * kPfBK);
        }
    };
    auto mma = [&](const Frags& F) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            if constexpr (BF) {
              acc[i][j] = mfma32_bf16(F.a[ks][i][0], F.b[ks][j][0], acc[i][j]);
              acc[i][j] = mfma32_bf16(F.a[ks][i][1], F.b[ks][j][1], acc[i][j]);
            } else {
              acc[i][j] = mfma32_fp8(F.a[ks][i][0], F.a[ks][i][1], F.b[ks][j][0], F.b[ks][j][1], acc[i][j]);
            }
          }
    };
    // Every K-step but the last loads step k+3 of the ring: this item's, the
    // next item's or, after the last item, a dummy copy of this item's first
    // steps into a slot nothing reads again; so every wait is the same (the
    // loads of the following step may be in flight) and every step has the
    // same interleaved body.  The kernel drains these loads before it ends.
    Frags F0, F1;
    // item start: step 0 landed, load step 2 (of this item: nk >= 4)
    wait_vm<kPfDma>();
    ring_barrier();
    issue(cs, 2, slot(2));
    make_src(nxt, ns);  // next item's token ids (unconditional: a conditional load would be copied at the join, waiting for it)
    read(F0, 0);
    // one K-step: multiply step k, read step k+1, load K-step `kstep` of src
    // into the slot of step k (step k+3 of the ring); `pre` runs first (its
    // loads precede the step's)
    auto body = [&](Frags& Fc, Frags& Fn, int k, const PfSrc& src, int kstep, auto id_tag, auto&& pre) {
      constexpr int ID = decltype(id_tag)::value;
      wait_vm<kPfDma>();  // step k+1 landed; k+2 may be in flight
      ring_barrier();
      pre();
      __builtin_amdgcn_sched_barrier(0);
      read(Fn, k + 1);
      issue(src, kstep, slot(k + 3));
      mma(Fc);
      pf_interleave<0, NMF, NDS, kPfDma, ID>();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto none = [] {};
    int s = 0;
    for (; s + 4 < nk; s += 2) {  // steps loading this item's steps (nk is even)
      body(F0, F1, s, cs, s + 3, std::integral_constant<int, 0>{}, none);
      body(F1, F0, s + 1, cs, s + 4, std::integral_constant<int, 1>{}, none);
    }
    // s = nk - 4: its step loads this item's last step; the metadata of the
    // item after the next is fetched across the last three steps
    PfFetch fnn;
    body(F0, F1, nk - 4, cs, nk - 1, std::integral_constant<int, 2>{},
         [&] { pf_fetch_a<MODE>(a, nb, L + stride, has_next, fnn); });
    if (!has_next) ns = cs;  // dummy source after the last item (valid addresses, never read)
    finish_src(ns);          // the next item's token ids are needed from here on
    // steps nk-3 and nk-2 load the next item's steps 0 and 1; step nk-1 only
    // multiplies
    body(F1, F0, nk - 3, ns, 0, std::integral_constant<int, 3>{}, [&] { pf_fetch_b(a, fnn); });
    body(F0, F1, nk - 2, ns, 1, std::integral_constant<int, 4>{}, none);
    mma(F1);

    // The accumulators stay in AGPRs until the epilogue reads them tile by
    // tile (otherwise the last MFMAs write all of them to VGPRs at once).
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) asm volatile("" : "+a"(acc[i][j]));

    // metadata of the item after the next (its loads completed under the
    // waits of the last steps)
    if (has_next) {
      L += stride;
      has_nn = pf_fetch_c(fnn, nn);
    }

    // epilogue (the next item's first loads are landing in the ring, so only
    // the wave's own area past the ring is used); one 32-token tile at a time,
    // so that few accumulators are out of AGPRs at once.  Transposed tiles
    // (down product): token row t holds 16-byte chunk c at chunk position
    // c ^ pf_mix(t), so that the writes (32 tokens, same chunk) and the reads
    // (8 tokens x 8 chunks) spread evenly over the LDS banks.
    lds_u8* ep = smem + kPfRing + wave * kPfEpiWave;
    auto ep_at = [&](int t, int c) { return ep + t * 128 + ((c ^ pf_mix(t)) << 4); };
    const int rt = lane >> 3, rc = lane & 7;  // read-back: token rt + 8*rr, chunk rc
    const float deq = (PC || BF) ? (BF ? 1.0f : 0.0f) : sa * a.w_scale[(int64_t)cur.e * a.w_es];  // the expert's or tensor's scale
    if (MODE == 0) {
      const int fbase = cur.tile * (kPfRows / 2) + 32 * wave;
      // per-row dequantisation of features fbase+8g+rq.. (gate) and I+.. (up)
      f32x4 dg4[4], du4[4];
      if constexpr (PC) {
        const float* ws = a.w_scale + (int64_t)cur.e * 2 * a.I;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          dg4[g] = sa * *(const f32x4*)(ws + fbase + 8 * g + rq);
          du4[g] = sa * *(const f32x4*)(ws + a.I + fbase + 8 * g + rq);
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = 32 * j + col;
        if (t < cur.ntok) {
          const int f = cs.f[j];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float gt = acc[0][j][4 * g + q] * (PC ? dg4[g][q] : deq);
              const float up = acc[1][j][4 * g + q] * (PC ? du4[g][q] : deq);
              hv[q] = silu_fast(gt) * up;
              hmax = fmaxf(hmax, fabsf(hv[q]));
            }
            const int64_t idx = (int64_t)f * a.I + fbase + 8 * g + rq;
            if (BF) {  // bf16 h, as the decode path's bf16 layers keep it
              *(u32x2*)(a.out + idx * 2) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            } else if (HDYN) {  // fp32, so that h is rounded once, to e4m3, after the amax is known
              *(f32x4*)(a.out + idx * 4) = f32x4{hv[0], hv[1], hv[2], hv[3]};
            } else {
              *(unsigned*)(a.out + idx) = pack_e4m3x4(hv[0] * rhs, hv[1] * rhs, hv[2] * rhs, hv[3] * rhs);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // bf16 partial sums: rows 64*wave.. of token t are its 128-byte row;
      // rows 32i+8g+rq.. are bytes 16*(4i+g) + 2*rq of it
      const int64_t obase = (int64_t)cur.tile * kPfRows + 64 * wave;
      // per-row dequantisation of rows obase+32i+8g+rq..
      f32x4 dd[2][4];
      if constexpr (PC) {
        const float* ws = a.w_scale + (int64_t)cur.e * a.H + obase;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) dd[i][g] = sa * *(const f32x4*)(ws + 32 * i + 8 * g + rq);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& c = acc[i][j];
            const f32x4 d = PC ? dd[i][g] : f32x4{deq, deq, deq, deq};
            u32x2 o = {pack_bf16x2(c[4 * g] * d[0], c[4 * g + 1] * d[1]),
                       pack_bf16x2(c[4 * g + 2] * d[2], c[4 * g + 3] * d[3])};
            *(__attribute__((address_space(3))) u32x2*)(ep_at(col, 4 * i + g) + 2 * rq) = o;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int t = 8 * rr + rt;
          const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)ep_at(t, rc);
          const int f = __shfl(cs.f[j], t);
          // non-temporal: the partial sums are read once, by the finalize, and
          // would otherwise take L2 lines from the W2 tiles still in use
          // (the down product 2-5 % faster; the same on the fp32 h of the
          // gate/up product made it 16-20 % slower)
          if (32 * j + t < cur.ntok)
            __builtin_nontemporal_store(v, (u32x4*)((uint16_t*)a.out + (int64_t)f * a.H + obase + 8 * rc));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  while (true) {
    const int nj = (cur.ntok + 31) >> 5;  // 32-token tiles holding tokens (1..4)
    if (nj == 4)
      item(std::integral_constant<int, 4>{});
    else if (nj == 3)
      item(std::integral_constant<int, 3>{});
    else if (nj == 2)
      item(std::integral_constant<int, 2>{});
    else
      item(std::integral_constant<int, 1>{});
    if (!has_next) break;
    cur = nxt;
    cs = ns;
    nxt = nn;
    has_next = has_nn;
    has_nn = false;
    slot0 = (slot0 + nk) % kPfStages;
  }
  wait_vm<0>();  // the dummy loads after the last item
  if (MODE == 0 && HDYN) {
    // one device-scope atomic per workgroup: same-address atomics serialise,
    // and every workgroup finishes at about the same time
    hmax = wave_max(hmax);
    __syncthreads();  // the epilogue areas are no longer read
    float* red = (float*)(smem_raw + kPfRing);
    if (lane == 0) red[wave] = hmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      if (m > 0.0f) atomicMax(a.h_amax_out, __float_as_uint(m));
    }
  }
}

// h (fp32, [P][I]) -> e4m3 with the dynamic scale amax/448; 16 per thread.
static __global__ __launch_bounds__(256) void prefill_quant_h_kernel(const float* __restrict__ h, int64_t n,
                                                              const unsigned* __restrict__ h_amax,
                                                              uint8_t* __restrict__ hq) {
  const float r = 1.0f / scale_from_amax(__uint_as_float(*h_amax));
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (i >= n) return;
  const f32x4* src = (const f32x4*)(h + i);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = src[q];
    o[q] = pack_e4m3x4(v[0] * r, v[1] * r, v[2] * r, v[3] * r);
  }
  *(u32x4*)(hq + i) = o;
}

// y[m,n] = bf16( sum_j w[m*k+j] * part[m*k+j][n] ), j ascending, fp32 sum;
// 8 outputs per thread.
static __global__ __launch_bounds__(256) void prefill_finalize_kernel(const uint16_t* __restrict__ part,
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
  // all k partial rows are loaded before the sum (k loads in flight per
  // thread), then summed with j ascending
  u32x4 v[kMaxTopK];
  float w[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < top_k) {
      v[j] = *(const u32x4*)(part + (m * top_k + j) * H + n);
      w[j] = topk_w[m * top_k + j];
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < top_k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w[j] * bf16_lo(v[j][q]);
        acc[2 * q + 1] += w[j] * bf16_hi(v[j][q]);
      }
    }
  }
  u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
             pack_bf16x2(acc[6], acc[7])};
  *(u32x4*)(y + i) = o;
}

}  // namespace moe
