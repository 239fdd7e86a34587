// Grouped expert products for small token counts (decode), gfx950 MFMA.
//
// Orientation: the expert's weight rows are the MFMA's A operand (16 rows per
// tile, the wide side of the problem) and the expert's few tokens are the B
// operand (16 token columns per tile).  This is the operand order the pages
// call Swap-AB (B^T A^T instead of A B, "Fused MoE on Hopper, ...", TL;DR and
// flowchart; wagnersolution page, body), adopted here because at decode the
// weight rows are the only large dimension; CDNA4 MFMA tiles have no 64-row
// minimum, so the orientation is chosen for the memory stream, not for a
// fixed tile height.
//
// Memory stream: each lane loads 16 (bf16) or 32 (fp8) contiguous bytes of
// one weight row per MFMA step; the four lanes sharing a row cover 64 or 128
// contiguous bytes, and the U steps of a pipeline stage cover U times that.
// Weights go straight from HBM to VGPRs (every weight byte feeds exactly one
// lane once per token pass, so staging them through LDS would only add LDS
// traffic); the next stage's loads are issued before the current stage's
// MFMAs, two stages in flight per wave.
//
// Work: a workgroup serves one (expert with pairs, weight-row tile, token pass)
// triple.  The expert comes from the align step's list of experts that hold
// pairs, so no host readback is needed and surplus workgroups exit at once.
#pragma once

#include <type_traits>

#include "moe_device.h"

namespace moe {

enum HFormat { H_BF16 = 0, H_F32 = 1, H_E4M3 = 2 };

struct Segments {
  const int32_t* sorted_ids;
  const int32_t* offsets;
  const int32_t* counts;
  const int32_t* active;
  const int32_t* num_active;
  // 1: the products take their grid's y (active expert) and z (token pass)
  // indices in reverse, so that the workgroups of the last experts and of the
  // late token passes are dispatched first.  Set when a few experts hold many
  // more tokens than the rest (shared experts take every token): their long
  // workgroups then start first instead of running alone at the end.
  int rev;
};

__device__ __forceinline__ int grid_y(const Segments& g) { return g.rev ? gridDim.y - 1 - blockIdx.y : blockIdx.y; }
__device__ __forceinline__ int grid_z(const Segments& g) { return g.rev ? gridDim.z - 1 - blockIdx.z : blockIdx.z; }

// One MFMA step's operand fragment for one 16-row (or 16-token) tile.
template <bool FP8>
struct Frag {
  u32x4 v[FP8 ? 2 : 1];
};

template <bool FP8>
__device__ __forceinline__ void load_frag(Frag<FP8>& f, const uint8_t* p) {
  f.v[0] = *(const u32x4*)p;
  if constexpr (FP8) f.v[1] = *(const u32x4*)(p + 16);
}

template <bool FP8>
__device__ __forceinline__ f32x4 mma(const Frag<FP8>& a, const Frag<FP8>& b, f32x4 c) {
  if constexpr (FP8)
    return mfma_fp8(a.v[0], a.v[1], b.v[0], b.v[1], c);
  else
    return mfma_bf16(a.v[0], b.v[0], c);
}

// --------------------------------------------------------------------------
// K-loop shared by both products: NA weight tiles (A operands) times NB
// token tiles (B operands), U MFMA k-steps per pipeline stage, two stages in
// registers.  The steady state has no branches between a stage's loads and
// the MFMAs of the previous stage, so the compiler's wait before those MFMAs
// covers only the older stage and one full stage of loads stays in flight
// while the wave computes.  pa[i] / pb[t] point at the lane's first bytes;
// consecutive k-steps are SB bytes apart.
// --------------------------------------------------------------------------
// BS (block-scaled fp8): every k-step also carries the E8M0 block scales of
// its operands, one per A tile (qa[i][step], the same for every lane of the
// tile: a 16-row tile and a 128-element k-step lie in one 128 x 128 weight
// block) and one per token column (qb[t][step]: the token's 128-element
// group), loaded with the stage and fed to the scaled MFMA.
template <bool FP8, int NA, int NB, int U, bool BS = false>
struct StageRegs {
  Frag<FP8> a[U][NA];
  Frag<FP8> b[U][NB];
  int sa[BS ? U : 1][NA];
  int sb[BS ? U : 1][NB];
};

template <bool FP8, int NA, int NB, int U, int SB, bool BS = false>
__device__ __forceinline__ void stage_load(StageRegs<FP8, NA, NB, U, BS>& s, const uint8_t* const* pa,
                                           const uint8_t* const* pb, int64_t off, const uint8_t* const* qa = nullptr,
                                           const uint8_t* const* qb = nullptr, int step = 0) {
#pragma unroll
  for (int q = 0; q < U; ++q) {
#pragma unroll
    for (int i = 0; i < NA; ++i) load_frag<FP8>(s.a[q][i], pa[i] + off + q * SB);
#pragma unroll
    for (int t = 0; t < NB; ++t) load_frag<FP8>(s.b[q][t], pb[t] + off + q * SB);
    if constexpr (BS) {
#pragma unroll
      for (int i = 0; i < NA; ++i) s.sa[q][i] = qa[i][step + q];
#pragma unroll
      for (int t = 0; t < NB; ++t) s.sb[q][t] = qb[t][step + q];
    }
  }
}

template <bool FP8, int NA, int NB, int U, bool BS = false>
__device__ __forceinline__ void stage_mma(const StageRegs<FP8, NA, NB, U, BS>& s, f32x4 (&acc)[NA][NB]) {
#pragma unroll
  for (int q = 0; q < U; ++q)
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if constexpr (BS)
          acc[i][t] = mfma_fp8_scaled(s.a[q][i].v[0], s.a[q][i].v[1], s.b[q][t].v[0], s.b[q][t].v[1], acc[i][t],
                                      s.sa[q][i], s.sb[q][t]);
        else
          acc[i][t] = mma<FP8>(s.a[q][i], s.b[q][t], acc[i][t]);
      }
}

// acc += sum over nsteps k-steps of A_i . B_t (BS: with the k-steps' block
// scales from qa, qb)
template <bool FP8, int NA, int NB, int U, int SB, bool BS = false>
__device__ __forceinline__ void stream_k(const uint8_t* const* pa, const uint8_t* const* pb, int nsteps,
                                         f32x4 (&acc)[NA][NB], const uint8_t* const* qa = nullptr,
                                         const uint8_t* const* qb = nullptr) {
  constexpr int SS = U * SB;  // bytes per row per stage
  const int nfull = nsteps / U;
  if (nfull > 0) {
    StageRegs<FP8, NA, NB, U, BS> s0, s1;
    stage_load<FP8, NA, NB, U, SB, BS>(s0, pa, pb, 0, qa, qb, 0);
    int it = 0;
    for (; it + 2 < nfull; it += 2) {
      stage_load<FP8, NA, NB, U, SB, BS>(s1, pa, pb, (int64_t)(it + 1) * SS, qa, qb, (it + 1) * U);
      __builtin_amdgcn_sched_barrier(0);  // keep the whole stage's loads ahead of the MFMAs
      stage_mma<FP8, NA, NB, U, BS>(s0, acc);
      __builtin_amdgcn_sched_barrier(0);
      stage_load<FP8, NA, NB, U, SB, BS>(s0, pa, pb, (int64_t)(it + 2) * SS, qa, qb, (it + 2) * U);
      __builtin_amdgcn_sched_barrier(0);
      stage_mma<FP8, NA, NB, U, BS>(s1, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (it + 1 < nfull) {
      stage_load<FP8, NA, NB, U, SB, BS>(s1, pa, pb, (int64_t)(it + 1) * SS, qa, qb, (it + 1) * U);
      __builtin_amdgcn_sched_barrier(0);
      stage_mma<FP8, NA, NB, U, BS>(s0, acc);
      stage_mma<FP8, NA, NB, U, BS>(s1, acc);
    } else {
      stage_mma<FP8, NA, NB, U, BS>(s0, acc);
    }
  }
  for (int st = nfull * U; st < nsteps; ++st) {
    StageRegs<FP8, NA, NB, 1, BS> s;
    stage_load<FP8, NA, NB, 1, SB, BS>(s, pa, pb, (int64_t)st * SB, qa, qb, st);
    stage_mma<FP8, NA, NB, 1, BS>(s, acc);
  }
}

// --------------------------------------------------------------------------
// Gate/up product with the SiLU(gate)*up epilogue.
//
// Wave tile: FT groups of 16 output features i0+16f..i0+16f+15, i.e. gate
// rows i0+16f.. and up rows I+i0+16f.. of W13[e] (16-row MFMA tiles whose
// gate and up accumulators land in the same lanes, so the epilogue pairs
// gate and up without data exchange), times NT 16-token tiles.  KSPLIT waves
// of the workgroup split K = H and are summed through LDS; FT*4/KSPLIT
// feature groups per workgroup.  With FT = 2 a wave's token fragments serve
// twice the weight rows, which halves the token rows the workgroups read per
// weight byte; every output's k-steps and K-split sum keep their order, so
// the results are those of FT = 1, bit for bit.
// --------------------------------------------------------------------------
struct Gemm1Args {
  const uint8_t* w13;        // [E][2I][H]
  const uint8_t* act;        // bf16 x [M][H] or e4m3 xq [M][H]
  Segments seg;
  int H, I, top_k;
  const float* w_scale;      // fp8: s_w13, one per tensor or one per W13 row ([E][2I], w_cs = 1)
  const float* x_scale;      // fp8: s_x in effect
  const float* h_scale;      // fp8 static h: s_h
  uint8_t* h;                // [P][I] in HFMT
  unsigned* h_amax;          // fp8 dynamic: running max of |h| (float bits)
  int w_cs = 0;              // fp8: 1 = w_scale holds one scale per weight row, 0 = one per tensor
  int w_es = 0;              // fp8 without w_cs: 1 = one scale per expert (w_scale[e]), 0 = w_scale[0]
  int w_bs = 0;              // fp8: 1 = block-scaled (w_block, x_block; h written as fp32)
  const uint8_t* w_block;    // block-scaled: E8M0 codes [E][2I/128][H/128], one per 128 x 128 block of W13
  const uint8_t* x_block;    // block-scaled: E8M0 codes [M][H/128] of the activations' 128-element groups
};

// Weight-scale kinds of the fp8 bodies (template parameter WS): one scale per
// tensor or per expert (0), per weight row (1), or per 128 x 128 block, with
// the activations' per-128-element scales, fed to the scaled MFMA (2).
constexpr int kWsTensor = 0, kWsRow = 1, kWsBlock = 2;

// fp8 dequantisation factors s_a * s_w: with one scale per weight row (PC)
// those of the four rows row0..row0+3 of expert e (rows_e rows per expert),
// else the one scale of expert e (es = 1) or of the tensor (es = 0) for all
// four.  The kernels branch on w_cs once,
// at entry, into bodies specialised on PC, so the per-tensor bodies carry no
// per-row work.
template <bool PC>
__device__ __forceinline__ void row_deq4(const float* w_scale, int e, int rows_e, int row0, float sa, float (&d)[4],
                                         int es) {
  if constexpr (PC) {
    const float* ws = w_scale + (int64_t)e * rows_e;
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = sa * ws[row0 + r];
  } else {
    const float v = sa * w_scale[(int64_t)e * es];
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = v;
  }
}

// Body for NB (<= NT) token tiles; the kernel picks NB from the workgroup's
// token count so that tiles with no token issue no loads and no MFMAs.  bx:
// the workgroup's group of 4/KSPLIT feature tiles.  Returns the lane's
// largest |h| (0 in lanes that store nothing), which the caller reduces
// when the h scale is dynamic.
template <bool FP8, int HFMT, int NT, int NB, int U, int KSPLIT, int WS, int FT = 1>
__device__ __forceinline__ float gemm1_body(const Gemm1Args& a, f32x4* s_red, int e, int seg, int cnt, int pass0,
                                            int bx) {
  constexpr bool PC = WS == kWsRow, BS = FP8 && WS == kWsBlock;
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;   // k per MFMA
  constexpr int LB = FP8 ? 32 : 16;       // bytes per lane per operand per step
  constexpr int SB = KSTEP * ESZ;         // bytes per row per step
  constexpr int TPW = FT * 4 / KSPLIT;    // 16-feature groups per workgroup
  constexpr int NA = 2 * FT;              // weight tiles per wave: gate, up of each group

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kpart = wave % KSPLIT, tile = wave / KSPLIT;
  const int r16 = lane & 15, kq = lane >> 4;
  const int i0 = (bx * TPW + tile * FT) * 16;  // the wave's first feature
  const int Kw = a.H / KSPLIT;
  const int kbeg = kpart * Kw;

  const int64_t rowb = (int64_t)a.H * ESZ;
  const uint8_t* pa[NA];
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    pa[2 * f] = a.w13 + ((int64_t)e * 2 * a.I + i0 + 16 * f + r16) * rowb + (int64_t)kbeg * ESZ + kq * LB;  // gate
    pa[2 * f + 1] = pa[2 * f] + (int64_t)a.I * rowb;                                                        // up
  }
  const uint8_t* pb[NB];
  const uint8_t* qb[NB];  // block-scaled: the lane's token's group scales from kbeg on
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int slot = min(pass0 + t * 16 + r16, cnt - 1);
    const int m = a.seg.sorted_ids[seg + slot] / a.top_k;
    pb[t] = a.act + (int64_t)m * rowb + (int64_t)kbeg * ESZ + kq * LB;
    if constexpr (BS) qb[t] = a.x_block + (int64_t)m * (a.H / 128) + kbeg / 128;
  }

  f32x4 acc[NA][NB];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (BS) {
    // each gate and up tile's 128 x 128 weight block: rows (i0+16f)/128 and (I+i0+16f)/128
    const uint8_t* qa[NA];
    const int kg = a.H / 128;
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      qa[2 * f] = a.w_block + ((int64_t)e * (2 * a.I / 128) + (i0 + 16 * f) / 128) * kg + kbeg / 128;
      qa[2 * f + 1] = a.w_block + ((int64_t)e * (2 * a.I / 128) + (a.I + i0 + 16 * f) / 128) * kg + kbeg / 128;
    }
    stream_k<FP8, NA, NB, U, SB, true>(pa, pb, Kw / KSTEP, acc, qa, qb);
  } else {
    stream_k<FP8, NA, NB, U, SB>(pa, pb, Kw / KSTEP, acc);
  }

  if constexpr (KSPLIT > 1) {
    // partial tiles of K parts 1..KSPLIT-1: group g of the workgroup, token
    // tile t, gate (0) or up (1) at ((part-1)*TPW + g)*2*NT + 2t + (0|1)
    if (kpart > 0) {
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        f32x4* dst = s_red + (((kpart - 1) * TPW + tile * FT + f) * 2 * NT) * 64 + lane;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          dst[(2 * t) * 64] = acc[2 * f][t];
          dst[(2 * t + 1) * 64] = acc[2 * f + 1][t];
        }
      }
    }
    __syncthreads();
    if (kpart > 0) return 0.0f;
#pragma unroll
    for (int p = 0; p < KSPLIT - 1; ++p)
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const f32x4* src = s_red + ((p * TPW + tile * FT + f) * 2 * NT) * 64 + lane;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          acc[2 * f][t] += src[(2 * t) * 64];
          acc[2 * f + 1][t] += src[(2 * t + 1) * 64];
        }
      }
  }

  float rh = 1.0f;
  if constexpr (HFMT == H_E4M3) rh = 1.0f / *a.h_scale;
  float hmax = 0.0f;
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    const int i0f = i0 + 16 * f;
    // dequantisation of this lane's rows: gate rows i0f+4kq.., up rows I+i0f+4kq..
    float dg[4] = {1.0f, 1.0f, 1.0f, 1.0f}, du[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (FP8 && !BS) {  // block-scaled: the MFMA applied the scales
      row_deq4<PC>(a.w_scale, e, 2 * a.I, i0f + kq * 4, *a.x_scale, dg, a.w_es);
      row_deq4<PC>(a.w_scale, e, 2 * a.I, a.I + i0f + kq * 4, *a.x_scale, du, a.w_es);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int slot = pass0 + t * 16 + r16;
      if (slot < cnt) {
        const int pf = a.seg.sorted_ids[seg + slot];
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = acc[2 * f][t][r] * dg[r];
          const float u = acc[2 * f + 1][t][r] * du[r];
          hv[r] = g / (1.0f + expf(-g)) * u;
          hmax = fmaxf(hmax, fabsf(hv[r]));
        }
        const int64_t idx = (int64_t)pf * a.I + i0f + kq * 4;
        if constexpr (HFMT == H_BF16) {
          u32x2 o = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          *(u32x2*)(a.h + idx * 2) = o;
        } else if constexpr (HFMT == H_F32) {
          *(f32x4*)(a.h + idx * 4) = f32x4{hv[0], hv[1], hv[2], hv[3]};
        } else {
          *(unsigned*)(a.h + idx) = pack_e4m3x4(hv[0] * rh, hv[1] * rh, hv[2] * rh, hv[3] * rh);
        }
      }
    }
  }
  return hmax;
}

template <bool FP8, int HFMT, int NT, int U, int KSPLIT, int FT = 1>
static __global__ __launch_bounds__(256) void gemm1_decode_kernel(Gemm1Args a) {
  constexpr int TPW = FT * 4 / KSPLIT;
  __shared__ f32x4 s_red[KSPLIT > 1 ? (KSPLIT - 1) * TPW * 2 * NT * 64 : 1];
  const int s = grid_y(a.seg);
  if (s >= *a.seg.num_active) return;
  const int e = a.seg.active[s];
  const int seg = a.seg.offsets[e], cnt = a.seg.counts[e];
  const int pass0 = grid_z(a.seg) * NT * 16;
  if (pass0 >= cnt) return;
  const int ntile = min(NT, (cnt - pass0 + 15) >> 4);  // uniform over the workgroup
  auto run = [&](auto ws_tag) {
    constexpr int WS = decltype(ws_tag)::value;
    const int bx = blockIdx.x;
    if constexpr (NT >= 4)
      if (ntile == 4) return gemm1_body<FP8, HFMT, NT, 4, U, KSPLIT, WS, FT>(a, s_red, e, seg, cnt, pass0, bx);
    if constexpr (NT >= 3)
      if (ntile == 3) return gemm1_body<FP8, HFMT, NT, 3, U, KSPLIT, WS, FT>(a, s_red, e, seg, cnt, pass0, bx);
    if constexpr (NT >= 2)
      if (ntile == 2) return gemm1_body<FP8, HFMT, NT, 2, U, KSPLIT, WS, FT>(a, s_red, e, seg, cnt, pass0, bx);
    return gemm1_body<FP8, HFMT, NT, 1, U, KSPLIT, WS, FT>(a, s_red, e, seg, cnt, pass0, bx);
  };
  float hmax;
  if constexpr (FP8 && HFMT == H_F32) {
    if (a.w_bs) {  // block-scaled: h is quantised per block later, no tensor amax
      run(std::integral_constant<int, kWsBlock>{});
      return;
    }
  }
  if constexpr (FP8)  // one weight scale per row, or per tensor / expert
    hmax = a.w_cs ? run(std::integral_constant<int, kWsRow>{}) : run(std::integral_constant<int, kWsTensor>{});
  else
    hmax = run(std::integral_constant<int, kWsTensor>{});
  if constexpr (HFMT == H_F32) {
    // one device-scope atomic per wave that stored h (same-address atomics
    // serialise: an atomic from every wave cost 8-25 us on the M = 1 layers)
    hmax = wave_max(hmax);
    if ((threadIdx.x & 63) == 0 && hmax > 0.0f) atomicMax(a.h_amax, __float_as_uint(hmax));
  }
}

// --------------------------------------------------------------------------
// Long-stream pipeline shared by the long-stream variants of both products.
//
// A wave walks T tiles of one expert over the same K range; tile j's A rows
// start at pa[i] + j * tstride and the token operand (B) is the same for all
// tiles.  The K loop of a tile has S stages of U MFMA k-steps; the stages of
// all tiles form one flat sequence through a ring of NS register stages
// (NS-1 stages of loads in flight while one is computed), so the first loads
// of tile j+1 are in flight while tile j finishes and the pipeline ramps once
// per T tiles.  Past the last stage the loads repeat the first stage (in
// range, never used).  epi(j, acc) consumes and clears the accumulators of
// tile j.
// --------------------------------------------------------------------------
template <int U>
constexpr int stream_stages() { return U == 1 ? 4 : 3; }

template <bool FP8, int NB, int U, int SB, typename Epi>
__device__ __forceinline__ void stream_tiles(const uint8_t* const (&pa)[2], int64_t tstride, const uint8_t* const* pb,
                                             int ntiles, int S, f32x4 (&acc)[2][NB], Epi&& epi) {
  constexpr int SS = U * SB;
  constexpr int NS = stream_stages<U>();
  const int G = ntiles * S;
  StageRegs<FP8, 2, NB, U> sr[NS];
  int lj = 0, ls = 0;  // next stage to load
  auto load_next = [&](StageRegs<FP8, 2, NB, U>& r) {
    const bool in = lj < ntiles;
    const int64_t ao = in ? (int64_t)lj * tstride + (int64_t)ls * SS : 0;
    const int bo = in ? ls * SS : 0;
#pragma unroll
    for (int q = 0; q < U; ++q) {
      load_frag<FP8>(r.a[q][0], pa[0] + ao + q * SB);
      load_frag<FP8>(r.a[q][1], pa[1] + ao + q * SB);
#pragma unroll
      for (int t = 0; t < NB; ++t) load_frag<FP8>(r.b[q][t], pb[t] + bo + q * SB);
    }
    if (++ls == S) {
      ls = 0;
      ++lj;
    }
  };
  int cj = 0, cs = 0;  // stage being computed
  auto compute = [&](const StageRegs<FP8, 2, NB, U>& r) {
    stage_mma<FP8, 2, NB, U>(r, acc);
    if (++cs == S) {
      epi(cj, acc);
      cs = 0;
      ++cj;
    }
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) load_next(sr[p]);
  for (int g = 0; g < G; g += NS) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      load_next(sr[(p + NS - 1) % NS]);  // stage g + p + NS - 1
      __builtin_amdgcn_sched_barrier(0);
      if (p == 0 || g + p < G) compute(sr[p]);  // stage g + p
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Gate/up product, long-stream variant.  Wave w of the workgroup walks tw
// feature tiles (tile f: gate rows 16f.. and up rows I+16f.. of W13[e])
// ft0 + 4j, ft0 = 4*tw*blockIdx.x + w, over the whole K = H, so that the four
// waves read 64 adjacent gate rows and their up partners at each point of the
// stream.  Token rows and output slots are read once per wave.  No K split,
// no LDS, no barrier.
template <bool FP8, int HFMT, int NB, int U, bool PC>
__device__ __forceinline__ void gemm1_stream_body(const Gemm1Args& a, int e, int seg, int cnt, int pass0, int tw) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;
  constexpr int LB = FP8 ? 32 : 16;
  constexpr int SB = KSTEP * ESZ;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
  const int r16 = lane & 15, kq = lane >> 4;
  const int ftiles = a.I >> 4;
  const int ft0 = blockIdx.x * 4 * tw + wave;
  if (ft0 >= ftiles) return;
  const int ntw = min(tw, (ftiles - ft0 + 3) >> 2);

  const int64_t rowb = (int64_t)a.H * ESZ;
  const uint8_t* pa[2];
  pa[0] = a.w13 + ((int64_t)e * 2 * a.I + ft0 * 16 + r16) * rowb + kq * LB;  // gate rows
  pa[1] = pa[0] + (int64_t)a.I * rowb;                                        // up rows
  const uint8_t* pb[NB];
  int fo[NB];  // pair of the lane's token column, -1 past the expert's count
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int slot = pass0 + t * 16 + r16;
    const int f = a.seg.sorted_ids[seg + min(slot, cnt - 1)];
    pb[t] = a.act + (int64_t)(f / a.top_k) * rowb + kq * LB;
    fo[t] = slot < cnt ? f : -1;
  }

  const float sx = FP8 ? *a.x_scale : 1.0f;
  float dg[4] = {1.0f, 1.0f, 1.0f, 1.0f}, du[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if constexpr (FP8 && !PC) {  // one scale per tensor: the same factors for every tile
    row_deq4<false>(a.w_scale, e, 0, 0, sx, dg, a.w_es);
    row_deq4<false>(a.w_scale, e, 0, 0, sx, du, a.w_es);
  }
  float rh = 1.0f;
  if constexpr (HFMT == H_E4M3) rh = 1.0f / *a.h_scale;
  float hmax = 0.0f;
  f32x4 acc[2][NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[0][t] = acc[1][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto epi = [&](int j, f32x4 (&c)[2][NB]) {
    const int i0 = (ft0 + 4 * j) * 16;
    if constexpr (FP8 && PC) {
      row_deq4<true>(a.w_scale, e, 2 * a.I, i0 + kq * 4, sx, dg, a.w_es);
      row_deq4<true>(a.w_scale, e, 2 * a.I, a.I + i0 + kq * 4, sx, du, a.w_es);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      if (fo[t] >= 0) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = c[0][t][r] * dg[r];
          const float u = c[1][t][r] * du[r];
          hv[r] = g / (1.0f + expf(-g)) * u;
          hmax = fmaxf(hmax, fabsf(hv[r]));
        }
        const int64_t idx = (int64_t)fo[t] * a.I + i0 + kq * 4;
        if constexpr (HFMT == H_BF16) {
          u32x2 o = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          *(u32x2*)(a.h + idx * 2) = o;
        } else if constexpr (HFMT == H_F32) {
          *(f32x4*)(a.h + idx * 4) = f32x4{hv[0], hv[1], hv[2], hv[3]};
        } else {
          *(unsigned*)(a.h + idx) = pack_e4m3x4(hv[0] * rh, hv[1] * rh, hv[2] * rh, hv[3] * rh);
        }
      }
      c[0][t] = c[1][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  stream_tiles<FP8, NB, U, SB>(pa, 64 * rowb, pb, ntw, a.H / KSTEP / U, acc, epi);
  if constexpr (HFMT == H_F32) {
    hmax = wave_max(hmax);
    if (lane == 0 && hmax > 0.0f) atomicMax(a.h_amax, __float_as_uint(hmax));
  }
}

// Grid: x = chunks of 4*tw feature tiles, y = active expert, z = token pass.
template <bool FP8, int HFMT, int NT, int U>
static __global__ __launch_bounds__(256) void gemm1_stream_kernel(Gemm1Args a, int tw) {
  const int s = grid_y(a.seg);
  if (s >= *a.seg.num_active) return;
  const int e = a.seg.active[s];
  const int seg = a.seg.offsets[e], cnt = a.seg.counts[e];
  const int pass0 = grid_z(a.seg) * NT * 16;
  if (pass0 >= cnt) return;
  const int ntile = min(NT, (cnt - pass0 + 15) >> 4);  // uniform over the workgroup
  auto run = [&](auto pc_tag) {
    constexpr bool PC = decltype(pc_tag)::value;
    if constexpr (NT >= 4)
      if (ntile == 4) return gemm1_stream_body<FP8, HFMT, 4, U, PC>(a, e, seg, cnt, pass0, tw);
    if constexpr (NT >= 3)
      if (ntile == 3) return gemm1_stream_body<FP8, HFMT, 3, U, PC>(a, e, seg, cnt, pass0, tw);
    if constexpr (NT >= 2)
      if (ntile == 2) return gemm1_stream_body<FP8, HFMT, 2, U, PC>(a, e, seg, cnt, pass0, tw);
    gemm1_stream_body<FP8, HFMT, 1, U, PC>(a, e, seg, cnt, pass0, tw);
  };
  if constexpr (FP8)
    if (a.w_cs) return run(std::true_type{});  // one weight scale per row
  run(std::false_type{});
}

// --------------------------------------------------------------------------
// Down product.
//
// Wave tile: 32 output rows (two 16-row MFMA tiles of W2[e]) over one K
// slice of I, times the workgroup's 16-token tiles.  Each wave stores its
// dequantised partial sums with plain stores into part[kslice][pair][row]:
// every element is written by exactly one wave, so no atomics and no
// clearing are needed, and the top-k combine (the routing-weighted sum over
// the token's experts and over the K slices) happens in a fixed order in
// the finalize kernel, which makes the layer's output bitwise reproducible.
//
// Token operand: bf16 h or static-scale e4m3 h is read from global memory
// (L2-resident) like the weights.  With a dynamic fp8 scale h is kept in fp32
// and its per-tensor scale is only known once the gate/up product is done, so
// each workgroup first quantises the h slice of its tokens into LDS (the four
// waves of a workgroup share the same tokens and K slice) and the main loop
// reads the token operand from there.
// --------------------------------------------------------------------------
struct Gemm2Args {
  const uint8_t* w2;         // [E][H][I]
  const uint8_t* h;          // [P][I] in HFMT
  Segments seg;
  const float* topk_w;       // [P]
  int H, I, top_k, ksplit;
  const float* w_scale;      // fp8: s_w2, one per tensor or one per W2 row ([E][H], w_cs = 1)
  const float* h_scale;      // fp8 static: s_h
  const unsigned* h_amax;    // fp8 dynamic: max |h| (float bits)
  float* part;               // [ksplit][P][H] partial outputs
  int P;
  int w_cs = 0;              // fp8: 1 = one scale per weight row, 0 = one per tensor
  int w_es = 0;              // fp8 without w_cs: 1 = one scale per expert (w_scale[e]), 0 = w_scale[0]
  int w_bs = 0;              // fp8: 1 = block-scaled (w_block; h, fp32, quantised per 128-element group)
  const uint8_t* w_block;    // block-scaled: E8M0 codes [E][H/128][I/128], one per 128 x 128 block of W2
};

// LDS row stride (bytes) of the quantised token slice: Kw plus 16 bytes so
// that the 16 token rows read by one instruction fall in different banks.
__host__ __device__ constexpr int gemm2_lds_stride(int kw_bytes) { return kw_bytes + 16; }

// Quantise the workgroup's token slice of fp32 h into LDS: NB*16 rows (token
// slots pass0.., clamped to the expert's count) of Kw e4m3 bytes from column
// kbeg, row stride gemm2_lds_stride(Kw).  All 256 threads take part; the
// caller synchronises.
template <int NB>
__device__ __forceinline__ void stage_h_e4m3(const Gemm2Args& a, uint8_t* s_tok, int seg, int cnt, int pass0, int kbeg,
                                             int Kw, float rh) {
  const int stride = gemm2_lds_stride(Kw);
  const int per_row = Kw / 16;  // 16 elements per thread-step
  for (int idx = threadIdx.x; idx < NB * 16 * per_row; idx += 256) {
    const int row = idx / per_row, c = (idx - row * per_row) * 16;
    const int slot = min(pass0 + row, cnt - 1);
    const int f = a.seg.sorted_ids[seg + slot];
    const float* src = (const float*)a.h + (int64_t)f * a.I + kbeg + c;
    const f32x4 v0 = *(const f32x4*)(src), v1 = *(const f32x4*)(src + 4);
    const f32x4 v2 = *(const f32x4*)(src + 8), v3 = *(const f32x4*)(src + 12);
    u32x4 q = {pack_e4m3x4(v0[0] * rh, v0[1] * rh, v0[2] * rh, v0[3] * rh),
               pack_e4m3x4(v1[0] * rh, v1[1] * rh, v1[2] * rh, v1[3] * rh),
               pack_e4m3x4(v2[0] * rh, v2[1] * rh, v2[2] * rh, v2[3] * rh),
               pack_e4m3x4(v3[0] * rh, v3[1] * rh, v3[2] * rh, v3[3] * rh)};
    *(u32x4*)(s_tok + row * stride + c) = q;
  }
}

// Block-scaled variant: each 128-element group of a token row gets its own
// power-of-two scale (OCP MX rule, block_scale_code), whose E8M0 code goes to
// the byte array after the NB*16 token rows, Kw/128 codes per row.  Eight
// consecutive threads take one group (16 elements each) and share its amax
// through DPP, so every thread runs every round (rows past the slice take
// part with zeros).
__host__ __device__ constexpr int gemm2_block_scale_bytes(int rows, int kw_bytes) { return rows * (kw_bytes / 128); }

template <int NB>
__device__ __forceinline__ void stage_h_block(const Gemm2Args& a, uint8_t* s_tok, int seg, int cnt, int pass0,
                                              int kbeg, int Kw) {
  const int stride = gemm2_lds_stride(Kw);
  const int per_row = Kw / 16;  // 16 elements per thread-step, 8 steps per group
  const int total = NB * 16 * per_row;
  uint8_t* s_scale = s_tok + NB * 16 * stride;
  for (int base = 0; base < total; base += 256) {
    const int idx = base + threadIdx.x;
    const bool live = idx < total;  // whole groups are live or not: total is a multiple of 128
    const int j = live ? idx : 0;
    const int row = j / per_row, c = (j - row * per_row) * 16;
    const int slot = min(pass0 + row, cnt - 1);
    const int f = a.seg.sorted_ids[seg + slot];
    const float* src = (const float*)a.h + (int64_t)f * a.I + kbeg + c;
    const f32x4 v0 = *(const f32x4*)(src), v1 = *(const f32x4*)(src + 4);
    const f32x4 v2 = *(const f32x4*)(src + 8), v3 = *(const f32x4*)(src + 12);
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v0[q]), fabsf(v1[q])), fmaxf(fabsf(v2[q]), fabsf(v3[q]))));
    m = max8(live ? m : 0.0f);
    const int code = block_scale_code(m);
    const float r = block_scale_recip(code);
    if (live) {
      u32x4 q = {pack_e4m3x4(v0[0] * r, v0[1] * r, v0[2] * r, v0[3] * r),
                 pack_e4m3x4(v1[0] * r, v1[1] * r, v1[2] * r, v1[3] * r),
                 pack_e4m3x4(v2[0] * r, v2[1] * r, v2[2] * r, v2[3] * r),
                 pack_e4m3x4(v3[0] * r, v3[1] * r, v3[2] * r, v3[3] * r)};
      *(u32x4*)(s_tok + row * stride + c) = q;
      if ((idx & 7) == 0) s_scale[row * (Kw / 128) + c / 128] = (uint8_t)code;
    }
  }
}

// Body for NB (<= NT) token tiles.  WKS waves of the workgroup split the
// slice's K range and are summed through LDS (s_red); each wave computes FR
// groups of 32 rows, FR*4/WKS groups per workgroup (FR = 2: a wave's token
// fragments serve twice the weight rows; every output's sums keep their
// order, so the results are those of FR = 1, bit for bit).
template <bool FP8, int HFMT, int NT, int NB, int U, int WKS, int WS, int FR = 1>
__device__ __forceinline__ void gemm2_body(const Gemm2Args& a, uint8_t* s_tok, f32x4* s_red, int e, int seg, int cnt,
                                           int pass0, int kslice, int bx) {
  constexpr bool PC = WS == kWsRow, BS = FP8 && HFMT == H_F32 && WS == kWsBlock;
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;
  constexpr int LB = FP8 ? 32 : 16;
  constexpr int SB = KSTEP * ESZ;
  constexpr int HSZ = HFMT == H_BF16 ? 2 : (HFMT == H_F32 ? 4 : 1);
  constexpr bool QH = FP8 && HFMT == H_F32;  // token operand staged in LDS
  constexpr int TPW = FR * 4 / WKS;          // 32-row groups per workgroup
  constexpr int NA = 2 * FR;                 // 16-row weight tiles per wave

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kpart = wave % WKS, tile = wave / WKS;
  const int r16 = lane & 15, kq = lane >> 4;
  const int n0 = (bx * TPW + tile * FR) * 32;  // the wave's first row
  const int Kw = a.I / a.ksplit;       // K range of the workgroup
  const int kbeg = kslice * Kw;
  const int Kp = Kw / WKS;             // K range of the wave
  const int koff = kpart * Kp;

  // dequantisation of this lane's rows n0+16i+4kq.. of weight tile i
  float d[NA][4];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) d[i][r] = 1.0f;
  if constexpr (BS) {  // the MFMA applies the scales
    stage_h_block<NB>(a, s_tok, seg, cnt, pass0, kbeg, Kw);
    __syncthreads();
  } else if constexpr (FP8) {
    const float sh = (HFMT == H_F32) ? scale_from_amax(__uint_as_float(*a.h_amax)) : *a.h_scale;
#pragma unroll
    for (int i = 0; i < NA; ++i) row_deq4<PC>(a.w_scale, e, a.H, n0 + 16 * i + kq * 4, sh, d[i], a.w_es);
    if constexpr (QH) {
      stage_h_e4m3<NB>(a, s_tok, seg, cnt, pass0, kbeg, Kw, 1.0f / sh);
      __syncthreads();
    }
  }

  const int64_t rowb = (int64_t)a.I * ESZ;
  const uint8_t* pa[NA];
  pa[0] = a.w2 + ((int64_t)e * a.H + n0 + r16) * rowb + (int64_t)(kbeg + koff) * ESZ + kq * LB;
#pragma unroll
  for (int i = 1; i < NA; ++i) pa[i] = pa[0] + 16 * i * rowb;
  const uint8_t* pb[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if constexpr (QH) {
      pb[t] = s_tok + (t * 16 + r16) * gemm2_lds_stride(Kw) + koff + kq * LB;
    } else {
      const int slot = min(pass0 + t * 16 + r16, cnt - 1);
      const int f = a.seg.sorted_ids[seg + slot];
      pb[t] = a.h + ((int64_t)f * a.I + kbeg + koff) * HSZ + kq * LB;
    }
  }

  f32x4 acc[NA][NB];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (BS) {
    // each 16-row tile's 128 x 128 weight block; the token rows' group
    // scales follow the staged slice
    const uint8_t* qa[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i)
      qa[i] = a.w_block + ((int64_t)e * (a.H / 128) + (n0 + 16 * i) / 128) * (a.I / 128) + (kbeg + koff) / 128;
    const uint8_t* qb[NB];
    const uint8_t* s_scale = s_tok + NB * 16 * gemm2_lds_stride(Kw);
#pragma unroll
    for (int t = 0; t < NB; ++t) qb[t] = s_scale + (t * 16 + r16) * (Kw / 128) + koff / 128;
    stream_k<FP8, NA, NB, U, SB, true>(pa, pb, Kp / KSTEP, acc, qa, qb);
  } else {
    stream_k<FP8, NA, NB, U, SB>(pa, pb, Kp / KSTEP, acc);
  }

  if constexpr (WKS > 1) {
    // partial tiles of K parts 1..WKS-1: group g of the workgroup, token tile
    // t, 16-row half h at ((part-1)*TPW + g)*2*NT + 2t + h
    if (kpart > 0) {
#pragma unroll
      for (int g = 0; g < FR; ++g) {
        f32x4* dst = s_red + (((kpart - 1) * TPW + tile * FR + g) * 2 * NT) * 64 + lane;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          dst[(2 * t) * 64] = acc[2 * g][t];
          dst[(2 * t + 1) * 64] = acc[2 * g + 1][t];
        }
      }
    }
    __syncthreads();
    if (kpart > 0) return;
#pragma unroll
    for (int p = 0; p < WKS - 1; ++p)
#pragma unroll
      for (int g = 0; g < FR; ++g) {
        const f32x4* src = s_red + ((p * TPW + tile * FR + g) * 2 * NT) * 64 + lane;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          acc[2 * g][t] += src[(2 * t) * 64];
          acc[2 * g + 1][t] += src[(2 * t + 1) * 64];
        }
      }
  }

  float* part = a.part + (int64_t)kslice * a.P * a.H;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int slot = pass0 + t * 16 + r16;
    if (slot < cnt) {
      const int f = a.seg.sorted_ids[seg + slot];
      float* dst = part + (int64_t)f * a.H + n0 + kq * 4;
#pragma unroll
      for (int i = 0; i < NA; ++i)
        *(f32x4*)(dst + 16 * i) = acc[i][t] * f32x4{d[i][0], d[i][1], d[i][2], d[i][3]};
    }
  }
}

// Grid: x = groups of 32*FR*(4/WKS) output rows, y = active expert, z = K
// slice + ksplit * token pass.
template <bool FP8, int HFMT, int NT, int U, int WKS, int FR = 1>
static __global__ __launch_bounds__(256) void gemm2_decode_kernel(Gemm2Args a) {
  extern __shared__ __align__(16) uint8_t s_tok[];
  constexpr int TPW = FR * 4 / WKS;
  __shared__ f32x4 s_red[WKS > 1 ? (WKS - 1) * TPW * 2 * NT * 64 : 1];
  const int s = grid_y(a.seg);
  if (s >= *a.seg.num_active) return;
  const int e = a.seg.active[s];
  const int seg = a.seg.offsets[e], cnt = a.seg.counts[e];
  const int z = grid_z(a.seg), kslice = z % a.ksplit;
  const int pass0 = (z / a.ksplit) * NT * 16;
  if (pass0 >= cnt) return;
  const int ntile = min(NT, (cnt - pass0 + 15) >> 4);  // uniform over the workgroup
  auto run = [&](auto ws_tag) {
    constexpr int WS = decltype(ws_tag)::value;
    if constexpr (NT >= 4)
      if (ntile == 4)
        return gemm2_body<FP8, HFMT, NT, 4, U, WKS, WS, FR>(a, s_tok, s_red, e, seg, cnt, pass0, kslice, blockIdx.x);
    if constexpr (NT >= 3)
      if (ntile == 3)
        return gemm2_body<FP8, HFMT, NT, 3, U, WKS, WS, FR>(a, s_tok, s_red, e, seg, cnt, pass0, kslice, blockIdx.x);
    if constexpr (NT >= 2)
      if (ntile == 2)
        return gemm2_body<FP8, HFMT, NT, 2, U, WKS, WS, FR>(a, s_tok, s_red, e, seg, cnt, pass0, kslice, blockIdx.x);
    gemm2_body<FP8, HFMT, NT, 1, U, WKS, WS, FR>(a, s_tok, s_red, e, seg, cnt, pass0, kslice, blockIdx.x);
  };
  if constexpr (FP8 && HFMT == H_F32)
    if (a.w_bs) return run(std::integral_constant<int, kWsBlock>{});  // block-scaled
  if constexpr (FP8)
    if (a.w_cs) return run(std::integral_constant<int, kWsRow>{});  // one weight scale per row
  run(std::integral_constant<int, kWsTensor>{});
}

// Down product, long-stream variant.  Wave w of the workgroup walks tw tiles
// of 32 output rows of W2[e] (tile rt0 + 4j, rt0 = 4*tw*blockIdx.x + w) over
// the workgroup's K slice, the pipeline running on from tile to tile; the
// token slice (quantised into LDS once per workgroup with a dynamic fp8 h
// scale, else read from global memory) serves all of them.
template <bool FP8, int HFMT, int NB, int U, bool PC>
__device__ __forceinline__ void gemm2_stream_body(const Gemm2Args& a, uint8_t* s_tok, int e, int seg, int cnt,
                                                  int pass0, int kslice, int tw) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;
  constexpr int LB = FP8 ? 32 : 16;
  constexpr int SB = KSTEP * ESZ;
  constexpr int HSZ = HFMT == H_BF16 ? 2 : (HFMT == H_F32 ? 4 : 1);
  constexpr bool QH = FP8 && HFMT == H_F32;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
  const int r16 = lane & 15, kq = lane >> 4;
  const int Kw = a.I / a.ksplit;
  const int kbeg = kslice * Kw;

  float sh = 1.0f;
  float d0[4] = {1.0f, 1.0f, 1.0f, 1.0f}, d1[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if constexpr (FP8) {
    sh = (HFMT == H_F32) ? scale_from_amax(__uint_as_float(*a.h_amax)) : *a.h_scale;
    if constexpr (!PC) {  // one scale per tensor: the same factors for every tile
      row_deq4<false>(a.w_scale, e, 0, 0, sh, d0, a.w_es);
      row_deq4<false>(a.w_scale, e, 0, 0, sh, d1, a.w_es);
    }
    if constexpr (QH) {
      stage_h_e4m3<NB>(a, s_tok, seg, cnt, pass0, kbeg, Kw, 1.0f / sh);
      __syncthreads();
    }
  }
  const int rtiles = a.H >> 5;
  const int rt0 = blockIdx.x * 4 * tw + wave;
  if (rt0 >= rtiles) return;  // after the workgroup's only barrier
  const int ntw = min(tw, (rtiles - rt0 + 3) >> 2);

  const int64_t rowb = (int64_t)a.I * ESZ;
  const uint8_t* pa[2];
  pa[0] = a.w2 + ((int64_t)e * a.H + rt0 * 32 + r16) * rowb + (int64_t)kbeg * ESZ + kq * LB;
  pa[1] = pa[0] + 16 * rowb;
  const uint8_t* pb[NB];
  int fo[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int slot = pass0 + t * 16 + r16;
    const int f = a.seg.sorted_ids[seg + min(slot, cnt - 1)];
    fo[t] = slot < cnt ? f : -1;
    if constexpr (QH)
      pb[t] = s_tok + (t * 16 + r16) * gemm2_lds_stride(Kw) + kq * LB;
    else
      pb[t] = a.h + ((int64_t)f * a.I + kbeg) * HSZ + kq * LB;
  }

  float* part = a.part + (int64_t)kslice * a.P * a.H;
  f32x4 acc[2][NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[0][t] = acc[1][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto epi = [&](int j, f32x4 (&c)[2][NB]) {
    const int n0 = (rt0 + 4 * j) * 32;
    if constexpr (FP8 && PC) {
      row_deq4<true>(a.w_scale, e, a.H, n0 + kq * 4, sh, d0, a.w_es);
      row_deq4<true>(a.w_scale, e, a.H, n0 + 16 + kq * 4, sh, d1, a.w_es);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      if (fo[t] >= 0) {
        float* dst = part + (int64_t)fo[t] * a.H + n0 + kq * 4;
        *(f32x4*)dst = c[0][t] * f32x4{d0[0], d0[1], d0[2], d0[3]};
        *(f32x4*)(dst + 16) = c[1][t] * f32x4{d1[0], d1[1], d1[2], d1[3]};
      }
      c[0][t] = c[1][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  stream_tiles<FP8, NB, U, SB>(pa, 128 * rowb, pb, ntw, Kw / KSTEP / U, acc, epi);
}

// Grid: x = chunks of 4*tw row tiles, y = active expert, z = K slice +
// ksplit * token pass.
template <bool FP8, int HFMT, int NT, int U>
static __global__ __launch_bounds__(256) void gemm2_stream_kernel(Gemm2Args a, int tw) {
  extern __shared__ __align__(16) uint8_t s_tok[];
  const int s = grid_y(a.seg);
  if (s >= *a.seg.num_active) return;
  const int e = a.seg.active[s];
  const int seg = a.seg.offsets[e], cnt = a.seg.counts[e];
  const int z = grid_z(a.seg), kslice = z % a.ksplit;
  const int pass0 = (z / a.ksplit) * NT * 16;
  if (pass0 >= cnt) return;
  const int ntile = min(NT, (cnt - pass0 + 15) >> 4);  // uniform over the workgroup
  auto run = [&](auto pc_tag) {
    constexpr bool PC = decltype(pc_tag)::value;
    if constexpr (NT >= 4)
      if (ntile == 4) return gemm2_stream_body<FP8, HFMT, 4, U, PC>(a, s_tok, e, seg, cnt, pass0, kslice, tw);
    if constexpr (NT >= 3)
      if (ntile == 3) return gemm2_stream_body<FP8, HFMT, 3, U, PC>(a, s_tok, e, seg, cnt, pass0, kslice, tw);
    if constexpr (NT >= 2)
      if (ntile == 2) return gemm2_stream_body<FP8, HFMT, 2, U, PC>(a, s_tok, e, seg, cnt, pass0, kslice, tw);
    gemm2_stream_body<FP8, HFMT, 1, U, PC>(a, s_tok, e, seg, cnt, pass0, kslice, tw);
  };
  if constexpr (FP8)
    if (a.w_cs) return run(std::true_type{});  // one weight scale per row
  run(std::false_type{});
}

// LDS of a down-product workgroup: the K-split reduction buffer (fr 32-row
// groups per wave).
__host__ __device__ constexpr int gemm2_red_bytes(int nt, int wks, int fr = 1) {
  return wks > 1 ? (wks - 1) * (fr * 4 / wks) * 2 * nt * 64 * 16 : 16;
}

// Top-k combine and output rounding:
//   y[m,n] = bf16( sum_j w[m,j] * (sum_s part[s][m*k+j][n]) )
// One lane per (G groups of four outputs, expert slot j): the lane loads its
// K slices (s ascending), scales by w[m,j], and the KP lanes of a
// group (KP = k rounded up to a power of two) add their terms by a fixed
// xor-butterfly, so the result does not depend on scheduling and every call
// gives the same bits.  G = 4 at large M keeps four groups' loads in flight
// per lane with a quarter of the workgroups; every output is the same sum.
// Also reports the fp8 scales in effect.
template <int G>
static __global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ part, const float* __restrict__ topk_w,
                                                       uint16_t* __restrict__ y, int M, int H, int top_k, int log2kp,
                                                       int ksplit, const float* x_scale, const unsigned* h_amax,
                                                       const float* h_scale, float* scales_out) {
  if (scales_out && blockIdx.x == 0 && threadIdx.x == 0) {
    scales_out[0] = *x_scale;
    scales_out[1] = h_scale ? *h_scale : scale_from_amax(__uint_as_float(*h_amax));
  }
  const int kp = 1 << log2kp;
  const int64_t g = (((int64_t)blockIdx.x * 256 + threadIdx.x) >> log2kp) * G;  // first output group
  const int j = threadIdx.x & (kp - 1);
  const int64_t i = g * 4;  // G groups of 4 outputs, one row (H is a multiple of 4*G)
  const bool live = i < (int64_t)M * H;
  const int m = live ? (int)(i / H) : 0, n = live ? (int)(i - (int64_t)m * H) : 0;
  f32x4 acc[G];
#pragma unroll
  for (int q = 0; q < G; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (live && j < top_k) {
    const int64_t f = (int64_t)m * top_k + j;
    const int64_t slice = (int64_t)M * top_k * H;
    const float* p = part + f * H + n;
    const float w = topk_w[f];
    if constexpr (G == 1) {  // every slice in flight at once
      f32x4 v[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) v[s] = s < ksplit ? *(const f32x4*)(p + s * slice) : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 o = v[0];
#pragma unroll
      for (int s = 1; s < 16; ++s)
        if (s < ksplit) o += v[s];
      acc[0] = o * w;
    } else {  // the G groups of a slice in flight at once, slices in order
      f32x4 o[G];
#pragma unroll
      for (int q = 0; q < G; ++q) o[q] = *(const f32x4*)(p + 4 * q);
      for (int s = 1; s < ksplit; ++s)
#pragma unroll
        for (int q = 0; q < G; ++q) o[q] += *(const f32x4*)(p + s * slice + 4 * q);
#pragma unroll
      for (int q = 0; q < G; ++q) acc[q] = o[q] * w;
    }
  }
#pragma unroll
  for (int q = 0; q < G; ++q)
    for (int off = 1; off < kp; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[q][c] += __shfl_xor(acc[q][c], off);
    }
  if (live && j == 0) {
#pragma unroll
    for (int q = 0; q < G; ++q) {
      uint2 out = {pack_bf16x2(acc[q][0], acc[q][1]), pack_bf16x2(acc[q][2], acc[q][3])};
      *(uint2*)(y + i + 4 * q) = out;
    }
  }
}

// --------------------------------------------------------------------------
// Down product with the weighted top-k combine in its epilogue, for small
// layers (at most kTokDownPairs pairs).  One workgroup owns 16 output rows of
// one token and computes
//   y[m][n0..n0+15] = bf16( sum_j w_j * d_j * (W2[e_j][n0..n0+15] . h_(m,j)) )
// over the token's pairs j itself (d_j: the pair's fp8 dequantisation
// s_h * s_w2, 1 in bf16).  The token's pairs use different experts, so the
// four waves split the token's units (pair j, K chunk c) of 16 weight rows:
// wave w takes units w, w + 4, ..., two at a time (two weight tiles and two h
// chunks in flight, the two cross products of the MFMA pair unused); every
// MFMA's sixteen B columns hold the same h chunk and column 0's results are
// used.  Each wave adds its units' weighted, dequantised sums in unit order,
// and the four waves' sums are added in wave order through LDS.  So every
// output is one workgroup's fixed sequence of operations: no partial sums in
// HBM, no atomics, no finalize launch, repeated calls give the same bits.
// With a dynamic fp8 h scale the workgroup first quantises its token's h
// rows into LDS (the token's pairs m*kk..m*kk+kk-1 are consecutive rows of h).
// --------------------------------------------------------------------------
constexpr int kTokDownPairs = 64;     // layers with at most this many pairs M*kk
constexpr int kTokDownLds = 65536;    // LDS of the staged e4m3 h rows of one token (dynamic scale)

struct DownTokArgs {
  const uint8_t* w2;       // [E][H][I]
  const uint8_t* h;        // [P][I] in HFMT
  const int32_t* ids;      // [M*kk] expert of pair m*kk+j
  const float* topk_w;     // [M*kk] routing weight of pair m*kk+j
  uint16_t* y;             // [M][H] bf16
  int H, I, kk;            // kk: pairs per token (top_k + shared experts)
  int kchunks;             // K chunks per pair's product (divides I / k-step)
  const float* w_scale;    // fp8: s_w2 per tensor, per expert (w_es) or per row ([E][H], w_cs)
  int w_cs = 0, w_es = 0;
  const float* h_scale;    // fp8 static: s_h
  const unsigned* h_amax;  // fp8 dynamic: max |h| (float bits)
  const float* x_scale;    // fp8: s_x in effect (reported)
  float* scales_out;       // optional fp32[2]: s_x, s_h in effect
  const float* wg_hmax = nullptr;  // fp8 dynamic, instead of h_amax: the gate/up workgroups' largest |h|
  int n_wg = 0;                    // entries of wg_hmax
};

// Unit u of the token: pair u / kchunks, K chunk u % kchunks of csteps
// k-steps.  Sets the lane's weight-row and h pointers and the pair.
template <bool FP8, int HFMT>
__device__ __forceinline__ void tok_unit(const DownTokArgs& a, const uint8_t* s_h8, int m, int n0, int u,
                                         int csteps, const uint8_t*& pa, const uint8_t*& pb, int& f, int& e) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;
  constexpr int LB = FP8 ? 32 : 16;
  constexpr int HSZ = HFMT == H_BF16 ? 2 : (HFMT == H_F32 ? 4 : 1);
  const int lane = threadIdx.x & 63, r16 = lane & 15, kq = lane >> 4;
  const int j = u / a.kchunks, c = u - j * a.kchunks;
  const int kbeg = c * csteps * KSTEP;
  f = m * a.kk + j;
  e = a.ids[f];
  pa = a.w2 + ((int64_t)e * a.H + n0 + r16) * a.I * ESZ + (int64_t)kbeg * ESZ + kq * LB;
  if constexpr (HFMT == H_F32)
    pb = s_h8 + j * a.I + kbeg + kq * LB;  // e4m3 in LDS
  else
    pb = a.h + ((int64_t)f * a.I + kbeg) * HSZ + kq * LB;
}

// The unit's sum for this lane's rows n0+4kq.., dequantised and weighted,
// added to ysum in place.
template <bool FP8>
__device__ __forceinline__ void tok_add(const DownTokArgs& a, f32x4& ysum, const f32x4& acc, int f, int e, int n0,
                                        float sh) {
  const int kq = (threadIdx.x & 63) >> 4;
  const float w = a.topk_w[f];
  float d[4] = {w, w, w, w};
  if constexpr (FP8) {
    if (a.w_cs) {
      const float* ws = a.w_scale + (int64_t)e * a.H + n0 + kq * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = w * (sh * ws[r]);
    } else {
      const float v = w * (sh * a.w_scale[(int64_t)e * a.w_es]);
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = v;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) ysum[r] += acc[r] * d[r];
}

// Grid: x = 16-row tiles of H, y = tokens.
template <bool FP8, int HFMT, int U>
static __global__ __launch_bounds__(256) void down_token_kernel(DownTokArgs a) {
  extern __shared__ __align__(16) uint8_t s_h8[];  // dynamic fp8 h: the token's [kk][I] e4m3 rows
  __shared__ f32x4 s_sum[4][4];                     // wave, row quad
  constexpr int KSTEP = FP8 ? 128 : 32;
  constexpr int SB = KSTEP * (FP8 ? 1 : 2);
  const int m = blockIdx.y, n0 = blockIdx.x * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float sh = 1.0f;
  if constexpr (HFMT == H_F32) {
    if (a.wg_hmax) {  // the largest of the gate/up workgroups' maxima
      __shared__ float s_m[4];
      float m = 0.0f;
      for (int i = threadIdx.x; i < a.n_wg; i += 256) m = fmaxf(m, a.wg_hmax[i]);
      m = wave_max(m);
      if (lane == 0) s_m[wave] = m;
      __syncthreads();
      sh = scale_from_amax(fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3])));
    } else {
      sh = scale_from_amax(__uint_as_float(*a.h_amax));
    }
  } else if constexpr (FP8) {
    sh = *a.h_scale;
  }
  if (FP8 && a.scales_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    a.scales_out[0] = *a.x_scale;
    a.scales_out[1] = sh;
  }
  if constexpr (HFMT == H_F32) {
    const float rh = 1.0f / sh;
    const int n = a.kk * a.I;  // a multiple of 128
    const float* src = (const float*)a.h + (int64_t)m * n;
    for (int i = threadIdx.x * 16; i < n; i += 256 * 16) {
      const f32x4 v0 = *(const f32x4*)(src + i), v1 = *(const f32x4*)(src + i + 4);
      const f32x4 v2 = *(const f32x4*)(src + i + 8), v3 = *(const f32x4*)(src + i + 12);
      *(u32x4*)(s_h8 + i) = u32x4{pack_e4m3x4(v0[0] * rh, v0[1] * rh, v0[2] * rh, v0[3] * rh),
                                  pack_e4m3x4(v1[0] * rh, v1[1] * rh, v1[2] * rh, v1[3] * rh),
                                  pack_e4m3x4(v2[0] * rh, v2[1] * rh, v2[2] * rh, v2[3] * rh),
                                  pack_e4m3x4(v3[0] * rh, v3[1] * rh, v3[2] * rh, v3[3] * rh)};
    }
    __syncthreads();
  }
  const int csteps = a.I / KSTEP / a.kchunks;
  const int units = a.kk * a.kchunks;
  f32x4 ysum = {0.f, 0.f, 0.f, 0.f};
  int u = wave;
  for (; u + 4 < units; u += 8) {  // units u and u + 4 together
    const uint8_t *pa[2], *pb[2];
    int f[2], e[2];
    tok_unit<FP8, HFMT>(a, s_h8, m, n0, u, csteps, pa[0], pb[0], f[0], e[0]);
    tok_unit<FP8, HFMT>(a, s_h8, m, n0, u + 4, csteps, pa[1], pb[1], f[1], e[1]);
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_k<FP8, 2, 2, U, SB>(pa, pb, csteps, acc);
    tok_add<FP8>(a, ysum, acc[0][0], f[0], e[0], n0, sh);
    tok_add<FP8>(a, ysum, acc[1][1], f[1], e[1], n0, sh);
  }
  if (u < units) {
    const uint8_t *pa[1], *pb[1];
    int f, e;
    tok_unit<FP8, HFMT>(a, s_h8, m, n0, u, csteps, pa[0], pb[0], f, e);
    f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
    stream_k<FP8, 1, 1, U, SB>(pa, pb, csteps, acc);
    tok_add<FP8>(a, ysum, acc[0][0], f, e, n0, sh);
  }
  if ((lane & 15) == 0) s_sum[wave][lane >> 4] = ysum;  // column 0: rows 4kq..4kq+3
  __syncthreads();
  if (threadIdx.x < 16) {
    const int q = threadIdx.x >> 2, r = threadIdx.x & 3;
    const float v = ((s_sum[0][q][r] + s_sum[1][q][r]) + s_sum[2][q][r]) + s_sum[3][q][r];
    const __bf16 b = (__bf16)v;
    a.y[(int64_t)m * a.H + n0 + threadIdx.x] = __builtin_bit_cast(unsigned short, b);
  }
}

// Stand-alone per-tensor e4m3 quantisation of fp32 data with a given scale.
static __global__ __launch_bounds__(256) void quant_f32_kernel(const float* __restrict__ in, int64_t n,
                                                        const float* __restrict__ scale, uint8_t* __restrict__ out) {
  const float r = 1.0f / *scale;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const f32x4 v = *(const f32x4*)(in + i);
    *(unsigned*)(out + i) = pack_e4m3x4(v[0] * r, v[1] * r, v[2] * r, v[3] * r);
  } else {
    for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)(pack_e4m3x4(in[j] * r, 0.f, 0.f, 0.f) & 0xffu);
  }
}

}  // namespace moe
