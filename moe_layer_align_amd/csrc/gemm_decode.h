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

#include "moe_device.h"

namespace moe {

enum HFormat { H_BF16 = 0, H_F32 = 1, H_E4M3 = 2 };

struct Segments {
  const int32_t* sorted_ids;
  const int32_t* offsets;
  const int32_t* counts;
  const int32_t* active;
  const int32_t* num_active;
};

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
// Gate/up product with the SiLU(gate)*up epilogue.
//
// Wave tile: 16 output features i0..i0+15, i.e. gate rows i0.. and up rows
// I+i0.. of W13[e] (two 16-row MFMA tiles whose accumulators land in the same
// lanes, so the epilogue pairs gate and up without data exchange), times NT
// 16-token tiles.  KSPLIT waves of the workgroup split K = H and are summed
// through LDS; 4/KSPLIT feature tiles per workgroup.
// --------------------------------------------------------------------------
struct Gemm1Args {
  const uint8_t* w13;        // [E][2I][H]
  const uint8_t* act;        // bf16 x [M][H] or e4m3 xq [M][H]
  Segments seg;
  int H, I, top_k;
  const float* w_scale;      // fp8: s_w13
  const float* x_scale;      // fp8: s_x in effect
  const float* h_scale;      // fp8 static h: s_h
  uint8_t* h;                // [P][I] in HFMT
  unsigned* h_amax;          // fp8 dynamic: running max of |h| (float bits)
};

template <bool FP8, int HFMT, int NT, int U, int KSPLIT>
__global__ __launch_bounds__(256) void gemm1_decode_kernel(Gemm1Args a) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;   // k per MFMA
  constexpr int LB = FP8 ? 32 : 16;       // bytes per lane per operand per step
  constexpr int SB = KSTEP * ESZ;         // bytes per row per step
  constexpr int TPW = 4 / KSPLIT;         // feature tiles per workgroup
  __shared__ f32x4 s_red[KSPLIT > 1 ? (KSPLIT - 1) * TPW * 2 * NT * 64 : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kpart = wave % KSPLIT, tile = wave / KSPLIT;
  const int s = blockIdx.y;
  if (s >= *a.seg.num_active) return;
  const int e = a.seg.active[s];
  const int seg = a.seg.offsets[e], cnt = a.seg.counts[e];
  const int pass0 = blockIdx.z * NT * 16;
  if (pass0 >= cnt) return;

  const int r16 = lane & 15, kq = lane >> 4;
  const int i0 = (blockIdx.x * TPW + tile) * 16;
  const int Kw = a.H / KSPLIT;
  const int kbeg = kpart * Kw;
  const int nsteps = Kw / KSTEP;

  const int64_t rowb = (int64_t)a.H * ESZ;
  const uint8_t* pg = a.w13 + ((int64_t)e * 2 * a.I + i0 + r16) * rowb + (int64_t)kbeg * ESZ + kq * LB;
  const uint8_t* pu = pg + (int64_t)a.I * rowb;
  const uint8_t* pb[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int slot = min(pass0 + t * 16 + r16, cnt - 1);
    const int m = a.seg.sorted_ids[seg + slot] / a.top_k;
    pb[t] = a.act + (int64_t)m * rowb + (int64_t)kbeg * ESZ + kq * LB;
  }

  f32x4 accg[NT], accu[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    accg[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  struct Stage {
    Frag<FP8> g[U], u[U], b[U][NT];
  };
  auto load_stage = [&](Stage& st, int step0) {
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int64_t off = (int64_t)(step0 + q) * SB;
      load_frag<FP8>(st.g[q], pg + off);
      load_frag<FP8>(st.u[q], pu + off);
#pragma unroll
      for (int t = 0; t < NT; ++t) load_frag<FP8>(st.b[q][t], pb[t] + off);
    }
  };
  auto compute_stage = [&](const Stage& st) {
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        accg[t] = mma<FP8>(st.g[q], st.b[q][t], accg[t]);
        accu[t] = mma<FP8>(st.u[q], st.b[q][t], accu[t]);
      }
  };

  const int nfull = nsteps / U;
  if (nfull > 0) {
    Stage s0, s1;
    load_stage(s0, 0);
    for (int it = 0; it < nfull; it += 2) {
      if (it + 1 < nfull) load_stage(s1, (it + 1) * U);
      compute_stage(s0);
      if (it + 1 < nfull) {
        if (it + 2 < nfull) load_stage(s0, (it + 2) * U);
        compute_stage(s1);
      }
    }
  }
  for (int st = nfull * U; st < nsteps; ++st) {
    Frag<FP8> g, u, b[NT];
    load_frag<FP8>(g, pg + (int64_t)st * SB);
    load_frag<FP8>(u, pu + (int64_t)st * SB);
#pragma unroll
    for (int t = 0; t < NT; ++t) load_frag<FP8>(b[t], pb[t] + (int64_t)st * SB);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      accg[t] = mma<FP8>(g, b[t], accg[t]);
      accu[t] = mma<FP8>(u, b[t], accu[t]);
    }
  }

  if constexpr (KSPLIT > 1) {
    if (kpart > 0) {
      f32x4* dst = s_red + (((kpart - 1) * TPW + tile) * 2 * NT) * 64 + lane;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        dst[(2 * t) * 64] = accg[t];
        dst[(2 * t + 1) * 64] = accu[t];
      }
    }
    __syncthreads();
    if (kpart > 0) return;
#pragma unroll
    for (int p = 0; p < KSPLIT - 1; ++p) {
      const f32x4* src = s_red + ((p * TPW + tile) * 2 * NT) * 64 + lane;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        accg[t] += src[(2 * t) * 64];
        accu[t] += src[(2 * t + 1) * 64];
      }
    }
  }

  const float deq = FP8 ? (*a.x_scale) * (*a.w_scale) : 1.0f;
  float rh = 1.0f;
  if constexpr (HFMT == H_E4M3) rh = 1.0f / *a.h_scale;
  float hmax = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int slot = pass0 + t * 16 + r16;
    if (slot < cnt) {
      const int f = a.seg.sorted_ids[seg + slot];
      float hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = accg[t][r] * deq;
        const float u = accu[t][r] * deq;
        hv[r] = g / (1.0f + expf(-g)) * u;
        hmax = fmaxf(hmax, fabsf(hv[r]));
      }
      const int64_t idx = (int64_t)f * a.I + i0 + kq * 4;
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
  if constexpr (HFMT == H_F32) {
    hmax = wave_max(hmax);
    if (lane == 0) atomicMax(a.h_amax, __float_as_uint(hmax));
  }
}

// --------------------------------------------------------------------------
// Down product with the routing-weighted scatter-add combine.
//
// Wave tile: 32 output rows (two 16-row MFMA tiles of W2[e]) over one K slice
// of I, times NT 16-token tiles.  Every wave adds w[pair] * (partial product)
// into the fp32 accumulator y_acc[m] with hardware float atomics, so K slices
// need no other reduction and the top-k combine is part of the epilogue.
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
  const float* w_scale;      // fp8: s_w2
  const float* h_scale;      // fp8 static: s_h
  const unsigned* h_amax;    // fp8 dynamic: max |h| (float bits)
  float* y_acc;              // [M][H]
};

// LDS row stride (bytes) of the quantised token slice: Kw plus 16 bytes so
// that the 16 token rows read by one instruction fall in different banks.
__host__ __device__ constexpr int gemm2_lds_stride(int kw_bytes) { return kw_bytes + 16; }

template <bool FP8, int HFMT, int NT, int U>
__global__ __launch_bounds__(256) void gemm2_decode_kernel(Gemm2Args a) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;
  constexpr int LB = FP8 ? 32 : 16;
  constexpr int SB = KSTEP * ESZ;
  constexpr int HSZ = HFMT == H_BF16 ? 2 : (HFMT == H_F32 ? 4 : 1);
  constexpr bool QH = FP8 && HFMT == H_F32;  // token operand staged in LDS
  extern __shared__ __align__(16) uint8_t s_tok[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.y;
  if (s >= *a.seg.num_active) return;
  const int e = a.seg.active[s];
  const int seg = a.seg.offsets[e], cnt = a.seg.counts[e];
  const int kslice = blockIdx.z % a.ksplit;
  const int pass0 = (blockIdx.z / a.ksplit) * NT * 16;
  if (pass0 >= cnt) return;

  const int r16 = lane & 15, kq = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * 32;
  const int Kw = a.I / a.ksplit;
  const int kbeg = kslice * Kw;
  const int nsteps = Kw / KSTEP;

  float deq = 1.0f;
  if constexpr (FP8) {
    const float sh = (HFMT == H_F32) ? scale_from_amax(__uint_as_float(*a.h_amax)) : *a.h_scale;
    deq = sh * (*a.w_scale);
    if constexpr (QH) {
      // quantise the workgroup's token slice into LDS: NT*16 rows of Kw bytes
      const float rh = 1.0f / sh;
      const int stride = gemm2_lds_stride(Kw);
      const int per_row = Kw / 16;  // 16 elements per thread-step
      for (int idx = threadIdx.x; idx < NT * 16 * per_row; idx += 256) {
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
      __syncthreads();
    }
  }

  const int64_t rowb = (int64_t)a.I * ESZ;
  const uint8_t* pa0 = a.w2 + ((int64_t)e * a.H + n0 + r16) * rowb + (int64_t)kbeg * ESZ + kq * LB;
  const uint8_t* pa1 = pa0 + 16 * rowb;
  const uint8_t* pb[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if constexpr (QH) {
      pb[t] = s_tok + (t * 16 + r16) * gemm2_lds_stride(Kw) + kq * LB;
    } else {
      const int slot = min(pass0 + t * 16 + r16, cnt - 1);
      const int f = a.seg.sorted_ids[seg + slot];
      pb[t] = a.h + ((int64_t)f * a.I + kbeg) * HSZ + kq * LB;
    }
  }

  f32x4 acc0[NT], acc1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    acc0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  struct Stage {
    Frag<FP8> w0[U], w1[U], b[U][NT];
  };
  auto load_stage = [&](Stage& st, int step0) {
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int64_t off = (int64_t)(step0 + q) * SB;
      load_frag<FP8>(st.w0[q], pa0 + off);
      load_frag<FP8>(st.w1[q], pa1 + off);
#pragma unroll
      for (int t = 0; t < NT; ++t) load_frag<FP8>(st.b[q][t], pb[t] + off);
    }
  };
  auto compute_stage = [&](const Stage& st) {
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc0[t] = mma<FP8>(st.w0[q], st.b[q][t], acc0[t]);
        acc1[t] = mma<FP8>(st.w1[q], st.b[q][t], acc1[t]);
      }
  };

  const int nfull = nsteps / U;
  if (nfull > 0) {
    Stage s0, s1;
    load_stage(s0, 0);
    for (int it = 0; it < nfull; it += 2) {
      if (it + 1 < nfull) load_stage(s1, (it + 1) * U);
      compute_stage(s0);
      if (it + 1 < nfull) {
        if (it + 2 < nfull) load_stage(s0, (it + 2) * U);
        compute_stage(s1);
      }
    }
  }
  for (int st = nfull * U; st < nsteps; ++st) {
    Frag<FP8> w0, w1, b[NT];
    load_frag<FP8>(w0, pa0 + (int64_t)st * SB);
    load_frag<FP8>(w1, pa1 + (int64_t)st * SB);
#pragma unroll
    for (int t = 0; t < NT; ++t) load_frag<FP8>(b[t], pb[t] + (int64_t)st * SB);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc0[t] = mma<FP8>(w0, b[t], acc0[t]);
      acc1[t] = mma<FP8>(w1, b[t], acc1[t]);
    }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int slot = pass0 + t * 16 + r16;
    if (slot < cnt) {
      const int f = a.seg.sorted_ids[seg + slot];
      const int m = f / a.top_k;
      const float w = a.topk_w[f] * deq;
      float* yr = a.y_acc + (int64_t)m * a.H + n0 + kq * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        unsafeAtomicAdd(yr + r, acc0[t][r] * w);
        unsafeAtomicAdd(yr + 16 + r, acc1[t][r] * w);
      }
    }
  }
}

// y = bf16(y_acc), 8 elements per thread; also reports the scales in effect.
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ y_acc, uint16_t* __restrict__ y,
                                                       int64_t n, const float* x_scale, const unsigned* h_amax,
                                                       const float* h_scale, float* scales_out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (scales_out && blockIdx.x == 0 && threadIdx.x == 0) {
    scales_out[0] = *x_scale;
    scales_out[1] = h_scale ? *h_scale : scale_from_amax(__uint_as_float(*h_amax));
  }
  if (i >= n) return;
  const f32x4 a = *(const f32x4*)(y_acc + i);
  const f32x4 b = *(const f32x4*)(y_acc + i + 4);
  u32x4 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
  *(u32x4*)(y + i) = o;
}

// Stand-alone per-tensor e4m3 quantisation of fp32 data with a given scale.
__global__ __launch_bounds__(256) void quant_f32_kernel(const float* __restrict__ in, int64_t n,
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
