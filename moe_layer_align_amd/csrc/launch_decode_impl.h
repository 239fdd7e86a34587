// Template dispatch of the decode products: run-time variant -> template
// instance.  Included by launch_decode_bf16.hip and launch_decode_fp8.hip
// only, each instantiating the kernels of one dtype.
#pragma once

#include "launch.h"

namespace moe {
namespace decode_dispatch {

template <bool FP8, int HF, int NT, int U, int KS, int FT>
void g1(dim3 g, hipStream_t st, const Gemm1Args& a) {
  gemm1_decode_kernel<FP8, HF, NT, U, KS, FT><<<g, 256, 0, st>>>(a);
}

template <bool FP8, int HF, int NT, int U, int FT>
bool g1_ks(int ks, dim3 g, hipStream_t st, const Gemm1Args& a) {
  switch (ks) {
    case 1: g1<FP8, HF, NT, U, 1, FT>(g, st, a); return true;
    case 2: g1<FP8, HF, NT, U, 2, FT>(g, st, a); return true;
    case 4: g1<FP8, HF, NT, U, 4, FT>(g, st, a); return true;
  }
  return false;
}

template <bool FP8, int HF, int NT, int U>
bool g1_ft(int ft, int ks, dim3 g, hipStream_t st, const Gemm1Args& a) {
  if (ft == 1) return g1_ks<FP8, HF, NT, U, 1>(ks, g, st, a);
  if (ft == 2) return g1_ks<FP8, HF, NT, U, 2>(ks, g, st, a);
  return false;
}

// the two unrolls of a dtype: U0 and 2*U0 (bf16 2 and 4, fp8 1 and 2)
template <bool FP8>
constexpr int kU0 = FP8 ? 1 : 2;

template <bool FP8, int HF, int NT>
bool g1_u(int u, int ft, int ks, dim3 g, hipStream_t st, const Gemm1Args& a) {
  if (u == kU0<FP8>) return g1_ft<FP8, HF, NT, kU0<FP8>>(ft, ks, g, st, a);
  if (u == 2 * kU0<FP8>) return g1_ft<FP8, HF, NT, 2 * kU0<FP8>>(ft, ks, g, st, a);
  return false;
}

template <bool FP8, int HF, int NT>
bool g1s_u(int u, int tw, dim3 g, hipStream_t st, const Gemm1Args& a) {
  if (u == kU0<FP8>)
    gemm1_stream_kernel<FP8, HF, NT, kU0<FP8>><<<g, 256, 0, st>>>(a, tw);
  else if (u == 2 * kU0<FP8>)
    gemm1_stream_kernel<FP8, HF, NT, 2 * kU0<FP8>><<<g, 256, 0, st>>>(a, tw);
  else
    return false;
  return true;
}

template <bool FP8, int HF, int NT>
bool g2s_u(int u, int tw, dim3 g, size_t lds, hipStream_t st, const Gemm2Args& a) {
  if (u == kU0<FP8>)
    gemm2_stream_kernel<FP8, HF, NT, kU0<FP8>><<<g, 256, lds, st>>>(a, tw);
  else if (u == 2 * kU0<FP8>)
    gemm2_stream_kernel<FP8, HF, NT, 2 * kU0<FP8>><<<g, 256, lds, st>>>(a, tw);
  else
    return false;
  return true;
}

template <bool FP8, int HF, int NT, int U, int WKS, int FR>
void g2(dim3 g, size_t lds, hipStream_t st, const Gemm2Args& a) {
  gemm2_decode_kernel<FP8, HF, NT, U, WKS, FR><<<g, 256, lds, st>>>(a);
}

template <bool FP8, int HF, int NT, int U, int FR>
bool g2_wks(int wks, dim3 g, size_t lds, hipStream_t st, const Gemm2Args& a) {
  switch (wks) {
    case 1: g2<FP8, HF, NT, U, 1, FR>(g, lds, st, a); return true;
    case 2: g2<FP8, HF, NT, U, 2, FR>(g, lds, st, a); return true;
    case 4: g2<FP8, HF, NT, U, 4, FR>(g, lds, st, a); return true;
  }
  return false;
}

template <bool FP8, int HF, int NT, int U>
bool g2_fr(int fr, int wks, dim3 g, size_t lds, hipStream_t st, const Gemm2Args& a) {
  if (fr == 1) return g2_wks<FP8, HF, NT, U, 1>(wks, g, lds, st, a);
  if (fr == 2) return g2_wks<FP8, HF, NT, U, 2>(wks, g, lds, st, a);
  return false;
}

template <bool FP8, int HF, int NT>
bool g2_u(int u, int fr, int wks, dim3 g, size_t lds, hipStream_t st, const Gemm2Args& a) {
  if (u == kU0<FP8>) return g2_fr<FP8, HF, NT, kU0<FP8>>(fr, wks, g, lds, st, a);
  if (u == 2 * kU0<FP8>) return g2_fr<FP8, HF, NT, 2 * kU0<FP8>>(fr, wks, g, lds, st, a);
  return false;
}

// token tiles per pass: 1, 2 or 4 (the plan maps 3 to 4)
template <bool FP8, int HF>
bool gemm1(const DecodeShape& s, hipStream_t st, const Gemm1Args& a) {
  if (s.tw > 0) {
    switch (s.nt) {
      case 1: return g1s_u<FP8, HF, 1>(s.u, s.tw, s.grid, st, a);
      case 2: return g1s_u<FP8, HF, 2>(s.u, s.tw, s.grid, st, a);
      case 4: return g1s_u<FP8, HF, 4>(s.u, s.tw, s.grid, st, a);
    }
    return false;
  }
  switch (s.nt) {
    case 1: return g1_u<FP8, HF, 1>(s.u, s.ft, s.ks, s.grid, st, a);
    case 2: return g1_u<FP8, HF, 2>(s.u, s.ft, s.ks, s.grid, st, a);
    case 4: return g1_u<FP8, HF, 4>(s.u, s.ft, s.ks, s.grid, st, a);
  }
  return false;
}

template <bool FP8, int HF>
bool gemm2(const DecodeShape& s, hipStream_t st, const Gemm2Args& a) {
  if (s.tw > 0) {
    switch (s.nt) {
      case 1: return g2s_u<FP8, HF, 1>(s.u, s.tw, s.grid, s.lds, st, a);
      case 2: return g2s_u<FP8, HF, 2>(s.u, s.tw, s.grid, s.lds, st, a);
      case 4: return g2s_u<FP8, HF, 4>(s.u, s.tw, s.grid, s.lds, st, a);
    }
    return false;
  }
  switch (s.nt) {
    case 1: return g2_u<FP8, HF, 1>(s.u, s.ft, s.ks, s.grid, s.lds, st, a);
    case 2: return g2_u<FP8, HF, 2>(s.u, s.ft, s.ks, s.grid, s.lds, st, a);
    case 4: return g2_u<FP8, HF, 4>(s.u, s.ft, s.ks, s.grid, s.lds, st, a);
  }
  return false;
}

}  // namespace decode_dispatch
}  // namespace moe
