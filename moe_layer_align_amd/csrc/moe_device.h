// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA
// wrappers, number-format conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr float kE4m3Max = 448.0f;

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16 -> fp32.  A: lane l holds row (l%16), 8 consecutive k at
// 8*(l/16); B: lane l holds column (l%16), the same 8 k.  C: lane l holds
// rows 4*(l/16)+0..3 of column (l%16).
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// 16x16x128 OCP e4m3 x e4m3 -> fp32 (format code 0 for both operands; block
// scales fixed at 2^0, E8M0 code 127).  Each lane supplies 32 bytes of A
// (row l%16) and 32 bytes of B (column l%16) covering the same k positions,
// so the product does not depend on how the hardware orders k inside a lane.
__device__ __forceinline__ f32x4 mfma_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x4 c) {
  i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same product with per-lane E8M0 block scales (2^(s-127)): sa applies to
// this lane's 32 bytes of A, sb to its 32 bytes of B (lanes holding the same
// row of A, or the same column of B, at the same k positions pass the same
// scale).
__device__ __forceinline__ f32x4 mfma_fp8_scaled(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x4 c, int sa, int sb) {
  i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (hardware conversion).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (unsigned)__builtin_bit_cast(unsigned short, x) | ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

__device__ __forceinline__ float sat_e4m3(float v) { return fminf(fmaxf(v, -kE4m3Max), kE4m3Max); }

// Four fp32 -> four OCP e4m3 bytes (byte i from v_i), nearest even, after
// clamping to +-448 so the conversion never sees an out-of-range value.
__device__ __forceinline__ unsigned pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), w, true);
  return (unsigned)w;
}

// Scale from an amax: amax/448, or 1 when amax is 0.
__device__ __forceinline__ float scale_from_amax(float amax) { return amax > 0.0f ? amax / kE4m3Max : 1.0f; }

// Block scaling (OCP MX rule for E4M3 elements): the E8M0 code of a block
// whose largest magnitude is amax, max(biased exponent of amax - 8, 0), and
// the reciprocal of its scale, 2^(127 - code), an exact power of two.
__device__ __forceinline__ int block_scale_code(float amax) {
  const int f = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return f > 8 ? f - 8 : 0;
}
__device__ __forceinline__ float block_scale_recip(int code) { return __uint_as_float((unsigned)(254 - code) << 23); }

// ---------------------------------------------------------------- reductions
// Wavefront reductions by DPP lane moves (gfx9 controls): two quad
// permutations, the half-row and row mirrors leave every lane of a 16-lane row
// with the row's result; the two row broadcasts fold rows 0+1 into row 1 and
// rows 0..3 into row 3, so lane 63 ends with the wave's result, which
// readlane makes uniform.  Each step is a VALU operation on the same lane
// (a few cycles), where a ds_bpermute shuffle costs an LDS round trip.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i of each 8-lane half-row <- lane 7-i
constexpr int kDppMirror = 0x140;     // lane i of each row <- lane 15-i
constexpr int kDppBcast15 = 0x142;    // rows 1 and 3 <- lane 15 of rows 0 and 2 (row mask 0xA)
constexpr int kDppBcast31 = 0x143;    // rows 2 and 3 <- lane 31 (row mask 0xC)

// Lanes outside ROWS keep their own value.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ unsigned dpp_u32(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v)));
}

__device__ __forceinline__ float lane63_f32(float v) {
  return __uint_as_float((unsigned)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

// Largest value over each aligned group of 8 lanes (two quad permutations
// and the half-row mirror), in all 8 of them.  All lanes must be active.
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  return fmaxf(v, dpp_f32<kDppHalfMirror>(v));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  v = fmaxf(v, dpp_f32<kDppBcast15, 0xA>(v));
  v = fmaxf(v, dpp_f32<kDppBcast31, 0xC>(v));
  return lane63_f32(v);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  v += dpp_f32<kDppBcast15, 0xA>(v);
  v += dpp_f32<kDppBcast31, 0xC>(v);
  return lane63_f32(v);
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ unsigned long long max_dpp_u64(unsigned long long k) {
  const unsigned lo = dpp_u32<CTRL, ROWS>((unsigned)k), hi = dpp_u32<CTRL, ROWS>((unsigned)(k >> 32));
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  return o > k ? o : k;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k) {
  k = max_dpp_u64<kDppXor1>(k);
  k = max_dpp_u64<kDppXor2>(k);
  k = max_dpp_u64<kDppHalfMirror>(k);
  k = max_dpp_u64<kDppMirror>(k);
  k = max_dpp_u64<kDppBcast15, 0xA>(k);
  k = max_dpp_u64<kDppBcast31, 0xC>(k);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)k, 63);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(k >> 32), 63);
  return ((unsigned long long)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP: row shifts by
// 1, 2, 4 and 8 (lanes without a source add 0) scan each 16-lane row, then
// the two row broadcasts carry the totals of rows 0, 0+1 and 2 forward.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, kDppBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppBcast31, 0xC, 0xF, false);
  return v;
}

__device__ __forceinline__ unsigned long long lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
