// Host launchers of the expert products, one translation unit per family of
// kernel instantiations (so that the library's kernels compile in parallel):
//   launch_decode_bf16.hip, launch_decode_fp8.hip  decode products
//   launch_down_token.hip                           down product + combine per token
//   launch_prefill.hip                              prefill products
// Each launcher picks the template instance for the run-time variant and
// enqueues it on the stream; it returns false when the variant is not built.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_decode.h"
#include "gemm_prefill.h"

namespace moe {

// Launch shape of the two decode products (see make_plan in moe_api.hip).
struct DecodeShape {
  int nt, u;  // 16-token tiles per pass; MFMA k-steps per pipeline stage
  int ks;     // gate/up: waves splitting K; down: waves splitting a K slice
  int tw;     // > 0: long-stream variant with tw tiles per wave
  dim3 grid;  // grid of the chosen variant
  size_t lds; // dynamic LDS (down product, dynamic fp8 h scale)
  int ft = 1; // K-split variants: groups per wave (1 or 2) of 16 features (gate/up) or 32 rows (down)
};

bool launch_gemm1_bf16(const DecodeShape& s, hipStream_t st, const Gemm1Args& a);
bool launch_gemm2_bf16(const DecodeShape& s, hipStream_t st, const Gemm2Args& a);
// hf: H_F32 (dynamic h scale) or H_E4M3 (static)
bool launch_gemm1_fp8(int hf, const DecodeShape& s, hipStream_t st, const Gemm1Args& a);
bool launch_gemm2_fp8(int hf, const DecodeShape& s, hipStream_t st, const Gemm2Args& a);

// Down product with the weighted combine per token (small layers):
// hf H_BF16 (bf16 layers), H_F32 or H_E4M3 (fp8); u: k-steps per pipeline
// stage; lds: the staged e4m3 h rows of a token (dynamic fp8 h scale).
bool launch_down_token(bool fp8, int hf, int u, dim3 grid, size_t lds, hipStream_t st, const DownTokArgs& a);

// Persistent prefill product: mode 0 gate/up, 1 down; bf: bf16 layer (no
// scales); hdyn: dynamic fp8 h scale; pc: one weight scale per row.  The
// kernel's dynamic LDS ceiling is raised once per kernel and device; false
// when that fails.
bool launch_prefill_gemm(int mode, bool bf, bool hdyn, bool pc, int wgs, hipStream_t st, const PrefillArgs& g);
void launch_prefill_quant_h(const float* h, int64_t n, const unsigned* h_amax, uint8_t* hq, hipStream_t st);
void launch_prefill_finalize(const uint16_t* part, const float* wts, uint16_t* y, int M, int H, int k,
                             const float* x_scale, const unsigned* h_amax, const float* h_scale, float* scales_out,
                             hipStream_t st);

// The single-launch layer for tiny token counts (layer_small.h): a launch of
// `grid` workgroups, refused (hipErrorInvalidConfiguration) when they could
// not all be resident at once; otherwise the launch's own status.
struct Layer1Args;
hipError_t launch_layer1(bool fp8, int hf, int wks, int grid, size_t lds, hipStream_t st, const Layer1Args& a);
// The first launch of the two-launch layer for tiny token counts (routing,
// quantisation, sort-and-pad and the gate/up product); false when the
// dtype / h format is not built.
bool launch_tiny_gate_up(bool fp8, int hf, int grid, hipStream_t st, const Layer1Args& a);

}  // namespace moe
