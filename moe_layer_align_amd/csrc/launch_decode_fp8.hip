// fp8 decode products with h in fp32 (dynamic h scale).  The e4m3-h
// variants (static scale) are in launch_decode_fp8_static.hip.
#include "launch_decode_impl.h"

namespace moe {

bool launch_gemm1_fp8_static(const DecodeShape& s, hipStream_t st, const Gemm1Args& a);
bool launch_gemm2_fp8_static(const DecodeShape& s, hipStream_t st, const Gemm2Args& a);

bool launch_gemm1_fp8(int hf, const DecodeShape& s, hipStream_t st, const Gemm1Args& a) {
  if (hf == H_F32) return decode_dispatch::gemm1<true, H_F32>(s, st, a);
  if (hf == H_E4M3) return launch_gemm1_fp8_static(s, st, a);
  return false;
}

bool launch_gemm2_fp8(int hf, const DecodeShape& s, hipStream_t st, const Gemm2Args& a) {
  if (hf == H_F32) return decode_dispatch::gemm2<true, H_F32>(s, st, a);
  if (hf == H_E4M3) return launch_gemm2_fp8_static(s, st, a);
  return false;
}

}  // namespace moe
