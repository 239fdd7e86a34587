// fp8 decode products with h stored as e4m3 (static h scale).
#include "launch_decode_impl.h"

namespace moe {

bool launch_gemm1_fp8_static(const DecodeShape& s, hipStream_t st, const Gemm1Args& a) {
  return decode_dispatch::gemm1<true, H_E4M3>(s, st, a);
}

bool launch_gemm2_fp8_static(const DecodeShape& s, hipStream_t st, const Gemm2Args& a) {
  return decode_dispatch::gemm2<true, H_E4M3>(s, st, a);
}

}  // namespace moe
