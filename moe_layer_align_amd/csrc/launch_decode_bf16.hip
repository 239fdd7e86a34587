// bf16 decode products (all variants).
#include "launch_decode_impl.h"

namespace moe {

bool launch_gemm1_bf16(const DecodeShape& s, hipStream_t st, const Gemm1Args& a) {
  return decode_dispatch::gemm1<false, H_BF16>(s, st, a);
}

bool launch_gemm2_bf16(const DecodeShape& s, hipStream_t st, const Gemm2Args& a) {
  return decode_dispatch::gemm2<false, H_BF16>(s, st, a);
}

}  // namespace moe
