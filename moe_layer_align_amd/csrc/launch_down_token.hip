// The down product with the weighted top-k combine per token (small layers).
#include "launch.h"

namespace moe {
namespace {

template <bool FP8, int HF>
bool tok(int u, dim3 g, size_t lds, hipStream_t st, const DownTokArgs& a) {
  constexpr int U0 = FP8 ? 1 : 2;
  if (u == U0)
    down_token_kernel<FP8, HF, U0><<<g, 256, lds, st>>>(a);
  else if (u == 2 * U0)
    down_token_kernel<FP8, HF, 2 * U0><<<g, 256, lds, st>>>(a);
  else
    return false;
  return true;
}

}  // namespace

bool launch_down_token(bool fp8, int hf, int u, dim3 g, size_t lds, hipStream_t st, const DownTokArgs& a) {
  if (!fp8) return hf == H_BF16 && tok<false, H_BF16>(u, g, lds, st, a);
  if (hf == H_F32) return tok<true, H_F32>(u, g, lds, st, a);
  if (hf == H_E4M3) return tok<true, H_E4M3>(u, g, lds, st, a);
  return false;
}

}  // namespace moe
