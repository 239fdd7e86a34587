// Prefill products (persistent tiled kernels, fp8 and bf16), h quantisation
// and the per-token combine of the prefill path.
#include <atomic>

#include "launch.h"

namespace moe {
namespace {

// The dynamic LDS ceiling of a prefill kernel is raised once per kernel and
// device (the current device, as for the launch that follows).
template <int MODE, bool HDYN, bool PC, bool BF = false>
bool prefill(int wgs, hipStream_t st, const PrefillArgs& g) {
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> lds_set[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev >= kMaxDevices || !lds_set[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute((const void*)prefill_gemm_kernel<MODE, HDYN, PC, BF>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kPfLds) != hipSuccess)
      return false;
    if (dev < kMaxDevices) lds_set[dev].store(true, std::memory_order_release);
  }
  prefill_gemm_kernel<MODE, HDYN, PC, BF><<<wgs, kPfThreads, kPfLds, st>>>(g);
  return true;
}

template <int MODE>
bool prefill_mode(bool bf, bool hdyn, bool pc, int wgs, hipStream_t st, const PrefillArgs& g) {
  if (bf) return !hdyn && !pc && prefill<MODE, false, false, true>(wgs, st, g);
  return pc ? (hdyn ? prefill<MODE, true, true>(wgs, st, g) : prefill<MODE, false, true>(wgs, st, g))
            : (hdyn ? prefill<MODE, true, false>(wgs, st, g) : prefill<MODE, false, false>(wgs, st, g));
}

}  // namespace

bool launch_prefill_gemm(int mode, bool bf, bool hdyn, bool pc, int wgs, hipStream_t st, const PrefillArgs& g) {
  return mode == 0 ? prefill_mode<0>(bf, hdyn, pc, wgs, st, g) : prefill_mode<1>(bf, hdyn, pc, wgs, st, g);
}

void launch_prefill_quant_h(const float* h, int64_t n, const unsigned* h_amax, uint8_t* hq, hipStream_t st) {
  prefill_quant_h_kernel<<<(unsigned)((n + 4095) / 4096), 256, 0, st>>>(h, n, h_amax, hq);
}

void launch_prefill_finalize(const uint16_t* part, const float* wts, uint16_t* y, int M, int H, int k,
                             const float* x_scale, const unsigned* h_amax, const float* h_scale, float* scales_out,
                             hipStream_t st) {
  prefill_finalize_kernel<<<(unsigned)(((int64_t)M * H + 2047) / 2048), 256, 0, st>>>(
      part, wts, y, M, H, k, x_scale, h_amax, h_scale, scales_out);
}

}  // namespace moe
