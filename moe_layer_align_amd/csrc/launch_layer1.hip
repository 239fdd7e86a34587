// The small layers of layer_small.h: the single-launch layer (the instance
// for the dtype, h format and down-product wave split) and the first launch of
// the two-launch layer.
#include <atomic>

#include "launch.h"
#include "layer_small.h"

namespace moe {
namespace {

// The grid barrier's counters: zeroed by the loader, back at zero after every
// completed launch (layer1_barrier).
__device__ unsigned l1_sync[kL1SyncWords];

// The device address of l1_sync on the current device, looked up once per
// device (the array's name is a host-side stand-in in host code).
unsigned* sync_words() {
  constexpr int kMaxDevices = 64;
  static std::atomic<unsigned*> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  unsigned* p = cached[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(l1_sync)) != hipSuccess) return nullptr;
    p = (unsigned*)addr;
    cached[dev].store(p, std::memory_order_release);
  }
  return p;
}

template <bool FP8, int HF>
const void* pick_wks(int wks) {
  switch (wks) {
    case 1: return (const void*)layer1_kernel<FP8, HF, 1>;
    case 2: return (const void*)layer1_kernel<FP8, HF, 2>;
    case 4: return (const void*)layer1_kernel<FP8, HF, 4>;
  }
  return nullptr;
}

}  // namespace

bool launch_tiny_gate_up(bool fp8, int hf, int grid, hipStream_t st, const Layer1Args& a) {
  const bool x4 = (int64_t)a.M * a.H > 2 * 256 * 16;  // fp8 x in four register chunks per thread, else two
  if (!fp8 && hf == H_BF16)
    tiny_gate_up_kernel<false, H_BF16, 2><<<grid, 256, 0, st>>>(a);
  else if (fp8 && hf == H_F32 && !x4)
    tiny_gate_up_kernel<true, H_F32, 2><<<grid, 256, 0, st>>>(a);
  else if (fp8 && hf == H_F32)
    tiny_gate_up_kernel<true, H_F32, 4><<<grid, 256, 0, st>>>(a);
  else if (fp8 && hf == H_E4M3 && !x4)
    tiny_gate_up_kernel<true, H_E4M3, 2><<<grid, 256, 0, st>>>(a);
  else if (fp8 && hf == H_E4M3)
    tiny_gate_up_kernel<true, H_E4M3, 4><<<grid, 256, 0, st>>>(a);
  else
    return false;
  return true;
}

hipError_t launch_layer1(bool fp8, int hf, int wks, int grid, size_t lds, hipStream_t st, const Layer1Args& a) {
  const void* fn = !fp8 ? (hf == H_BF16 ? pick_wks<false, H_BF16>(wks) : nullptr)
                        : hf == H_F32 ? pick_wks<true, H_F32>(wks)
                        : hf == H_E4M3 ? pick_wks<true, H_E4M3>(wks) : nullptr;
  if (!fn) return hipErrorInvalidValue;
  // every workgroup must be resident at once (the barrier waits for all):
  // at most as many per CU as the kernel's occupancy allows
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err;
  if ((err = hipGetDevice(&dev)) != hipSuccess) return err;
  if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return err;
  if ((err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds)) != hipSuccess) return err;
  if (per_cu < 1 || grid > per_cu * cus) return hipErrorInvalidConfiguration;
  Layer1Args copy = a;
  copy.sync = sync_words();
  if (!copy.sync) return hipErrorInvalidSymbol;
  void* params[] = {(void*)&copy};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), params, lds, st);
}

}  // namespace moe
