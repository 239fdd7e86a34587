// Measurement probes for MI355X (gfx950), built as their own library
// (libmoe_probes.so) beside the layer's: what the chip delivers, as opposed to
// its nameplate figures, for the two resources the layer is bound by, and the
// summation precision of the fp8 matrix instructions that the fp8 layer's
// tolerance rests on.  Declarations and argument meaning: include/moe_probes.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probes.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

// Streaming read: every thread loads 16-byte words, kReadUnroll loads in
// flight per round, grid-stride over the buffer, and folds them by XOR into
// one word per workgroup (so no load is dead).  n16: 16-byte words.
__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_x[kReadThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kReadThreads / 64; ++w) r ^= s_x[w];
    sink[blockIdx.x] = r;
  }
}

// fp8 matrix-core issue rate: every wave runs `iters` rounds of four
// independent 32x32x64 e4m3 MFMAs (the prefill tile's instruction) on
// register operands with unit scales, and lane 0 of each wave stores its four
// accumulators' first elements.  Operands: 1.0 everywhere (code 0x38, so each
// round adds 64 to every accumulator element), or, with `random_ops`, bytes
// of a per-lane integer hash with the lowest mantissa bit cleared (never the
// NaN codes 0x7F / 0xFF), whose switching draws power the way real weights and
// activations do; the hardware then holds a lower clock.
__device__ __forceinline__ unsigned probe_hash(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_fp8_loop_kernel(float* __restrict__ out, int iters, int random_ops) {
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned seed = (threadIdx.x * 16u + (unsigned)i) * 2u;
    a[i] = random_ops ? (int)(probe_hash(seed) & 0xFEFEFEFEu) : 0x38383838;
    b[i] = random_ops ? (int)(probe_hash(seed + 1u) & 0xFEFEFEFEu) : 0x38383838;
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
  }
  if ((threadIdx.x & 63) == 0) {
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    out[w * 4 + 0] = c0[0];
    out[w * 4 + 1] = c1[0];
    out[w * 4 + 2] = c2[0];
    out[w * 4 + 3] = c3[0];
  }
}

// One wave: C[16][16] = sum over 128 k of A[r][k] * B[c][k] (e4m3 codes,
// A and B row-major [16][128]) times 2^(sa-127) * 2^(sb-127), plus c0, with
// one 16x16x128 scaled instruction.  Lane l supplies row/column l%16 at
// k = 32*(l/16)..+31; its accumulator holds rows 4*(l/16)+0..3 of column
// l%16.  The two forms are separate kernels on purpose: in one kernel with a
// branch per form, the compiler sized the wait before the shared store block
// for the shorter instruction only, and the store read a stale accumulator.
__global__ __launch_bounds__(64) void fp8_dot128_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                        float* __restrict__ C, int sa, int sb, float c0) {
  const int l = threadIdx.x;
  f32x4 c = {c0, c0, c0, c0};
  const u32x4* pa = (const u32x4*)(A + (l % 16) * 128 + 32 * (l / 16));
  const u32x4* pb = (const u32x4*)(B + (l % 16) * 128 + 32 * (l / 16));
  const u32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(4 * (l / 16) + r) * 16 + (l % 16)] = c[r];
}

// The same product as four 16x16x32 e4m3 MFMAs accumulating in k order
// (unit scales); lane l supplies k = 8*(l/16)..+7 of each 32-wide step.
__global__ __launch_bounds__(64) void fp8_dot32_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                       float* __restrict__ C, float c0) {
  const int l = threadIdx.x;
  f32x4 c = {c0, c0, c0, c0};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const long a = *(const long*)(A + (l % 16) * 128 + 32 * q + 8 * (l / 16));
    const long b = *(const long*)(B + (l % 16) * 128 + 32 * q + 8 * (l / 16));
    c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(4 * (l / 16) + r) * 16 + (l % 16)] = c[r];
}

// Publishing partial results to other XCDs inside one kernel: every
// workgroup writes its 32 KB slice of buf (8192 floats, value blockIdx.x + i)
// and then counts itself in at cnt[blockIdx.x % 1024], as a last-arriver
// combine would; mode 0: plain stores (no publication: only this kernel's end
// makes them visible to other XCDs), 1: plain stores and an agent-scope
// release fence (an L2 writeback) before the count, 2: write-through stores
// (agent-scope atomic stores) completed before the count.
template <int MODE>
__global__ __launch_bounds__(256) void publish_kernel(float* __restrict__ buf, unsigned* __restrict__ cnt) {
  float* p = buf + (int64_t)blockIdx.x * 8192;
  const float v = (float)blockIdx.x;
  for (int i = threadIdx.x; i < 2048; i += 256) {
    const f32x4 x = {v + 4 * i, v + 4 * i + 1, v + 4 * i + 2, v + 4 * i + 3};
    if constexpr (MODE == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) __hip_atomic_store(p + 4 * i + q, x[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *(f32x4*)(p + 4 * i) = x;
    }
  }
  if constexpr (MODE == 2) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores are performed
  __syncthreads();
  if (threadIdx.x == 0) {
    if constexpr (MODE == 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(cnt + (blockIdx.x & 1023), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

moe_status_t launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

}  // namespace

extern "C" {

int32_t moe_probes_abi_version(void) { return 3; }

moe_status_t moe_probe_hbm_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || grid < 1 || grid > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)buf % 16) != 0) return MOE_ERR_INVALID_ARG;
  hbm_read_kernel<<<grid, kReadThreads, 0, (hipStream_t)stream>>>((const u32x4*)buf, (int64_t)(bytes / 16), sink);
  return launch_status();
}

moe_status_t moe_probe_mfma_fp8_loop(float* out, int32_t grid, int32_t iters, int32_t random_operands,
                                     void* stream) {
  if (!out || grid < 1 || grid > (1 << 20) || iters < 1 || iters > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (random_operands != 0 && random_operands != 1) return MOE_ERR_INVALID_ARG;
  mfma_fp8_loop_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(out, iters, random_operands);
  return launch_status();
}

moe_status_t moe_probe_fp8_dot(const uint8_t* A, const uint8_t* B, float* C, int32_t sa, int32_t sb, float c0,
                               int32_t form, void* stream) {
  if (!A || !B || !C || sa < 0 || sa > 254 || sb < 0 || sb > 254 || (form != 0 && form != 1)) return MOE_ERR_INVALID_ARG;
  if (form == 1 && (sa != 127 || sb != 127)) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)A % 16) != 0 || ((uintptr_t)B % 16) != 0) return MOE_ERR_INVALID_ARG;
  if (form == 0)
    fp8_dot128_kernel<<<1, 64, 0, (hipStream_t)stream>>>(A, B, C, sa, sb, c0);
  else
    fp8_dot32_kernel<<<1, 64, 0, (hipStream_t)stream>>>(A, B, C, c0);
  return launch_status();
}

moe_status_t moe_probe_publish(float* buf, uint32_t* cnt, int32_t grid, int32_t mode, void* stream) {
  if (!buf || !cnt || grid < 1 || grid > (1 << 20) || mode < 0 || mode > 2) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)buf % 16) != 0 || ((uintptr_t)cnt % 4) != 0) return MOE_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (mode == 0) publish_kernel<0><<<grid, 256, 0, st>>>(buf, cnt);
  if (mode == 1) publish_kernel<1><<<grid, 256, 0, st>>>(buf, cnt);
  if (mode == 2) publish_kernel<2><<<grid, 256, 0, st>>>(buf, cnt);
  return launch_status();
}

}  // extern "C"
