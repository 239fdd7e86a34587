// Measurement probes for MI355X (gfx950), built as their own library
// (libmoe_probes.so) beside the layer's: what the chip delivers, as opposed to
// its nameplate figures, for the two resources the layer is bound by, and the
// summation precision of the fp8 matrix instructions that the fp8 layer's
// tolerance rests on.  Declarations and argument meaning: include/moe_probes.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// The operand stream of the tiled prefill product without its arithmetic:
// every workgroup walks `steps` K-steps of 128 bytes over 384 rows (256
// weight rows and 128 token rows of a 4096-byte-row matrix, a new tile of
// rows every 32 steps), each step's 48 KB landing in a three-slot LDS ring
// two steps ahead of its use, one barrier per step.  MODE 0: direct-to-LDS
// buffer loads (1 KB per instruction, eight whole rows' lines); MODE 1: the
// same loads into registers, written to the ring with 16-byte LDS stores;
// MODE 2: MODE 0 plus the LDS fragment reads of the product (each wave reads
// 24 KB of every step).  Rows wrap within the buffer (nrows = bytes / 4096),
// so a small buffer stays in L2 and a large one streams from HBM.  Every
// load goes through a buffer resource of `bytes` records.
constexpr int kRingRow = 4096, kRingBK = 128, kRingStage = 384 * kRingBK, kRingStages = 3;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

template <int N>
__device__ __forceinline__ void ring_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

// this lane's 12 rows of step s: 8 of the weight block (rows 64w + 8q +
// lane/8) and 4 of the token block (256 + 32w + 8q + lane/8), 16 bytes each;
// a new tile of 384 rows every 32 steps, wrapping within nrows
// (flags: 1 = each workgroup starts its tiles at K-step blockIdx.x % 32,
// 2 = rows 4096 + 128 bytes apart instead of 4096, 4 = every workgroup keeps
// its first tile and alternates between its first two K-steps: 96 KB per
// workgroup, re-read from L2)
// TB: token rows per step (128, or 256 with a two-slot ring)
template <int TB = 128>
__device__ __forceinline__ int ring_off(int s, int q, int wave, int lane, int nrows, int flags) {
  const int tile = (flags & 4) ? blockIdx.x : blockIdx.x + (s / 32) * gridDim.x;
  if (flags & 4) s %= 2;
  const int r = q < 8 ? 64 * wave + 8 * q + (lane >> 3) : 256 + (TB / 4) * wave + 8 * (q - 8) + (lane >> 3);
  const int row = (int)(((int64_t)tile * (256 + TB) + r) % nrows);
  const int ks = (flags & 1) ? (s + blockIdx.x) % 32 : s % 32;
  return row * (kRingRow + ((flags & 2) ? kRingBK : 0)) + ks * kRingBK + ((((lane & 7) ^ (lane >> 3)) & 7) << 4);
}
// LDS address of this wave's 8-row block q of a ring slot
template <int TB = 128>
__device__ __forceinline__ lds_u8* ring_dst(lds_u8* smem, int slot, int q, int wave) {
  const int r = q < 8 ? 64 * wave + 8 * q : 256 + (TB / 4) * wave + 8 * (q - 8);
  return smem + slot * (256 + TB) * kRingBK + r * kRingBK;
}
__device__ __forceinline__ void ring_sink(u32x4 x, uint32_t* sink, int wave, int lane) {
  uint32_t r = x[0] ^ x[1] ^ x[2] ^ x[3];
  for (int o = 32; o > 0; o >>= 1) r ^= (uint32_t)__shfl_xor((int)r, o, 64);
  if (lane == 0) sink[blockIdx.x * 4 + wave] = r;
}

// modes 0 (READS false) and 2 (READS true): direct-to-LDS loads; TB 128:
// three 48 KB slots, loads two steps ahead; TB 256: two 64 KB slots, loads
// one step ahead
template <bool READS, int TB>
__global__ __launch_bounds__(256) void ring_dma_kernel(const uint8_t* __restrict__ buf, int bytes, int steps,
                                                       uint32_t* __restrict__ sink, int flags) {
  constexpr int NS = TB == 128 ? 3 : 2, NQ = 8 + TB / 32, SB = (256 + TB) * kRingBK;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrows = bytes / (kRingRow + ((flags & 2) ? kRingBK : 0));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)buf, (short)0, bytes, 0x00020000);
  auto issue = [&](int s) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      // (computed apart: a template-dependent expression as the builtin's
      // argument drops the kernel's host stub)
      const int o = ring_off<TB>(s, q, wave, lane, nrows, flags);
      lds_u8* d = ring_dst<TB>(smem, s % NS, q, wave);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void __attribute__((address_space(3)))*)d, 16, o, 0, 0, 0);
    }
  };
  u32x4 x = {0u, 0u, 0u, 0u};
  issue(0);
  if (NS == 3) issue(1);
  for (int s = 0; s < steps; ++s) {
    // step s landed (three slots: s+1 may be in flight, its 12 loads); a
    // wait count that depends on TB would drop the kernel's host stub
    if (NS == 3)
      ring_wait_vm<12>();
    else
      ring_wait_vm<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const lds_u8* st = smem + (s % NS) * SB;
    if (READS) {
      // the product's reads: 8 A fragments of this wave's 64 rows and 16 B
      // fragments of all 128 token rows, 16 bytes per lane each, logical
      // chunk c of row r at position c ^ (r & 7) (the loads above put global
      // chunk (lane%8) ^ (lane/8) of row 8q + lane/8 at position lane%8)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = 64 * wave + (lane & 31) + 32 * (q & 1), c = (q >> 1) * 2 + (lane >> 5);
        x ^= *(const __attribute__((address_space(3))) u32x4*)(st + r * kRingBK + ((c ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int q = 0; q < TB / 8; ++q) {
        const int r = 256 + (lane & 31) + 32 * (q % (TB / 32)), c = (q / (TB / 32)) * 2 + (lane >> 5);
        x ^= *(const __attribute__((address_space(3))) u32x4*)(st + r * kRingBK + ((c ^ (r & 7)) << 4));
      }
    } else {
      x ^= *(const __attribute__((address_space(3))) u32x4*)(st + threadIdx.x * 16);
    }
    issue(s + NS - 1);  // into the slot of step s-1, which every wave has read
  }
  ring_wait_vm<0>();
  ring_sink(x, sink, wave, lane);
}

// modes 0 and 2 with 64-byte K-steps over 256 weight and 256 token rows
// (half a cache line of each row per step, 32 KB): four slots, loads three
// steps ahead (96 KB in flight).  A 1 KB load covers 16 rows; lane i loads
// logical chunk (i%4) ^ ((row/4)%4) of row i/4 into position i%4.
template <bool READS>
__global__ __launch_bounds__(256) void ring_half_kernel(const uint8_t* __restrict__ buf, int bytes, int steps,
                                                        uint32_t* __restrict__ sink) {
  constexpr int HB = 64, SB = 512 * HB;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrows = bytes / kRingRow;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)buf, (short)0, bytes, 0x00020000);
  const int lr = lane >> 2, lc = lane & 3;
  auto issue = [&](int s) {
    const int tile = blockIdx.x + (s / 64) * gridDim.x;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // rows 64w + 16q' + lane/4 of the weight block (q < 4) and of the token block
      const int r = (q < 4 ? 0 : 256) + 64 * wave + 16 * (q & 3) + lr;
      const int row = (int)(((int64_t)tile * 512 + r) % nrows);
      const int o = row * kRingRow + (s % 64) * HB + ((lc ^ ((r >> 2) & 3)) << 4);
      lds_u8* d = smem + (s % 4) * SB + (r - lr) * HB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void __attribute__((address_space(3)))*)d, 16, o, 0, 0, 0);
    }
  };
  u32x4 x = {0u, 0u, 0u, 0u};
  issue(0);
  issue(1);
  issue(2);
  for (int s = 0; s < steps; ++s) {
    ring_wait_vm<16>();  // step s landed; s+1 and s+2 may be in flight
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const lds_u8* st = smem + (s % 4) * SB;
    if (READS) {
      // one fp8 MFMA k-step: 2 A tiles and 8 B tiles of 32 rows, 32 bytes per
      // lane (logical chunks 2*(lane/32), +1)
#pragma unroll
      for (int q = 0; q < 20; ++q) {
        const int t = q >> 1, c = 2 * (lane >> 5) + (q & 1);
        const int r = t < 2 ? 64 * wave + 32 * t + (lane & 31) : 256 + 32 * (t - 2) + (lane & 31);
        x ^= *(const __attribute__((address_space(3))) u32x4*)(st + r * HB + ((c ^ ((r >> 2) & 3)) << 4));
      }
    } else {
      x ^= *(const __attribute__((address_space(3))) u32x4*)(st + threadIdx.x * 16);
    }
    issue(s + 3);  // into the slot of step s-1, which every wave has read
  }
  ring_wait_vm<0>();
  ring_sink(x, sink, wave, lane);
}

// mode 1: register loads (steps s+1 and s+2 in flight in registers while
// step s is stored), then 16-byte LDS stores
__global__ __launch_bounds__(256) void ring_reg_kernel(const uint8_t* __restrict__ buf, int bytes, int steps,
                                                       uint32_t* __restrict__ sink, int flags) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrows = bytes / (kRingRow + ((flags & 2) ? kRingBK : 0));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)buf, (short)0, bytes, 0x00020000);
  constexpr int TB = 128;
  u32x4 v[3][12];
  auto load = [&](u32x4 (&d)[12], int s) {
#pragma unroll
    for (int q = 0; q < 12; ++q) d[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, ring_off<TB>(s, q, wave, lane, nrows, flags), 0, 0);
  };
  auto store = [&](const u32x4 (&d)[12], int slot) {
#pragma unroll
    for (int q = 0; q < 12; ++q)
      *(__attribute__((address_space(3))) u32x4*)(ring_dst<128>(smem, slot, q, wave) + lane * 16) = d[q];
  };
  u32x4 x = {0u, 0u, 0u, 0u};
  load(v[0], 0);
  load(v[1], 1);
  int s = 0;
  auto body = [&](auto c) {
    constexpr int C = decltype(c)::value;
    load(v[(C + 2) % 3], s + 2);  // (the last two load steps nothing reads)
    store(v[C], s % 3);
    __syncthreads();
    x ^= *(__attribute__((address_space(3))) u32x4*)(smem + (s % 3) * kRingStage + threadIdx.x * 16);
    ++s;
  };
  while (s + 3 <= steps) {
    body(std::integral_constant<int, 0>{});
    body(std::integral_constant<int, 1>{});
    body(std::integral_constant<int, 2>{});
  }
  ring_sink(x, sink, wave, lane);
}

moe_status_t launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

}  // namespace

extern "C" {

int32_t moe_probes_abi_version(void) { return 4; }

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

moe_status_t moe_probe_ring_load(const void* buf, size_t bytes, int32_t grid, int32_t steps, int32_t mode,
                                 uint32_t* sink, void* stream) {
  const int flags = mode >> 2;
  mode &= 3;
  if (!buf || !sink || bytes % kRingRow != 0 || bytes < (size_t)512 * (kRingRow + kRingBK) ||
      bytes > ((size_t)1 << 30) || grid < 1 || grid > 65536 || steps < 3 || steps > (1 << 20) || steps % 3 != 0 ||
      mode > 2 || flags > 31 || ((flags & 24) && mode == 1) || ((flags & 16) && (flags & 15)))
    return MOE_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  const bool wide = (flags & 8) != 0;  // 256 token rows per step, two slots
  const bool half = (flags & 16) != 0;  // 256 token rows, 64-byte steps, four slots
  const size_t lds = half ? (size_t)4 * 512 * 64 : wide ? (size_t)2 * 512 * kRingBK : (size_t)kRingStages * kRingStage;
  const void* k = mode == 1 ? (const void*)ring_reg_kernel
                  : half ? (mode == 0 ? (const void*)ring_half_kernel<false> : (const void*)ring_half_kernel<true>)
                  : wide ? (mode == 0 ? (const void*)ring_dma_kernel<false, 256> : (const void*)ring_dma_kernel<true, 256>)
                         : (mode == 0 ? (const void*)ring_dma_kernel<false, 128> : (const void*)ring_dma_kernel<true, 128>);
  if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return MOE_ERR_DEVICE;
  const uint8_t* b = (const uint8_t*)buf;
  if (mode == 1) ring_reg_kernel<<<grid, 256, lds, st>>>(b, (int)bytes, steps, sink, flags);
  if (mode == 0 && half) ring_half_kernel<false><<<grid, 256, lds, st>>>(b, (int)bytes, steps, sink);
  if (mode == 2 && half) ring_half_kernel<true><<<grid, 256, lds, st>>>(b, (int)bytes, steps, sink);
  if (half) return launch_status();
  if (mode == 0 && !wide) ring_dma_kernel<false, 128><<<grid, 256, lds, st>>>(b, (int)bytes, steps, sink, flags);
  if (mode == 2 && !wide) ring_dma_kernel<true, 128><<<grid, 256, lds, st>>>(b, (int)bytes, steps, sink, flags);
  if (mode == 0 && wide) ring_dma_kernel<false, 256><<<grid, 256, lds, st>>>(b, (int)bytes, steps, sink, flags);
  if (mode == 2 && wide) ring_dma_kernel<true, 256><<<grid, 256, lds, st>>>(b, (int)bytes, steps, sink, flags);
  return launch_status();
}

}  // extern "C"
