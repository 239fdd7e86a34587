// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving, variant selection and stream-ordered launches.
// No device memory is allocated here and no call synchronises the stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "moe.h"
#include "launch.h"
#include "layer_small.h"
#include "moe_device.h"
#include "route_align.h"

using namespace moe;

namespace {

constexpr int kAlignBlockFused = 16;   // token tile of the decode products' B operand
constexpr int kPrefillMinPairs = 8192; // layers with at least this many pairs take the prefill products

// Layers with many pairs use the tiled prefill products (token block 128,
// weight tiles of 256 rows: 256 rows of H for the down product, 128 gate and
// 128 up rows for the gate/up product), fp8 or bf16.  Both contraction
// lengths (H and I, in bytes) must be an even number, at least four, of
// 128-byte K-steps.  The operand loads take 32-bit byte offsets into one
// expert's weights and into the activations.
bool use_prefill(int M, int k, moe_dtype_t dt, int H, int I) {
  const int64_t P = (int64_t)M * k, lim = INT32_MAX;
  const int esz = dt == MOE_DTYPE_FP8_E4M3 ? 1 : 2;
  auto steps_ok = [](int64_t K) { return K % (2 * kPfBK) == 0 && K >= 4 * kPfBK; };
  return (dt == MOE_DTYPE_FP8_E4M3 || dt == MOE_DTYPE_BF16) && P >= kPrefillMinPairs && H % kPfRows == 0 &&
         I % (kPfRows / 2) == 0 && steps_ok((int64_t)H * esz) && steps_ok((int64_t)I * esz) &&
         2 * (int64_t)I * H * esz <= lim && (int64_t)M * H * esz <= lim && P * I * esz <= lim;
}
// Align block of the fused call: 128 on the prefill path, else 16.
// decode_only: the deterministic and block-scaled modes take the decode path
// at every M.
int align_block(int M, int k, moe_dtype_t dt, int H, int I, bool decode_only) {
  return !decode_only && use_prefill(M, k, dt, H, I) ? kPfTok : kAlignBlockFused;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
int log2i(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return b;
}

moe_status_t launch_status() {
  hipError_t err = hipGetLastError();
  return err == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

constexpr int kDownLdsMax = 65536;  // LDS of one down-product workgroup staging e4m3 h
constexpr double kTokDownCachedW2 = 4.0 * (1 << 20);     // one XCD's L2
constexpr double kTokDownRepeatBytes = 16.0 * (1 << 20);  // repeated W2 reads the saved launch is worth

// Largest K split of the down product that the workspace holds partial sums
// for (ksplit * P * H fp32): as many slices as fit 64 MB, at most 16, and in
// fp8 mode at least the smallest split whose e4m3 token slice (64 tokens)
// fits the down product's LDS.
int down_ksplit_cap(int64_t P, int H, int I, bool fp8) {
  const int64_t per = std::max<int64_t>(1, P * (int64_t)H * 4);
  int cap = (int)std::max<int64_t>(1, std::min<int64_t>(16, (int64_t(64) << 20) / per));
  if (fp8) {
    const int nsteps = I / 128;
    for (int ks = 1; ks <= 16; ++ks) {
      if (nsteps % ks == 0 && 64 * gemm2_lds_stride(I / ks) <= kDownLdsMax) {
        cap = std::max(cap, ks);
        break;
      }
    }
  }
  return cap;
}

int64_t align_capacity(int64_t P, int E, int B) {
  int64_t cap = P + std::min<int64_t>(E, P) * (B - 1);
  return cdiv(cap, B) * B;
}

// ---------------------------------------------------------------- workspace
struct Layout {
  size_t ids, wts, counts, offsets, sorted, block_expert, num_padded, active, num_active;
  size_t xamax_part, scale_slot, h_amax, hist, logits, wg_hmax, xs_blk, xq, h, part, total;
  int64_t capacity;
  int block, n_blocks, n_route_wg;
};

// The workspace serves every mode of a shape (the default one and those that
// take the decode path at every M, whose align block may differ): the
// sort-and-pad arrays are sized for the larger of the two blocks' needs.
// capacity and n_blocks are those of the call's own block.
// part_slices: K slices of fp32 partial sums the layout holds for the down
// product (0: as many as any plan of the shape may take, down_ksplit_cap).
Layout make_layout(int M, int E, int H, int I, int k, moe_dtype_t dt, bool decode_only = false, int part_slices = 0) {
  Layout L{};
  const int64_t P = (int64_t)M * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += round_up(std::max<size_t>(bytes, 4), 256);
    return o;
  };
  const int B = align_block(M, k, dt, H, I, decode_only);
  L.block = B;
  L.capacity = align_capacity(P, E, B);
  L.n_blocks = (int)(L.capacity / B);
  int64_t cap_max = 0, blocks_max = 0;
  for (const int b : {align_block(M, k, dt, H, I, false), align_block(M, k, dt, H, I, true)}) {
    cap_max = std::max(cap_max, align_capacity(P, E, b));
    blocks_max = std::max(blocks_max, align_capacity(P, E, b) / b);
  }
  L.n_route_wg = route_grid(M, dt == MOE_DTYPE_FP8_E4M3 ? (int64_t)M * H : 0);
  L.ids = take(P * 4);
  L.wts = take(P * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.sorted = take((size_t)cap_max * 4);
  L.block_expert = take((size_t)blocks_max * 4);
  L.num_padded = take(4);
  L.active = take((size_t)E * 4);
  L.num_active = take(4);
  L.xamax_part = take((size_t)L.n_route_wg * 4);
  L.scale_slot = take(4);
  L.h_amax = take(4);
  L.hist = take((size_t)cdiv(M, 4 * kRouteRows) * E * 4);
  L.logits = take((size_t)M * E * 4);  // router logits computed by the layer (router_w given)
  L.wg_hmax = take((size_t)kLayer1MaxGrid * 4);  // single-launch layer: largest |h| of each workgroup
  const bool fp8 = dt == MOE_DTYPE_FP8_E4M3;
  L.xs_blk = take(fp8 ? (size_t)M * H / 128 : 0);  // block-scaled fp8: x's group scales
  L.xq = take(fp8 ? (size_t)M * H : 0);
  // h: bf16 (bf16 layers), fp32 (fp8 decode), fp32 + its e4m3 copy (fp8 prefill)
  L.h = take((size_t)P * I * (fp8 ? (use_prefill(M, k, dt, H, I) ? 5 : 4) : 2));
  const int slices = part_slices > 0 ? part_slices : down_ksplit_cap(P, H, I, dt == MOE_DTYPE_FP8_E4M3);
  // decode: [slices][P][H] fp32; prefill: [P][H] bf16 (never more)
  L.part = take((size_t)slices * (size_t)P * H * 4);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------- variants
// Launch shape of the two products.  The defaults come from cold-cache sweeps
// on the Mixtral-, Qwen3- and DeepSeek-shaped decode layers: streaming expert
// weights from HBM favours fewer waves with deeper software pipelines (the
// 4-token-tile variants keep a workgroup's registers high on purpose) over
// high occupancy.
struct Plan {
  int nt1, passes1, u1, ks1, tw1, ft1;     // gate/up (tw1 > 0: long-stream variant; ft1 groups per wave)
  int nt2, passes2, u2, ks2, wks2, lds2, tw2, fr2;  // down (tw2 > 0: long-stream variant; fr2 groups per wave)
  int rev;                                  // reversed grid order (Segments::rev)
  int tok, tok_chunks;                      // down product and combine per token (down_token_kernel)
};

bool valid_u(bool fp8, int u) { return fp8 ? (u == 1 || u == 2) : (u == 2 || u == 4); }
bool valid_wsplit(int ks) { return ks == 1 || ks == 2 || ks == 4; }

// blk: block-scaled fp8 (K-split variants only; h staged with its group
// scales in the down product's LDS, as for a dynamic h scale).
moe_status_t make_plan(int M, int E, int H, int I, int k, int S, bool fp8, bool qh, const moe_tuning_t* t, bool det,
                       bool blk, Plan* p) {
  const int kstep = fp8 ? 128 : 32;
  const int64_t P = (int64_t)M * k;
  const int n_act = (int)std::min<int64_t>(E, P);  // upper bound on experts with tokens
  // long-stream variants: one wave per SIMD walking tiles*n_act/1024 tiles,
  // taken when that is at most 8 (short K ranges, few tiles); otherwise the
  // K-split variants, whose many short workgroups are as fast
  const int ftiles = I / 16, rtiles = H / 32;
  auto stream_tiles = [&](int tiles) {
    const int64_t t = ((int64_t)n_act * tiles + 512) / 1024;
    return t > 8 ? 0 : (int)std::max<int64_t>(1, t);
  };
  p->tw1 = p->tw2 = 0;
  if (fp8) {
    p->nt1 = M >= 8 ? 4 : 1;
    p->u1 = (p->nt1 == 4 && H < 4096) ? 1 : 2;
    p->ks1 = (p->nt1 == 4 && H >= 4096) ? 1 : 4;
    p->nt2 = 1;
    p->u2 = 1;
    p->wks2 = 1;
    if (M >= 8) {
      p->tw1 = stream_tiles(ftiles);
      p->tw2 = stream_tiles(rtiles);
    }
  } else {
    p->nt1 = p->nt2 = 2;
    p->u1 = p->u2 = 4;
    p->ks1 = 4;
    p->wks2 = 4;
  }
  // Shared experts (S > 0) hold every token, the routed ones a few each: the
  // K-split variants' many short workgroups absorb the shared experts' long
  // ones, which the reversed grid order starts first.
  p->rev = S > 0 ? 1 : 0;
  if (S > 0) p->tw1 = p->tw2 = 0;
  if (t && t->reverse_order != 0) {
    if (t->reverse_order != 1 && t->reverse_order != -1) return MOE_ERR_UNSUPPORTED;
    p->rev = t->reverse_order > 0 ? 1 : 0;
  }
  if (t && t->token_tiles > 0) {
    if (t->token_tiles > 4) return MOE_ERR_UNSUPPORTED;
    p->nt1 = p->nt2 = t->token_tiles == 3 ? 4 : t->token_tiles;
  }
  if (t && t->unroll > 0) {
    if (!valid_u(fp8, t->unroll)) return MOE_ERR_UNSUPPORTED;
    p->u1 = p->u2 = t->unroll;
  }
  if (t && t->gemm1_ksplit > 0) {
    if (!valid_wsplit(t->gemm1_ksplit)) return MOE_ERR_UNSUPPORTED;
    p->ks1 = t->gemm1_ksplit;
  } else {
    while (p->ks1 > 1 && (H / p->ks1) % kstep != 0) p->ks1 /= 2;  // each wave takes whole K-steps
  }
  if (t && t->gemm2_wave_ksplit > 0) {
    if (!valid_wsplit(t->gemm2_wave_ksplit)) return MOE_ERR_UNSUPPORTED;
    p->wks2 = t->gemm2_wave_ksplit;
  }
  for (int* tw : {&p->tw1, &p->tw2}) {
    const int v = tw == &p->tw1 ? (t ? t->gemm1_stream_tiles : 0) : (t ? t->gemm2_stream_tiles : 0);
    if (v > 16) return MOE_ERR_UNSUPPORTED;
    if (v != 0) *tw = v > 0 ? v : 0;
  }
  if (blk) {  // block-scaled fp8: the K-split variants only
    if (t && (t->gemm1_stream_tiles > 0 || t->gemm2_stream_tiles > 0)) return MOE_ERR_UNSUPPORTED;
    p->tw1 = p->tw2 = 0;
  }
  if (p->tw1 > 0 && (H / kstep) % p->u1 != 0) {  // whole stages per row
    if (t && t->unroll > 0) return MOE_ERR_UNSUPPORTED;
    p->u1 = 1;
  }
  if (p->tw2 > 0) p->wks2 = 1;  // the long-stream down product does not split K over waves
  if (det) {
    // Deterministic mode: the order of every output's sums is fixed by the
    // shape alone, never by M.  Gate/up: K split over ks1 waves (fp8 1, bf16
    // 4), the long-stream variant only with ks1 = 1, whose one chain of
    // k-steps is the K-split variant's with one wave; down: one K slice split
    // over wks2 waves (fp8 1, bf16 4), the long-stream variant only with
    // wks2 = 1.  Tunings that change those orders are refused.
    if (t && (t->gemm1_ksplit > 0 || t->gemm2_ksplit > 0 || t->gemm2_wave_ksplit > 0)) return MOE_ERR_INVALID_ARG;
    p->ks1 = fp8 ? 1 : 4;
    const int wks = fp8 ? 1 : 4;
    if ((t && t->gemm1_stream_tiles > 0 && p->ks1 > 1) || (t && t->gemm2_stream_tiles > 0 && wks > 1))
      return MOE_ERR_INVALID_ARG;
    if (p->ks1 > 1) p->tw1 = 0;
    if (wks > 1) p->tw2 = 0;
    p->wks2 = wks;
  }
  if ((H / p->ks1) % kstep != 0) return MOE_ERR_UNSUPPORTED;
  // K-split gate/up: 16-feature groups per wave (each output's sums are the
  // same either way).  bf16: two, with two k-steps per stage unless the
  // unroll is given, where the halved grid keeps at least 2048 workgroups
  // (Mixtral shape: M = 63 334 vs 361 us, M = 4..32 1-2 % faster; at M = 1,
  // 896 workgroups, 86 vs 79 us); fp8: one (DeepSeek shape M = 64, 128: two
  // are 2 % slower)
  p->ft1 = 1;
  if (!fp8 && p->tw1 == 0 && (int64_t)(I / 16) / (8 / p->ks1) * n_act * cdiv(M, p->nt1 * 16) >= 2048) {
    p->ft1 = 2;
    if (!(t && t->unroll > 0)) p->u1 = 2;
  }
  if (t && t->gemm1_feature_tiles != 0) {
    if (t->gemm1_feature_tiles != 1 && t->gemm1_feature_tiles != 2) return MOE_ERR_UNSUPPORTED;
    if (t->gemm1_feature_tiles == 2 && p->tw1 > 0) return MOE_ERR_UNSUPPORTED;  // a long-stream gate/up
    p->ft1 = t->gemm1_feature_tiles;
  }
  if (p->tw1 > 0) p->ft1 = 1;
  p->passes1 = (int)cdiv(M, p->nt1 * 16);
  p->passes2 = (int)cdiv(M, p->nt2 * 16);

  // K-split down: 32-row groups per wave (each output's sums are the same
  // for the same K slices); the workgroup's rows must divide H.  Default:
  // two for bf16 layers with at least 12 pairs per expert that can hold
  // tokens, where most experts take two token tiles and the token rows
  // would be read as often as the weights (Mixtral shape M = 63: 170 vs
  // 182 us; at M <= 32 the halved grid takes more K slices and is slower)
  const bool fr2_ok = p->tw2 == 0 && (H / 32) % (8 / p->wks2) == 0;
  const bool fr2_pinned = t && t->gemm2_row_tiles != 0;
  p->fr2 = (!fp8 && fr2_ok && P >= 12 * (int64_t)n_act) ? 2 : 1;
  if (fr2_pinned) {
    if (t->gemm2_row_tiles != 1 && t->gemm2_row_tiles != 2) return MOE_ERR_UNSUPPORTED;
    if (t->gemm2_row_tiles == 2 && !fr2_ok) return MOE_ERR_UNSUPPORTED;
    p->fr2 = t->gemm2_row_tiles;
  }
  // down: K slices in separate workgroups; each slice's K range must split
  // evenly over wks2 waves, and with a dynamic fp8 h scale the quantised
  // token slice must fit the workgroup's LDS.  Default: the fewest slices
  // that give at least 1024 workgroups (4 per CU), or 256 (one per CU) for
  // the long-stream variant.
  const int nsteps2 = I / kstep;
  auto fits = [&](int ks) {
    if (nsteps2 % (ks * p->wks2) != 0) return false;
    if (p->tw2 > 0 && (nsteps2 / ks) % p->u2 != 0) return false;
    const int64_t lds = (qh ? (int64_t)p->nt2 * 16 * gemm2_lds_stride(I / ks) : 0) +
                        (blk ? gemm2_block_scale_bytes(p->nt2 * 16, I / ks) : 0) +
                        gemm2_red_bytes(p->nt2, p->wks2, p->fr2);
    return lds <= kDownLdsMax;
  };
  const int ks_cap = down_ksplit_cap(P, H, I, fp8);
  auto pick_ks2 = [&] {
    const int64_t groups2 = p->tw2 > 0 ? cdiv(rtiles, 4 * p->tw2) : H / (32 * (p->fr2 * 4 / p->wks2));
    const int64_t wgs_per_slice = groups2 * n_act * p->passes2;
    const int64_t wgs_target = p->tw2 > 0 ? 256 : 1024;
    p->ks2 = 0;
    for (int ks = 1; ks <= (det ? 1 : ks_cap); ++ks) {
      if (!fits(ks)) continue;
      p->ks2 = ks;
      if (wgs_per_slice * ks >= wgs_target) break;
    }
  };
  pick_ks2();
  if (p->ks2 == 0 && p->fr2 == 2 && !fr2_pinned) {  // the default's second group does not fit: one
    p->fr2 = 1;
    pick_ks2();
  }
  if (t && t->gemm2_ksplit > 0) {
    const int ks = t->gemm2_ksplit;
    if (ks > ks_cap || !fits(ks)) return MOE_ERR_UNSUPPORTED;
    p->ks2 = ks;
  }
  if (p->ks2 == 0) return MOE_ERR_UNSUPPORTED;
  p->lds2 = (qh ? p->nt2 * 16 * gemm2_lds_stride(I / p->ks2) : 0) +
            (blk ? gemm2_block_scale_bytes(p->nt2 * 16, I / p->ks2) : 0);

  // Down product and combine per token (small layers): K chunks per pair so
  // that the token has at least eight units (two per wave, streamed together)
  // where I's k-steps split evenly.  Per token, every pair of an expert after
  // its first reads that expert's W2 again: free while W2 fits an XCD's L2
  // (the repeats hit it), else a whole matrix from HBM.  The default takes
  // the per-token path when the expected repeats' bytes stay below what the
  // saved launch is worth (16 MB, about 2.5 us of HBM time): always at
  // M = 1, and with small experts (Qwen3-like) up to 64 pairs; not with a few
  // large experts that many tokens share (Mixtral at M >= 2 measured up to 3x
  // slower).
  const int mode = t ? t->down_per_token : 0;
  if (mode < -1 || mode > 1) return MOE_ERR_UNSUPPORTED;
  const bool pinned = t && (t->gemm2_ksplit > 0 || t->gemm2_wave_ksplit > 0 || t->gemm2_stream_tiles != 0 ||
                            t->gemm2_row_tiles != 0);
  const bool tok_fits = !det && !blk && P <= kTokDownPairs && (!qh || (int64_t)k * I <= kTokDownLds);
  if (mode == 1 && !tok_fits) return MOE_ERR_UNSUPPORTED;
  const int Er = E - S, kr = k - S;
  const double distinct = Er * (1.0 - std::pow(1.0 - (double)kr / Er, (double)M));  // expected routed experts
  const double repeats = ((double)M * kr - distinct) + (double)S * (M - 1);
  const double w2_bytes = (double)H * I * (fp8 ? 1 : 2);
  const bool tok_pays = w2_bytes <= kTokDownCachedW2 || repeats * w2_bytes <= kTokDownRepeatBytes;
  p->tok = tok_fits && (mode == 1 || (mode == 0 && !pinned && tok_pays)) ? 1 : 0;
  p->tok_chunks = 1;
  while (k * p->tok_chunks < 8 && nsteps2 % (2 * p->tok_chunks) == 0) p->tok_chunks *= 2;
  return MOE_OK;
}

// ---------------------------------------------------------------- launches
bool launch_route(const float* logits, int M, int E, int k, int S, int32_t* ids, float* wts, const RouteFusedArgs& fa,
                  hipStream_t st) {
  const dim3 grid((unsigned)route_grid(M, fa.x_amax_part ? (int64_t)M * fa.H : 0));
  switch ((int)cdiv(E, 16)) {  // keys per lane, rounded up to a power of two
    case 1: route_topk_kernel<1><<<grid, 256, 0, st>>>(logits, M, E, k, S, ids, wts, fa); break;
    case 2: route_topk_kernel<2><<<grid, 256, 0, st>>>(logits, M, E, k, S, ids, wts, fa); break;
    case 3: case 4: route_topk_kernel<4><<<grid, 256, 0, st>>>(logits, M, E, k, S, ids, wts, fa); break;
    case 5: case 6: case 7: case 8: route_topk_kernel<8><<<grid, 256, 0, st>>>(logits, M, E, k, S, ids, wts, fa); break;
    default:
      if (E <= 256)
        route_topk_kernel<16><<<grid, 256, 0, st>>>(logits, M, E, k, S, ids, wts, fa);
      else
        route_topk_kernel<32><<<grid, 256, 0, st>>>(logits, M, E, k, S, ids, wts, fa);
  }
  return true;
}

// Workgroups of a persistent launch with one workgroup per CU: the current
// device's CU count rounded down to a multiple of 8, so that workgroup b stays
// on XCD b % 8 while it walks items b, b + wgs, ...  Cached per device.
moe_status_t persistent_wgs(int* wgs) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // 0 until queried; callers may race, all store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *wgs = c;
      return MOE_OK;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    return MOE_ERR_DEVICE;
  const int n = cus / 8 * 8;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  *wgs = n;
  return MOE_OK;
}

void launch_prologue_small(const float* logits, int M, int E, int k, int S, int32_t* ids, float* wts, int B,
                           const AlignOut& o, const SmallQuant& q, hipStream_t st) {
  const int lb = log2i(B), ib = log2i(E + S);
  const dim3 grid(1 + (q.xq ? (unsigned)cdiv((int64_t)M * q.H, kSmallQuantPerWg) : 0u));
  switch ((int)cdiv(E, 16)) {
    case 1: prologue_small_kernel<1><<<grid, 1024, 0, st>>>(logits, M, E, k, S, ids, wts, lb, ib, o, q); break;
    case 2: prologue_small_kernel<2><<<grid, 1024, 0, st>>>(logits, M, E, k, S, ids, wts, lb, ib, o, q); break;
    case 3: case 4: prologue_small_kernel<4><<<grid, 1024, 0, st>>>(logits, M, E, k, S, ids, wts, lb, ib, o, q); break;
    case 5: case 6: case 7: case 8:
      prologue_small_kernel<8><<<grid, 1024, 0, st>>>(logits, M, E, k, S, ids, wts, lb, ib, o, q);
      break;
    default:  // E <= kSmallMaxExperts
      prologue_small_kernel<16><<<grid, 1024, 0, st>>>(logits, M, E, k, S, ids, wts, lb, ib, o, q);
  }
}

// The router's per-workgroup expert counts serve the align step when its
// workgroups hold a whole number of routing workgroups' pairs (k a power of
// two up to 16).
bool hist_usable(int k) { return is_pow2(k) && k <= 16; }

void launch_align(const int32_t* ids, int64_t P, int E, int B, const AlignOut& o, const QuantXArgs& q, int n_quant_wg,
                  hipStream_t st, const AlignHist& hist = AlignHist{nullptr, 0, 0}) {
  const int n_align = (int)std::max<int64_t>(1, cdiv(P, kAlignChunk));
  align_kernel<<<n_align + n_quant_wg, 256, 0, st>>>(ids, (int)P, E, B, log2i(B), log2i(E), n_align, o, q, hist);
}

// Router logits: 16 experts x 16 tokens per workgroup at decode sizes, x 64
// tokens beyond (the same per-tile sums, fewer reads of the router rows).
void launch_router_logits(const void* x, const void* w, int M, int E, int H, float* logits, hipStream_t st) {
  const uint16_t* xx = (const uint16_t*)x;
  const uint16_t* ww = (const uint16_t*)w;
  if (M <= 64) {
    router_logits_kernel<1><<<dim3((unsigned)cdiv(E, 16), (unsigned)cdiv(M, 16)), 1024, 0, st>>>(xx, ww, M, E, H, logits);
  } else {
    router_logits_kernel<4><<<dim3((unsigned)cdiv(E, 16), (unsigned)cdiv(M, 64)), 1024, 0, st>>>(xx, ww, M, E, H, logits);
  }
}

moe_status_t check_shape(int M, int E, int k) {
  if (M < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)M * k >= (int64_t)INT32_MAX - kAlignChunk) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// ---------------------------------------------------------------- two-launch layer
// Grid of its gate/up launch: as many workgroups as are resident at once
// (two per CU: the kernel's ~150 VGPRs allow two waves per SIMD), each
// paying the routing prologue once and then looping over gate/up items; a
// larger grid pays it again in every later round.  The default takes the two
// launches up to 1024 items (16-feature tiles x experts with tokens): at M = 1
// measured 1.8 us faster on the Qwen3-shaped layer (384 items) and 1 us on
// the DeepSeek-shaped one (1024), 1 us slower on the Mixtral-shaped one
// (1792: 3.5 items per workgroup, the pipeline drained between them).
constexpr int kTinyGrid = 512;
constexpr int64_t kTinyDefaultItems = 1024;
// Items of at most 64 KB (32 weight rows of H) cost little to switch between:
// the default takes the two launches up to 4096 of them (Qwen3-shaped layer,
// 1536 items at M = 4: 42.0 vs 46.0 us).
constexpr int64_t kTinySmallItemsMax = 4096;
constexpr int64_t kTinySmallItemBytes = 65536;

// ---------------------------------------------------------------- single-launch layer
// The single-launch layer's wave split of the down product (4, 2 or 1: the
// most that divides I's K-steps), or 0 when the layer does not fit it: more
// than 16 tokens or 64 pairs, more than 256 routed experts, a gate/up K that
// four waves cannot split into whole MFMA k-steps, or (dynamic fp8 h scale)
// a down-product token slice beyond the workgroup's LDS.
int layer1_wks(int M, int Er, int k, int H, int I, bool fp8, bool hdyn) {
  const int kstep = fp8 ? 128 : 32;
  if (M > kLayer1Tokens || (int64_t)M * k > kLayer1Pairs || Er > kLayer1Experts) return 0;
  if ((H / 4) % kstep != 0) return 0;
  if (hdyn && 16 * gemm2_lds_stride(I) > kLayer1LdsMax - 24 * 1024) return 0;  // static LDS is under 24 KB
  const int nsteps = I / kstep;
  return nsteps % 4 == 0 ? 4 : nsteps % 2 == 0 ? 2 : 1;
}

// ---------------------------------------------------------------- no-alloc scratch
// Workspace of moe_fused_forward_noalloc: one array per GPU, held by the
// loaded code object until the process ends.  Its name is a host-side
// stand-in in host code: the device address comes from hipGetSymbolAddress,
// taken once per device (with that device current) and cached.
constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

moe_status_t noalloc_scratch(uint8_t** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<uint8_t*> cached[kMaxDevices];  // null until taken; racing first calls store the same address
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  uint8_t* p = cached[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return MOE_ERR_DEVICE;
    p = (uint8_t*)addr;
    cached[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    default: break;
  }
  return "MOE_ERR_UNKNOWN";
}

int32_t moe_abi_version(void) { return 15; }

moe_status_t moe_route_topk(const float* logits, int32_t M, int32_t E, int32_t top_k, int32_t* topk_ids,
                            float* topk_weights, void* stream) {
  moe_status_t rc = check_shape(M, E, top_k);
  if (rc != MOE_OK) return rc;
  if (M == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4)) return MOE_ERR_INVALID_ARG;
  launch_route(logits, M, E, top_k, 0, topk_ids, topk_weights, RouteFusedArgs{}, (hipStream_t)stream);
  return launch_status();
}

moe_status_t moe_router_logits(const void* x, const void* router_w, int32_t M, int32_t E, int32_t H, float* logits,
                               void* stream) {
  if (M < 0 || E < 1 || E > kMaxExperts) return M < 0 || E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED;
  if (H < 128 || H % 128) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!x || !router_w || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(logits, 4)) return MOE_ERR_INVALID_ARG;
  launch_router_logits(x, router_w, M, E, H, logits, (hipStream_t)stream);
  return launch_status();
}

size_t moe_align_capacity(int32_t M, int32_t top_k, int32_t E, int32_t block) {
  if (check_shape(M, E, top_k) != MOE_OK || !is_pow2(block) || block > 256) return 0;
  return (size_t)align_capacity((int64_t)M * top_k, E, block);
}

moe_status_t moe_align(const int32_t* topk_ids, int32_t M, int32_t top_k, int32_t E, int32_t block,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_ids, int32_t* block_expert,
                       int32_t* num_padded, void* stream) {
  moe_status_t rc = check_shape(M, E, top_k);
  if (rc != MOE_OK) return rc;
  if (!is_pow2(block) || block > 256) return block > 256 && is_pow2(block) ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG;
  const int64_t P = (int64_t)M * top_k;
  const int64_t cap = align_capacity(P, E, block);
  if ((P > 0 && !topk_ids) || !expert_counts || !expert_offsets || !num_padded) return MOE_ERR_INVALID_ARG;
  if (cap > 0 && (!sorted_ids || !block_expert)) return MOE_ERR_INVALID_ARG;
  for (const void* p : {(const void*)topk_ids, (const void*)expert_counts, (const void*)expert_offsets,
                        (const void*)sorted_ids, (const void*)block_expert, (const void*)num_padded})
    if (!aligned(p, 4)) return MOE_ERR_INVALID_ARG;
  AlignOut o{expert_counts, expert_offsets, sorted_ids, block_expert, num_padded, nullptr, nullptr,
             (int)(cap / block)};
  launch_align(topk_ids, P, E, block, o, QuantXArgs{}, 0, (hipStream_t)stream);
  return launch_status();
}

moe_status_t moe_quant_e4m3(const float* in, int64_t n, const float* scale, uint8_t* out, void* stream) {
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!in || !scale || !out || !aligned(in, 16) || !aligned(out, 4) || !aligned(scale, 4))
    return MOE_ERR_INVALID_ARG;
  quant_f32_kernel<<<(unsigned)cdiv(n, 1024), 256, 0, (hipStream_t)stream>>>(in, n, scale, out);
  return launch_status();
}

size_t moe_fused_workspace_size(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, moe_dtype_t dtype) {
  if (check_shape(M, E, top_k) != MOE_OK || H < 128 || I < 128 || H % 128 || I % 128) return 0;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3) return 0;
  return make_layout(M, E, H, I, top_k, dtype).total;
}

moe_status_t moe_fused_align_shape(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, moe_dtype_t dtype,
                                   int32_t deterministic, int32_t weight_scale_mode, int32_t* block,
                                   int64_t* capacity) {
  moe_status_t rc = check_shape(M, E, top_k);
  if (rc != MOE_OK) return rc;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (deterministic != 0 && deterministic != 1) return MOE_ERR_INVALID_ARG;
  if (weight_scale_mode < 0 || weight_scale_mode > 3 || (weight_scale_mode != 0 && dtype != MOE_DTYPE_FP8_E4M3))
    return MOE_ERR_INVALID_ARG;
  if (!block || !capacity) return MOE_ERR_INVALID_ARG;
  if (H < 128 || I < 128 || H % 128 || I % 128) return MOE_ERR_UNSUPPORTED;
  const Layout L = make_layout(M, E, H, I, top_k, dtype, deterministic == 1 || weight_scale_mode == 3);
  *block = L.block;
  *capacity = L.capacity;
  return MOE_OK;
}

// fp8 prefill: router, align (block 128) with the activation quantisation,
// the two tiled products and the per-token combine.
static moe_status_t prefill_forward(const moe_fused_args_t* a, hipStream_t st, void* const* ev, const Layout& L,
                                    uint8_t* ws, int32_t* ids, float* wts, const AlignOut& o, float* xamax_part,
                                    float* scale_slot, unsigned* h_amax, uint8_t* xq, uint8_t* h, float* part,
                                    bool hdyn, int S) {
  const bool pc = a->weight_scale_mode == 1;
  const int es = a->weight_scale_mode == 2 ? 1 : 0;  // one weight scale per expert
  auto rec = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], st);
  };
  moe_status_t rc;
  const int M = a->M, E = a->E, H = a->H, I = a->I, k = a->top_k;
  int32_t* hist_buf = (int32_t*)(ws + L.hist);
  const int64_t P = (int64_t)M * k;
  rec(0);
  int32_t* hist = hist_usable(k) ? hist_buf : nullptr;
  const bool bf = a->dtype == MOE_DTYPE_BF16;
  RouteFusedArgs fa{(const uint16_t*)a->x, H, (bf || a->x_scale) ? nullptr : xamax_part, hdyn ? h_amax : nullptr,
                    hist};
  launch_route(a->logits, M, E - S, k - S, S, ids, wts, fa, st);
  rec(1);
  if ((rc = launch_status()) != MOE_OK) return rc;
  rec(2);
  QuantXArgs q{};
  if (!bf) {
    q.x = (const uint16_t*)a->x;
    q.n = (int64_t)M * H;
    q.amax_part = xamax_part;
    q.n_part = L.n_route_wg;
    q.static_scale = a->x_scale;
    q.xq = xq;
    q.scale_slot = scale_slot;
  }
  launch_align(ids, P, E, kPfTok, o, q, bf ? 0 : (int)cdiv(q.n, kAlignQuantPerWg), st,
               AlignHist{hist, (int)cdiv(M, 4 * kRouteRows), hist ? 16 / k : 0});
  rec(3);
  if ((rc = launch_status()) != MOE_OK) return rc;

  const PrefillSeg seg{o.sorted_ids, o.block_expert, o.offsets, o.counts, o.num_padded};
  uint8_t* hq = hdyn ? h + (size_t)P * I * 4 : h;  // e4m3 h read by the down product (after the fp32 h)
  // bound on the linear item index: 8 XCDs x tiles x the blocks per XCD that
  // the largest possible block count gives
  auto prefill_items = [&](int T) { return 8 * T * (int)cdiv(L.n_blocks, 8); };
  // persistent workgroups: one per CU, a multiple of 8 (one XCD each)
  int wgs = 0;
  if ((rc = persistent_wgs(&wgs)) != MOE_OK) return rc;
  rec(4);
  {
    const int T = I / (kPfRows / 2);  // 256-row tiles of W13: 128 gate + 128 up rows
    const int items = prefill_items(T);
    PrefillArgs g{(const uint8_t*)a->w13, bf ? (const uint8_t*)a->x : xq, seg, H, I, k, (int)P, T, items,
                  a->w13_scale, scale_slot, nullptr, a->h_scale, h, h_amax, es};
    if (!launch_prefill_gemm(0, bf, hdyn, pc, std::min(wgs, items), st, g)) return MOE_ERR_DEVICE;
  }
  rec(5);
  if ((rc = launch_status()) != MOE_OK) return rc;
  rec(6);
  {
    if (hdyn) {
      const int64_t n = P * I;
      launch_prefill_quant_h((const float*)h, n, h_amax, hq, st);
      if ((rc = launch_status()) != MOE_OK) return rc;
    }
    const int T = H / kPfRows;
    const int items = prefill_items(T);
    PrefillArgs g{(const uint8_t*)a->w2, hq, seg, H, I, k, (int)P, T, items, a->w2_scale, a->h_scale, h_amax, nullptr,
                  (uint8_t*)part, nullptr, es};
    if (!launch_prefill_gemm(1, bf, hdyn, pc, std::min(wgs, items), st, g)) return MOE_ERR_DEVICE;
  }
  rec(7);
  if ((rc = launch_status()) != MOE_OK) return rc;
  rec(8);
  launch_prefill_finalize((const uint16_t*)part, wts, (uint16_t*)a->y, M, H, k, scale_slot, h_amax, a->h_scale,
                          bf ? nullptr : a->scales_out, st);
  rec(9);
  return launch_status();
}

// noalloc: the workspace is the library's scratch array (the caller passes
// none), its partial-sum region sized for the plan's K slices only.
// path_out: validate and plan only (y and the workspace are not required),
// report the launch sequence in *path_out and enqueue nothing.
static moe_status_t fused_forward(const moe_fused_args_t* a, hipStream_t st, void* const* ev, bool noalloc = false,
                                  int32_t* path_out = nullptr) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (noalloc && (a->workspace || a->workspace_bytes)) return MOE_ERR_INVALID_ARG;
  auto rec = [&](int i) {
    if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], st);
  };
  moe_status_t rc = check_shape(a->M, a->E, a->top_k);
  if (rc != MOE_OK) return rc;
  // shared experts: every token also passes through experts E..E+S-1 with
  // weight one; from the routing on they are S more experts and S more slots
  // per token
  const int S = a->n_shared;
  if (S < 0) return MOE_ERR_INVALID_ARG;
  if ((rc = check_shape(a->M, a->E + S, a->top_k + S)) != MOE_OK) return rc;
  if (a->dtype != MOE_DTYPE_BF16 && a->dtype != MOE_DTYPE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (a->H < 128 || a->I < 128 || a->H % 128 || a->I % 128) return MOE_ERR_UNSUPPORTED;
  const bool fp8 = a->dtype == MOE_DTYPE_FP8_E4M3;
  const int Er = a->E, kr = a->top_k;  // the routed experts and slots
  const int M = a->M, E = Er + S, H = a->H, I = a->I, k = kr + S;
  if (!fp8 && (a->w13_scale || a->w2_scale || a->x_scale || a->h_scale)) return MOE_ERR_INVALID_ARG;
  if (fp8 && (!a->w13_scale || !a->w2_scale)) return MOE_ERR_INVALID_ARG;
  if (a->weight_scale_mode != 0 && (a->weight_scale_mode < 0 || a->weight_scale_mode > 3 || !fp8))
    return MOE_ERR_INVALID_ARG;
  // block-scaled: per-block weight scales, activations scaled per 128-element
  // group in the layer (no tensor scales to give)
  const bool blk = a->weight_scale_mode == 3;
  if (blk && (a->x_scale || a->h_scale)) return MOE_ERR_INVALID_ARG;
  const bool pc = a->weight_scale_mode == 1;
  if (pc && (!aligned(a->w13_scale, 16) || !aligned(a->w2_scale, 16))) return MOE_ERR_INVALID_ARG;
  if (M == 0) {
    if (path_out) {
      *path_out = MOE_PATH_NONE;
      return MOE_OK;
    }
    if (ev)
      for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i) rec(i);
    return MOE_OK;
  }
  if (!a->x || !a->w13 || !a->w2 || (!path_out && (!a->y || (!noalloc && !a->workspace)))) return MOE_ERR_INVALID_ARG;
  // logits: given, or computed from the router weights (exactly one of the two)
  if ((a->logits == nullptr) == (a->router_w == nullptr)) return MOE_ERR_INVALID_ARG;
  if (a->logits_out && !a->router_w) return MOE_ERR_INVALID_ARG;
  for (const void* p : {a->x, a->w13, a->w2, (const void*)a->y, a->router_w})
    if (!aligned(p, 16)) return MOE_ERR_INVALID_ARG;
  if (!aligned(a->logits_out, 4)) return MOE_ERR_INVALID_ARG;
  if (!aligned(a->workspace, 256)) return MOE_ERR_INVALID_ARG;
  for (const void* p : {(const void*)a->logits, (const void*)a->w13_scale, (const void*)a->w2_scale,
                        (const void*)a->x_scale, (const void*)a->h_scale, (const void*)a->topk_ids,
                        (const void*)a->topk_weights, (const void*)a->expert_counts, (const void*)a->scales_out,
                        (const void*)a->expert_offsets, (const void*)a->sorted_ids, (const void*)a->block_expert,
                        (const void*)a->num_padded})
    if (!aligned(p, 4)) return MOE_ERR_INVALID_ARG;
  // deterministic mode: batch-invariant only with per-tensor activation
  // scales fixed by the caller (a dynamic scale is an amax over the batch)
  if (a->deterministic != 0 && a->deterministic != 1) return MOE_ERR_INVALID_ARG;
  const bool det = a->deterministic == 1;
  if (det && fp8 && !blk && (!a->x_scale || !a->h_scale)) return MOE_ERR_INVALID_ARG;
  const bool hdyn = fp8 && !a->h_scale;
  const bool prefill = !det && !blk && use_prefill(M, k, a->dtype, a->H, a->I);
  Plan plan{};
  if (!prefill) {
    rc = make_plan(M, E, H, I, k, S, fp8, hdyn, a->tuning, det, blk, &plan);
    if (rc != MOE_OK) return rc;
  }
  // the single-launch layer for tiny token counts, on request (never with
  // router weights, whose product is a launch of its own, nor in the
  // deterministic mode, whose K order it does not keep)
  int l1_wks = 0;
  if (!prefill) {
    const int mode = a->tuning ? a->tuning->single_launch : 0;
    if (mode < -1 || mode > 1) return MOE_ERR_UNSUPPORTED;
    if (mode == 1) {
      if (!det && !blk && !a->router_w) l1_wks = layer1_wks(M, Er, k, H, I, fp8, hdyn);
      if (!l1_wks) return MOE_ERR_UNSUPPORTED;
    }
  }
  // tiny layers in two launches: the routing, quantisation and sort-and-pad
  // in every gate/up workgroup, the combine in the per-token down product
  // (taken by default unless the gate/up launch shape is pinned)
  bool tiny = false;
  const int rmode = a->tuning ? a->tuning->routing_in_gate_up : 0;
  if (rmode < -1 || rmode > 1) return MOE_ERR_UNSUPPORTED;
  if (!prefill && !l1_wks) {
    const bool g1_pinned = a->tuning && (a->tuning->gemm1_ksplit > 0 || a->tuning->token_tiles > 0 ||
                                         a->tuning->unroll > 0 || a->tuning->gemm1_stream_tiles != 0 ||
                                         a->tuning->gemm1_feature_tiles != 0);
    // (gate/up K split over four waves in whole MFMA k-steps, as in the single-launch layer)
    const bool fits = plan.tok && M <= kLayer1Tokens && (int64_t)M * k <= kLayer1Pairs && Er <= kLayer1Experts &&
                      (H / 4) % (fp8 ? 128 : 32) == 0 && (!fp8 || (int64_t)M * H <= kTinyXElems);
    const int64_t items = (int64_t)std::min<int64_t>(Er + S, (int64_t)M * k) * (I / 16);
    const bool pays = items <= kTinyDefaultItems ||
                      (items <= kTinySmallItemsMax && 32 * (int64_t)H * (fp8 ? 1 : 2) <= kTinySmallItemBytes);
    tiny = fits && (rmode == 1 || (rmode == 0 && !g1_pinned && pays));
  }
  if (rmode == 1 && !tiny) return MOE_ERR_UNSUPPORTED;  // required where the layer takes another path
  if (path_out) {
    *path_out = prefill ? MOE_PATH_PREFILL : l1_wks ? MOE_PATH_SINGLE_LAUNCH : tiny ? MOE_PATH_TWO_LAUNCHES
              : plan.tok ? MOE_PATH_DECODE_TOKEN_DOWN : MOE_PATH_DECODE;
    return MOE_OK;
  }
  // the scratch array holds the partial sums of the plan's K slices only
  const Layout L = make_layout(M, E, H, I, k, a->dtype, det || blk, noalloc && !prefill ? plan.ks2 : 0);
  uint8_t* ws = (uint8_t*)a->workspace;
  if (noalloc) {
    if (L.total > kNoallocScratchBytes) return MOE_ERR_UNSUPPORTED;
    if ((rc = noalloc_scratch(&ws)) != MOE_OK) return rc;
  } else if (a->workspace_bytes < L.total) {
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  // router logits from the hidden states (the step before routing), inside
  // the route stage: its start event is recorded here and not again
  moe_fused_args_t ax = *a;  // the layer as the steps after routing see it
  ax.E = E;
  ax.top_k = k;
  void* ev_rest[2 * MOE_NUM_STAGES];
  if (a->router_w) {
    float* lo = a->logits_out ? a->logits_out : (float*)(ws + L.logits);
    rec(0);
    launch_router_logits(a->x, a->router_w, M, Er, H, lo, st);
    if ((rc = launch_status()) != MOE_OK) return rc;
    ax.logits = lo;
    if (ev) {
      for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i) ev_rest[i] = ev[i];
      ev_rest[0] = nullptr;
      ev = ev_rest;
    }
  }
  a = &ax;
  int32_t* ids = a->topk_ids ? a->topk_ids : (int32_t*)(ws + L.ids);
  float* wts = a->topk_weights ? a->topk_weights : (float*)(ws + L.wts);
  int32_t* counts = a->expert_counts ? a->expert_counts : (int32_t*)(ws + L.counts);
  int32_t* offsets = a->expert_offsets ? a->expert_offsets : (int32_t*)(ws + L.offsets);
  int32_t* sorted = a->sorted_ids ? a->sorted_ids : (int32_t*)(ws + L.sorted);
  int32_t* block_expert = a->block_expert ? a->block_expert : (int32_t*)(ws + L.block_expert);
  int32_t* num_padded = a->num_padded ? a->num_padded : (int32_t*)(ws + L.num_padded);
  int32_t* active = (int32_t*)(ws + L.active);
  int32_t* num_active = (int32_t*)(ws + L.num_active);
  float* xamax_part = (float*)(ws + L.xamax_part);
  float* scale_slot = (float*)(ws + L.scale_slot);
  unsigned* h_amax = (unsigned*)(ws + L.h_amax);
  uint8_t* xq = ws + L.xq;
  uint8_t* xs_blk = ws + L.xs_blk;
  uint8_t* h = ws + L.h;
  float* part = (float*)(ws + L.part);
  const int64_t P = (int64_t)M * k;
  const int n_act = (int)std::min<int64_t>(E, P);

  AlignOut o{counts, offsets, sorted, block_expert, num_padded, active, num_active, L.n_blocks};
  if (prefill)
    return prefill_forward(a, st, ev, L, ws, ids, wts, o, xamax_part, scale_slot, h_amax, xq, h, part, hdyn, S);
  if (l1_wks) {
    int cus = 0;
    if ((rc = persistent_wgs(&cus)) != MOE_OK) return rc;
    // one workgroup per item of the larger product, at most one per CU (two
    // per CU measured slower: the barrier's cost grows with its workgroups)
    const int64_t items = (int64_t)n_act * std::max(I / 16, H / (32 * (4 / l1_wks)));
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(std::min(cus, kLayer1MaxGrid), items));
    Layer1Args la{};
    la.logits = a->logits;
    la.x = (const uint16_t*)a->x;
    la.M = M;
    la.E = Er;
    la.K = kr;
    la.S = S;
    la.H = H;
    la.I = I;
    la.w13 = (const uint8_t*)a->w13;
    la.w2 = (const uint8_t*)a->w2;
    la.w13_scale = a->w13_scale;
    la.w2_scale = a->w2_scale;
    la.w_cs = pc ? 1 : 0;
    la.w_es = a->weight_scale_mode == 2 ? 1 : 0;
    la.x_scale = a->x_scale;
    la.h_scale = a->h_scale;
    la.xq = xq;
    la.h = h;
    la.part = part;
    la.wg_hmax = (float*)(ws + L.wg_hmax);
    la.y = (uint16_t*)a->y;
    la.n_blocks = L.n_blocks;
    la.ids_out = a->topk_ids;
    la.wts_out = a->topk_weights;
    la.align_out = AlignOut{a->expert_counts, a->expert_offsets, a->sorted_ids, a->block_expert, a->num_padded,
                            nullptr, nullptr, L.n_blocks};
    la.scales_out = fp8 ? a->scales_out : nullptr;
    const int hf1 = !fp8 ? H_BF16 : (hdyn ? H_F32 : H_E4M3);
    rec(0);
    const hipError_t err = launch_layer1(fp8, hf1, l1_wks, grid, hdyn ? 16 * gemm2_lds_stride(I) : 0, st, la);
    for (int i = 1; i < 2 * MOE_NUM_STAGES; ++i) rec(i);
    if (err != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ERR_DEVICE;
    }
    return launch_status();
  }
  const bool small = P <= kSmallPairs && E <= kSmallMaxExperts && (!fp8 || (int64_t)M * H <= kSmallQuantElems);
  if (tiny) {
    const int hf = !fp8 ? H_BF16 : (hdyn ? H_F32 : H_E4M3);
    const int grid = (int)std::min<int64_t>((int64_t)n_act * (I / 16), kTinyGrid);
    Layer1Args la{};
    la.logits = a->logits;
    la.x = (const uint16_t*)a->x;
    la.M = M;
    la.E = Er;
    la.K = kr;
    la.S = S;
    la.H = H;
    la.I = I;
    la.w13 = (const uint8_t*)a->w13;
    la.w2 = (const uint8_t*)a->w2;
    la.w13_scale = a->w13_scale;
    la.w2_scale = a->w2_scale;
    la.w_cs = pc ? 1 : 0;
    la.w_es = a->weight_scale_mode == 2 ? 1 : 0;
    la.x_scale = a->x_scale;
    la.h_scale = a->h_scale;
    la.h = h;
    la.wg_hmax = (float*)(ws + L.wg_hmax);
    la.n_blocks = L.n_blocks;
    la.ids_out = ids;
    la.wts_out = wts;
    la.align_out = o;
    la.scales_out = fp8 ? a->scales_out : nullptr;
    la.sx_out = fp8 ? scale_slot : nullptr;
    rec(0);
    rec(1);
    rec(2);
    rec(3);
    rec(4);
    if (!launch_tiny_gate_up(fp8, hf, grid, st, la)) return MOE_ERR_UNSUPPORTED;
    rec(5);
    if ((rc = launch_status()) != MOE_OK) return rc;
    rec(6);
    DownTokArgs g{(const uint8_t*)a->w2, h, ids, wts, (uint16_t*)a->y, H, I, k, plan.tok_chunks, a->w2_scale};
    g.w_cs = pc ? 1 : 0;
    g.w_es = a->weight_scale_mode == 2 ? 1 : 0;
    g.h_scale = a->h_scale;
    g.h_amax = h_amax;
    g.x_scale = scale_slot;
    g.scales_out = fp8 ? a->scales_out : nullptr;
    if (hf == H_F32) {
      g.wg_hmax = (const float*)(ws + L.wg_hmax);
      g.n_wg = grid;
    }
    const size_t lds = hf == H_F32 ? (size_t)k * I : 0;
    if (!launch_down_token(fp8, hf, plan.u2, dim3((unsigned)(H / 16), (unsigned)M), lds, st, g))
      return MOE_ERR_UNSUPPORTED;
    rec(7);
    rec(8);
    rec(9);
    return launch_status();
  }
  if (small) {
    // 1+2. routing, align (and fp8 activation quantisation) in one workgroup
    rec(0);
    SmallQuant q{(const uint16_t*)a->x, H, a->x_scale, fp8 ? xq : nullptr, scale_slot, hdyn ? h_amax : nullptr,
                 blk ? xs_blk : nullptr};
    launch_prologue_small(a->logits, M, Er, kr, S, ids, wts, kAlignBlockFused, o, q, st);
    rec(1);
    rec(2);
    rec(3);
    if ((rc = launch_status()) != MOE_OK) return rc;
  } else {
    // 1. routing (+ per-workgroup amax of x)
    rec(0);
    // the routing workgroups' expert counts serve the multi-workgroup align
    int32_t* hist = (P > kSmallPairs && hist_usable(k)) ? (int32_t*)(ws + L.hist) : nullptr;
    RouteFusedArgs fa{(const uint16_t*)a->x, H, (fp8 && !blk && !a->x_scale) ? xamax_part : nullptr,
                      hdyn ? h_amax : nullptr, hist};
    launch_route(a->logits, M, Er, kr, S, ids, wts, fa, st);
    rec(1);
    if ((rc = launch_status()) != MOE_OK) return rc;

    // 2. align (+ activation quantisation in fp8 mode)
    rec(2);
    QuantXArgs q{};
    int n_quant = 0;
    if (fp8) {
      q.x = (const uint16_t*)a->x;
      q.n = (int64_t)M * H;
      q.amax_part = xamax_part;
      q.n_part = L.n_route_wg;
      q.static_scale = a->x_scale;
      q.xq = xq;
      q.scale_slot = scale_slot;
      q.xs = blk ? xs_blk : nullptr;
      n_quant = (int)cdiv(q.n, kAlignQuantPerWg);
    }
    if (P <= kSmallPairs) {  // one 1024-thread align workgroup, 16K-element quantising workgroups
      const unsigned g = 1 + (fp8 ? (unsigned)cdiv(q.n, kSmallQuantPerWg) : 0u);
      align_small_kernel<<<g, 1024, 0, st>>>(ids, (int)P, E, log2i(kAlignBlockFused), log2i(E), o, q);
    } else {
      launch_align(ids, P, E, kAlignBlockFused, o, q, n_quant, st,
                   AlignHist{hist, (int)cdiv(M, 4 * kRouteRows), hist ? 16 / k : 0});
    }
    rec(3);
    if ((rc = launch_status()) != MOE_OK) return rc;
  }

  const Segments segs{sorted, offsets, counts, active, num_active, plan.rev};
  const int hf = !fp8 ? H_BF16 : (hdyn ? H_F32 : H_E4M3);

  // 3. gate/up product + SiLU(gate)*up
  rec(4);
  {
    Gemm1Args g{(const uint8_t*)a->w13, fp8 ? xq : (const uint8_t*)a->x, segs, H, I, k, a->w13_scale, scale_slot,
                a->h_scale, h, h_amax};
    g.w_cs = pc ? 1 : 0;
    g.w_es = a->weight_scale_mode == 2 ? 1 : 0;
    g.w_bs = blk ? 1 : 0;
    g.w_block = blk ? (const uint8_t*)a->w13_scale : nullptr;
    g.x_block = xs_blk;
    DecodeShape sh{plan.nt1, plan.u1, plan.ks1, plan.tw1, dim3(), 0, plan.ft1};
    sh.grid = plan.tw1 > 0
                  ? dim3((unsigned)cdiv(I / 16, 4 * plan.tw1), (unsigned)n_act, (unsigned)plan.passes1)
                  : dim3((unsigned)(I / 16 / (plan.ft1 * 4 / plan.ks1)), (unsigned)n_act, (unsigned)plan.passes1);
    const bool ok = fp8 ? launch_gemm1_fp8(hdyn ? H_F32 : H_E4M3, sh, st, g) : launch_gemm1_bf16(sh, st, g);
    if (!ok) return MOE_ERR_UNSUPPORTED;
  }
  rec(5);
  if ((rc = launch_status()) != MOE_OK) return rc;

  // 4+5 for small layers: the down product with the weighted combine, one
  // workgroup per (16 output rows, token)
  if (plan.tok) {
    rec(6);
    DownTokArgs g{(const uint8_t*)a->w2, h, ids, wts, (uint16_t*)a->y, H, I, k, plan.tok_chunks, a->w2_scale};
    g.w_cs = pc ? 1 : 0;
    g.w_es = a->weight_scale_mode == 2 ? 1 : 0;
    g.h_scale = a->h_scale;
    g.h_amax = h_amax;
    g.x_scale = scale_slot;
    g.scales_out = fp8 ? a->scales_out : nullptr;
    const size_t lds = hf == H_F32 ? (size_t)k * I : 0;
    if (!launch_down_token(fp8, hf, plan.u2, dim3((unsigned)(H / 16), (unsigned)M), lds, st, g))
      return MOE_ERR_UNSUPPORTED;
    rec(7);
    rec(8);
    rec(9);
    return launch_status();
  }

  // 4. down product (partial sums per K slice)
  rec(6);
  {
    Gemm2Args g{(const uint8_t*)a->w2, h, segs, wts, H, I, k, plan.ks2, a->w2_scale, a->h_scale, h_amax, part,
                (int)P};
    g.w_cs = pc ? 1 : 0;
    g.w_es = a->weight_scale_mode == 2 ? 1 : 0;
    g.w_bs = blk ? 1 : 0;
    g.w_block = blk ? (const uint8_t*)a->w2_scale : nullptr;
    DecodeShape sh{plan.nt2, plan.u2, plan.wks2, plan.tw2, dim3(), (size_t)(hf == H_F32 ? plan.lds2 : 0), plan.fr2};
    sh.grid = plan.tw2 > 0
                  ? dim3((unsigned)cdiv(H / 32, 4 * plan.tw2), (unsigned)n_act, (unsigned)(plan.ks2 * plan.passes2))
                  : dim3((unsigned)(H / (32 * (plan.fr2 * 4 / plan.wks2))), (unsigned)n_act,
                         (unsigned)(plan.ks2 * plan.passes2));
    const bool ok = fp8 ? launch_gemm2_fp8(hf, sh, st, g) : launch_gemm2_bf16(sh, st, g);
    if (!ok) return MOE_ERR_UNSUPPORTED;
  }
  rec(7);
  if ((rc = launch_status()) != MOE_OK) return rc;

  // 5. y = bf16(sum_j w_j * sum_s part_s), fixed order
  rec(8);
  {
    const int64_t groups = (int64_t)M * H / 4;
    const int lkp = log2i(k);
    float* so = fp8 ? a->scales_out : nullptr;
    // block-scaled: no tensor scales; both reported scales read the slot
    // that the quantisation set to 0
    const float* hs = blk ? scale_slot : a->h_scale;
    // four groups per lane once that still leaves at least 256 workgroups
    if ((groups << lkp) >= (int64_t)4 * 256 * 256)
      finalize_kernel<4><<<(unsigned)cdiv((groups / 4) << lkp, 256), 256, 0, st>>>(
          part, wts, (uint16_t*)a->y, M, H, k, lkp, plan.ks2, scale_slot, h_amax, hs, so);
    else
      finalize_kernel<1><<<(unsigned)cdiv(groups << lkp, 256), 256, 0, st>>>(
          part, wts, (uint16_t*)a->y, M, H, k, lkp, plan.ks2, scale_slot, h_amax, hs, so);
  }
  rec(9);
  return launch_status();
}

moe_status_t moe_fused_forward(const moe_fused_args_t* args, void* stream) {
  return fused_forward(args, (hipStream_t)stream, nullptr);
}

moe_status_t moe_fused_forward_profiled(const moe_fused_args_t* args, void* stream, void* const* events) {
  return fused_forward(args, (hipStream_t)stream, events);
}

moe_status_t moe_fused_path(const moe_fused_args_t* args, int32_t* path) {
  if (!path) return MOE_ERR_INVALID_ARG;
  return fused_forward(args, nullptr, nullptr, false, path);
}

moe_status_t moe_fused_forward_noalloc(const moe_fused_args_t* args, void* stream) {
  return fused_forward(args, (hipStream_t)stream, nullptr, true);
}

}  // extern "C"
