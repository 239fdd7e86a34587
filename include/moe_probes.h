/*
 * moe_probes.h -- C ABI of the measurement probes (libmoe_probes.so).
 *
 * Not part of the layer: small kernels that measure what an MI355X
 * delivers for the resources the fused MoE layer is bound by, so that its
 * roofline fractions can be read against achieved as well as nameplate
 * ceilings, and the summation precision of the fp8 matrix instructions that
 * the fp8 layer's tolerance rests on, and what publishing partial results
 * across XCDs inside a kernel costs.  The layer's decode products stream
 * expert weights from HBM and its prefill products run on the fp8 matrix
 * cores (wagnersolution, "AWS describes a fused MoE optimization for the
 * NVIDIA Hopper architecture", body: the fused kernel's throughput and
 * latency goals; "Fused MoE on Hopper, ...", TL;DR: FP8 experts).
 *
 * Conventions as in moe.h: device pointers owned by the caller, `stream` a
 * hipStream_t as void* (NULL = default stream), arguments checked on the
 * host before anything is enqueued (MOE_ERR_INVALID_ARG, nothing enqueued),
 * MOE_ERR_DEVICE when the launch fails.  The caller times a probe with HIP
 * events recorded on the same stream around the call.
 */
#ifndef MOE_MI355X_PROBES_H
#define MOE_MI355X_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ABI version of this header. */
int32_t moe_probes_abi_version(void);

/* Streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a
 * multiple of 16) by `grid` workgroups of 256 threads (1..2^20), each thread
 * reading 16-byte words with four loads in flight, grid-stride.  Writes
 * sink[g] (uint32 [grid]) = XOR of all 32-bit words that workgroup g read,
 * so every load is live; the XOR of sink over all g is the XOR of the whole
 * buffer.  Achieved read bandwidth = bytes / the call's duration; a buffer
 * well above the 256 MB last-level cache measures HBM. */
moe_status_t moe_probe_hbm_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, void* stream);

/* fp8 matrix-core issue rate: `grid` workgroups of four waves (1..2^20),
 * every wave running `iters` rounds (1..2^20) of four independent
 * 32x32x64 e4m3 MFMAs (the prefill products' instruction) on register
 * operands with unit scales.  random_operands 0: every operand 1.0, so each
 * round adds 64 to every accumulator element; 1: fixed pseudo-random e4m3
 * bytes per lane (no NaN codes), the same every round, whose bit switching
 * draws power as real data does (the clock the hardware then holds is lower).
 * Lane 0 of wave w writes out[4w + j] = the first element of accumulator j:
 * 64 * iters (exact up to 2^24) with operands 1.0, else iters times the
 * one-round value up to fp32 accumulation.  out: fp32 [grid * 4 * 4].
 * Other random_operands values: MOE_ERR_INVALID_ARG.  Achieved rate =
 * grid * 4 waves * iters * 4 * 2*32*32*64 flops / the call's duration. */
moe_status_t moe_probe_mfma_fp8_loop(float* out, int32_t grid, int32_t iters, int32_t random_operands,
                                     void* stream);

/* One wave: C[r][c] = c0 + 2^(sa-127) * 2^(sb-127) * sum over k < 128 of
 * A[r][k] * B[c][k], for e4m3 codes A, B [16][128] row-major (16-byte
 * aligned) and fp32 C [16][16], as the fp8 matrix instructions compute it:
 * form 0 = one 16x16x128 block-scaled MFMA (sa, sb: E8M0 codes 0..254);
 * form 1 = four 16x16x32 MFMAs accumulating in order (unit scales only, sa
 * and sb must be 127).  Comparing C with the exact sum shows the
 * instructions' own summation precision. */
moe_status_t moe_probe_fp8_dot(const uint8_t* A, const uint8_t* B, float* C, int32_t sa, int32_t sb, float c0,
                               int32_t form, void* stream);

/* The cost of publishing partial results to workgroups on other XCDs inside
 * one kernel (each XCD has its own L2, not kept coherent with the others
 * within a kernel), as a last-arriver combine would need: `grid` workgroups
 * (1..2^20) each write 32 KB, buf[8192*g + i] = g + i for i < 8192 (buf: fp32
 * [grid * 8192], 16-byte aligned), and then add one to cnt[g % 1024] (cnt:
 * uint32 [1024], caller-zeroed; after the call it holds the number of
 * workgroups that counted themselves in at each slot).  mode 0: plain
 * stores; 1: plain stores and an agent-scope release fence (an L2
 * writeback) before the count; 2: write-through stores (agent-scope atomic
 * stores) completed before the count.  Other modes: MOE_ERR_INVALID_ARG.
 * The caller times the call with events. */
moe_status_t moe_probe_publish(float* buf, uint32_t* cnt, int32_t grid, int32_t mode, void* stream);

/* The operand stream of the tiled prefill product without its arithmetic,
 * to tell the load path's limits from the product's: `grid` workgroups
 * (1..65536) of 256 threads each walk `steps` K-steps (3..2^20, a multiple
 * of 3) of 128 bytes over 384 rows of a [bytes/4096][4096] byte matrix (256
 * weight rows, 128 token rows; the next 384 rows every 32 steps, wrapping
 * within the buffer), each step's 48 KB landing in a three-slot LDS ring two
 * steps ahead of its use with one barrier per step.  mode 0: direct-to-LDS
 * buffer loads; 1: the same loads into registers, then 16-byte LDS stores;
 * 2: mode 0 plus the product's LDS fragment reads (24 KB per wave per step,
 * swizzled as the product's).  Added to mode: 4 = each workgroup starts its
 * tiles at K-step g % 32 (the operands' addresses then differ between
 * workgroups in their low 12 bits); 8 = rows 4224 bytes apart instead of
 * 4096; 16 = every workgroup keeps its first tile and alternates between
 * its first two K-steps (96 KB per workgroup, re-read from L2); 32 (modes 0
 * and 2) = 256 token rows per step (64 KB, 512 rows per tile) in a two-slot
 * ring, loads one step ahead; 64 (modes 0 and 2, no other flag) = 256 token
 * rows and 64-byte K-steps (32 KB, half a line of each row) in a four-slot
 * ring, loads three steps ahead.  buf at least 512 * 4224 bytes.  buf: bytes a multiple of 4096, from 384*4224 to 2^30 (a buffer below the
 * L2 size stays there; one far above the last-level cache streams from
 * HBM).  sink: uint32 [grid * 4], each wave's XOR of what it read.  Other
 * arguments: MOE_ERR_INVALID_ARG.  The caller times the call with events:
 * bytes moved = grid * steps * 48 KB. */
moe_status_t moe_probe_ring_load(const void* buf, size_t bytes, int32_t grid, int32_t steps, int32_t mode,
                                 uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_PROBES_H */
