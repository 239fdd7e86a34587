/*
 * moe.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts layer.
 *
 * The layer, as the web pages on the subject describe it, combines token
 * routing, the movement of tokens to their experts and the expert computation
 * into one batched GPU operation (wagnersolution, "AWS describes a fused MoE
 * optimization for the NVIDIA Hopper architecture", body), with scaling, the
 * matrix products and the aggregation of expert outputs fused rather than
 * round-tripped through HBM (The Neural Net, "AWS details MoE kernel fixes
 * for SageMaker ...", body), in bf16 or with FP8 tensor-quantised experts
 * ("Fused MoE on Hopper, ...", TL;DR).  The pages give no formulas; the
 * operations below state the definitions this library implements.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless stated otherwise.  Every buffer is
 *    owned by the caller; the library allocates no device memory, keeps no
 *    per-call state and is re-entrant.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    All work is enqueued on it in order; outputs are valid once the stream
 *    reaches the call.  Inputs are never written.
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    error nothing is enqueued and the error code is returned.
 *    MOE_ERR_INVALID_ARG: a required pointer is NULL, a size is negative,
 *    top_k < 1 or top_k > E, a pointer is misaligned (16 bytes for tensors,
 *    4 bytes for scalars), or a scale pointer is given in bf16 mode.
 *    MOE_ERR_UNSUPPORTED: a shape outside the built envelope
 *    (E <= 512, top_k <= 16, H and I multiples of 128, block a power of two
 *    in [1, 256], M*top_k < 2^31).
 *    MOE_ERR_WORKSPACE_TOO_SMALL: workspace_bytes below the required size.
 *    MOE_ERR_DEVICE: a launch failed (hipGetLastError after the launch).
 *  - M = 0 is valid: route, router logits and the fused forward enqueue
 *    nothing; align writes the empty layout.
 *  - Kernels are compiled ahead of time for gfx950; no argument value
 *    (token count included) triggers a compilation.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The *_RANGE_ enumerators are not values of their type: they give each
 * enumeration the range of int32_t, so that any int a C caller passes is a
 * valid value of the type on the C++ side (the library rejects unknown ones
 * with MOE_ERR_INVALID_ARG). */
typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_DEVICE = 4,
  MOE_STATUS_RANGE_LO_ = -2147483647 - 1,
  MOE_STATUS_RANGE_HI_ = 2147483647
} moe_status_t;

typedef enum {
  MOE_DTYPE_BF16 = 0,
  MOE_DTYPE_FP8_E4M3 = 1,
  MOE_DTYPE_RANGE_LO_ = -2147483647 - 1,
  MOE_DTYPE_RANGE_HI_ = 2147483647
} moe_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status_t status);

/* ABI version of this header; bumped on any incompatible change. */
int32_t moe_abi_version(void);

/*
 * Router top-k ("token routing", wagnersolution page, body; the decode batch
 * holds one token per sequence, M = 1..63 in the pages' flowchart).
 * For every token m (row of `logits`, fp32 [M,E] row-major): the top_k
 * largest logits, in decreasing order; equal logits go to the lower expert
 * index, and -0.0 equals +0.0.  topk_ids int32 [M,top_k] receives the
 * experts, topk_weights fp32 [M,top_k] the softmax over the selected logits
 * (equal to the softmax over all E renormalised over the selection).
 * Logits must be finite (otherwise the selection is unspecified).
 */
moe_status_t moe_route_topk(const float* logits, int32_t M, int32_t E, int32_t top_k, int32_t* topk_ids,
                            float* topk_weights, void* stream);

/*
 * Host-only: length of `sorted_ids` needed by moe_align, in elements:
 * P + min(E,P)*(block-1) rounded up to a multiple of block, P = M*top_k
 * (every expert that holds a pair adds at most block-1 padding entries).
 * Returns 0 for invalid arguments.  block_expert needs capacity/block entries.
 */
size_t moe_align_capacity(int32_t M, int32_t top_k, int32_t E, int32_t block);

/*
 * Sort and pad (the "data transfers" step between routing and the expert
 * products, wagnersolution page, body): groups the P = M*top_k pairs
 * f = m*top_k + j by expert so that each expert's tokens form one contiguous,
 * tile-aligned operand.
 *   expert_counts  int32 [E]   pairs routed to each expert
 *   expert_offsets int32 [E+1] exclusive prefix sum of ceil(count/block)*block
 *   sorted_ids     int32 [capacity]  for each expert, its pair indices in
 *                  increasing f, then the sentinel P up to the padded length;
 *                  entries at or beyond num_padded are left unwritten
 *   block_expert   int32 [capacity/block] expert of each block, -1 for blocks
 *                  at or beyond num_padded/block
 *   num_padded     int32 [1]  sum of the padded lengths; -1 if an id was
 *                  outside [0,E) (such ids are ignored, never dereferenced)
 * The result is deterministic (no dependence on scheduling).
 */
moe_status_t moe_align(const int32_t* topk_ids, int32_t M, int32_t top_k, int32_t E, int32_t block,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_ids,
                       int32_t* block_expert, int32_t* num_padded, void* stream);

/*
 * Per-tensor FP8 quantisation of an fp32 vector with a given scale:
 * out[i] = e4m3(saturate(in[i] * fp32(1/scale))), OCP E4M3FN (max 448),
 * round to nearest even, magnitudes above 448 clamp to 448.
 * scale: device pointer to one fp32 (> 0).  This is the conversion the fused
 * forward applies to its activations ("FP8 tensor-quantized" MoE, "Fused MoE
 * on Hopper, ..." TL;DR; The Neural Net page, the facts).
 */
moe_status_t moe_quant_e4m3(const float* in, int64_t n, const float* scale, uint8_t* out, void* stream);

/*
 * Router logits, the step before routing: logits[m,e] = sum_t x[m,t] *
 * router_w[e,t] with fp32 accumulation in a fixed order (the same bits on
 * every call and for every M).  The pages' fused operation starts from the
 * tokens: routing, data movement and expert computation in one batched GPU
 * operation (wagnersolution page, "AWS describes a fused MoE optimization for
 * the NVIDIA Hopper architecture", body).
 *   x         [M,H] bf16, 16-byte aligned
 *   router_w  [E,H] bf16, 16-byte aligned
 *   logits    [M,E] fp32 out
 * H a multiple of 128, E <= 512.  M = 0 is a no-op.  Errors: MOE_ERR_INVALID_ARG
 * (null or misaligned pointers, M < 0, E < 1), MOE_ERR_UNSUPPORTED (E > 512,
 * H not a multiple of 128).
 */
moe_status_t moe_router_logits(const void* x, const void* router_w, int32_t M, int32_t E, int32_t H, float* logits,
                               void* stream);

/*
 * Optional tuning of the fused forward; NULL selects the built-in table.
 * Any field 0 keeps its default; negative values are invalid except where
 * stated.  Values outside the supported set return MOE_ERR_UNSUPPORTED.
 *
 * Each product of the decode path (fewer than 8192 pairs, or bf16) has two
 * variants: the K-split variant (one 16-feature or 32-row tile per wave, K
 * split over the waves of a workgroup) and the long-stream variant (each wave
 * walks several tiles over the whole K range, its load pipeline running from
 * tile to tile).
 */
typedef struct {
  int32_t gemm1_ksplit;      /* K-split gate/up: waves of a workgroup splitting K: 1, 2 or 4 */
  int32_t gemm2_ksplit;      /* K slices of the down product in separate workgroups: 1..16, within the
                                workspace's partial-sum capacity */
  int32_t token_tiles;       /* 16-token tiles held per pass, both products: 1..4 */
  int32_t unroll;            /* MFMA K-steps per pipeline stage, both products: bf16 2 or 4, fp8 1 or 2 */
  int32_t gemm2_wave_ksplit; /* K-split down: waves of a workgroup splitting K: 1, 2 or 4 */
  int32_t gemm1_stream_tiles; /* gate/up: > 0 long-stream variant with this many feature tiles per wave
                                 (1..16), < 0 K-split variant */
  int32_t gemm2_stream_tiles; /* down: > 0 long-stream variant with this many row tiles per wave (1..16),
                                 < 0 K-split variant */
  int32_t reverse_order;     /* both products: 1 = take the grid's expert and token-pass indices in reverse
                                (the last experts' and late passes' workgroups first), -1 = in order;
                                default: reversed with shared experts, which then also take the K-split
                                variants unless the stream fields say otherwise */
  int32_t single_launch;     /* 1 = the whole layer in one launch (tiny token counts: at most 16 tokens
                                and 64 pairs, at most 256 routed experts, given logits, default mode;
                                MOE_ERR_UNSUPPORTED where it does not fit); 0 or -1 = the multi-launch
                                path (default: on MI355X a grid barrier costs about as much as the kernel
                                boundary it replaces).  Single-launch calls on one GPU must not overlap
                                (they share the barrier's device counters) */
  int32_t down_per_token;    /* layers of at most 64 pairs M*(top_k+S): 1 = the down product and the
                                weighted combine as one launch, a workgroup per (16 output rows, token)
                                summing the token's pairs in a fixed order (MOE_ERR_UNSUPPORTED where it
                                does not fit: deterministic or block-scaled mode, more pairs, or a dynamic
                                fp8 h scale with (top_k+S)*I above 64 KB); -1 = the per-expert down
                                product and the finalize; 0 = default: per token where it fits and the
                                tokens that share an expert would not re-read much of its W2 (always at
                                M = 1; small experts up to 64 pairs), unless a down-product field
                                (gemm2_ksplit, gemm2_wave_ksplit, gemm2_stream_tiles, gemm2_row_tiles) is
                                set */
  int32_t routing_in_gate_up; /* tiny layers taking the per-token down product (at most 16 tokens and 64
                                pairs, at most 256 routed experts, H a multiple of 512 in fp8 or of 128 in
                                bf16, fp8 x of at most 16384 elements, not the single-launch layer): 1 = the
                                layer in two launches, every gate/up workgroup routing, quantising and
                                sorting the few tokens itself before its items (MOE_ERR_UNSUPPORTED where
                                the layer would take another path); -1 = the routing launch of its own;
                                0 = default: two launches where it fits and the gate/up product has at
                                most 1024 items of 16 features (min(E+S, M*(top_k+S)) * I/16), or at most
                                4096 items of at most 64 KB (32 weight rows of H), unless a
                                gate/up field (gemm1_ksplit, token_tiles, unroll, gemm1_stream_tiles,
                                gemm1_feature_tiles) is set.  The
                                outputs are those of the routing launch of its own, bit for bit, wherever
                                that path's gate/up product splits K over four waves (bf16; fp8 below 8
                                tokens) */
  int32_t gemm1_feature_tiles; /* K-split gate/up: 16-feature groups per wave, 1 or 2 (2: the workgroup
                                covers twice the features and reads each token row once for both, half
                                the token-row reads per weight byte; same results bit for bit); 0 =
                                default: 2 for bf16 layers whose gate/up grid keeps at least 2048
                                workgroups with two (then with unroll 2 for the gate/up product unless
                                unroll is given), else 1 */
  int32_t gemm2_row_tiles;   /* K-split down: 32-row groups per wave, 1 or 2 (2 only where H divides into
                                the workgroup's 32*2*4/gemm2_wave_ksplit rows and the K-split reduction
                                buffer fits the workgroup's LDS): the same results bit for bit with the same
                                K slices (the default slice count follows the number of workgroups, which
                                two groups halve); 0 = default: 2 for bf16 layers with at least 12 pairs
                                per expert that can hold tokens (M*(top_k+S) >= 12*min(E+S, M*(top_k+S))),
                                where it fits, else 1 */
} moe_tuning_t;

/*
 * The fused layer, all in one stream-ordered call:
 *   route (as moe_route_topk) -> align (as moe_align, block 16) ->
 *   for each pair (m,j) with expert e = topk_ids[m,j]:
 *     g = W13[e][0:I] . a_m,  u = W13[e][I:2I] . a_m       (fp32 accumulation)
 *     h = SiLU(g) * u,  SiLU(g) = g / (1 + exp(-g))
 *     o = W2[e] . h
 *   y[m] = bf16( sum_j topk_weights[m,j] * o_(m,j) )        (fp32 accumulation)
 * bf16 mode: a_m = x[m]; h is rounded to bf16 before the second product.
 * fp8 mode: a_m = e4m3(x[m] / s_x) and hq = e4m3(h / s_h) (moe_quant_e4m3's
 * rounding); the products are rescaled by s_x*s_w13 and s_h*s_w2.  s_x and
 * s_h are the caller's static scales when given, else amax/448 over all of x
 * and over h of all pairs (1.0 when the amax is 0).  The weight scales
 * (weight_scale_mode) are one per tensor (0: s_w13 = w13_scale[0]), one per
 * weight row (1, output channel: row n of W13[e], a gate or up feature, is
 * rescaled by w13_scale[e*2I + n] and row n of W2[e], an output feature, by
 * w2_scale[e*H + n]) or one per expert (2: every row of W13[e] by
 * w13_scale[e], of W2[e] by w2_scale[e]) (the pages name tensor-quantised FP8 experts and routing among
 * quantisation schemes: "Fused MoE on Hopper, ...", TL;DR; ZICQ, "AWS Unveils
 * MoE Kernel Optimizations ...", §Triton Backend Routing for FP8
 * Quantization).
 * Block-scaled fp8 (weight_scale_mode 3; the pages name routing among
 * quantisation schemes, ZICQ page, §Triton Backend Routing for FP8
 * Quantization): w13_scale and w2_scale then point to uint8 E8M0 codes (the
 * OCP microscaling scale format, value 2^(c-127)), one per 128 x 128 block:
 * [E+S][2I/128][H/128] for W13 and [E+S][H/128][I/128] for W2; every weight
 * is its e4m3 value times its block's scale.  Activations take one
 * power-of-two scale per 128 consecutive elements of a token's x row and of
 * a pair's h row, chosen by the OCP microscaling rule for E4M3 elements
 * (code = max(biased exponent of the group's amax - 8, 0)), each element
 * rounded to e4m3 after division by it; x_scale and h_scale must be NULL
 * (else MOE_ERR_INVALID_ARG) and scales_out reports 0, 0.  The scales go
 * into the scaled MFMA with the operands.  The decode products serve every M
 * in this mode (the K-split variants; tunings asking for a long-stream
 * variant return MOE_ERR_UNSUPPORTED); a token's output does not depend on
 * the rest of its batch.
 * Shared experts (n_shared = S > 0; the pages do not describe them, and here
 * they are the plain form): every token also passes through experts
 * E..E+S-1, stacked after the routed ones in w13/w2 (and in per-row scales),
 * with weight one.  From the routing on they are S more experts and S more
 * slots per token: the sums above run over j < top_k+S, slot top_k+s of
 * token m holds expert E+s with weight 1, s_h covers their h too, and
 * topk_ids/topk_weights are [M,top_k+S], expert_counts [E+S].  Size the
 * workspace with moe_fused_workspace_size(M, E+S, H, I, top_k+S, dtype).
 * top_k+S <= 16 and E+S <= 512, else MOE_ERR_UNSUPPORTED.
 * The expert products put expert-weight rows in the wide MFMA operand and
 * the few tokens in the narrow one; at decode sizes this is the orientation
 * the pages call Swap-AB (B^T A^T instead of A B, "Fused MoE on Hopper, ..."
 * TL;DR and flowchart; wagnersolution page, body).
 */
typedef struct {
  int32_t M, E, H, I, top_k;
  moe_dtype_t dtype;
  const void* x;           /* [M,H] bf16 hidden states */
  const float* logits;     /* [M,E] fp32 router logits, or NULL with router_w */
  const void* w13;         /* [E+S,2I,H] bf16 or e4m3; rows [0,I) gate, [I,2I) up */
  const void* w2;          /* [E+S,H,I] bf16 or e4m3 */
  const float* w13_scale;  /* fp8: device fp32[1], fp32[(E+S)*2I] per row (16-byte aligned) or fp32[E+S] per
                              expert; bf16: NULL */
  const float* w2_scale;   /* fp8: device fp32[1], fp32[(E+S)*H] per row (16-byte aligned) or fp32[E+S] per
                              expert; bf16: NULL */
  const float* x_scale;    /* fp8: NULL = dynamic, else device fp32[1]; bf16: NULL */
  const float* h_scale;    /* fp8: NULL = dynamic, else device fp32[1]; bf16: NULL */
  void* y;                 /* [M,H] bf16 output (overwritten) */
  int32_t* topk_ids;       /* optional out [M,top_k+S]; NULL = kept in the workspace */
  float* topk_weights;     /* optional out [M,top_k+S] */
  int32_t* expert_counts;  /* optional out [E+S] */
  float* scales_out;       /* optional out fp32[2]: s_x, s_h used (fp8 only) */
  void* workspace;         /* device scratch, 256-byte aligned */
  size_t workspace_bytes;
  const moe_tuning_t* tuning; /* host pointer or NULL */
  int32_t weight_scale_mode; /* fp8: 0 = one scale per weight tensor, 1 = one per weight row, 2 = one per
                                expert, 3 = block-scaled (below); any other value, or non-zero in bf16
                                mode: MOE_ERR_INVALID_ARG */
  const void* router_w;    /* bf16 [E,H] router weights, 16-byte aligned, or NULL.  Exactly one of logits and
                              router_w is non-NULL (else MOE_ERR_INVALID_ARG); with router_w the layer first
                              computes logits = x . router_w^T as moe_router_logits does and routes on them */
  float* logits_out;       /* optional out [M,E]: the logits computed from router_w (NULL = kept in the
                              workspace); must be NULL when logits is given */
  int32_t n_shared;        /* S >= 0 shared experts after the E routed ones (see above); < 0: INVALID_ARG */
  /* Optional outputs of the call's sort-and-pad step (NULL = kept in the
   * workspace), in moe_align's layout for the block and capacity that
   * moe_fused_align_shape reports for the call (E and top_k counting the
   * shared experts): expert_offsets [E+S+1], sorted_ids [capacity] (entries
   * at or beyond *num_padded unspecified), block_expert [capacity/block],
   * num_padded [1].  The layer reads them back, so they must not alias any
   * other argument. */
  int32_t* expert_offsets;
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* num_padded;
  /* 1 = deterministic mode: a token's outputs (routing, weights and y) are
   * the same bits whatever the batch it is in and its position there, on
   * every call and in every process (the pages report a serving process and
   * a separate rescoring process agreeing to the bit once the kernel
   * configurations were pinned: "Fused MoE on Hopper, ...", TL;DR and key
   * points).  The order of every sum is then fixed by the shape alone:
   * the decode products run at every M (no switch to the prefill products),
   * with the gate/up K split over a fixed number of waves and the down
   * product in one K slice.  fp8 layers need static activation scales
   * (x_scale and h_scale non-NULL; a dynamic scale is an amax over the
   * batch), else MOE_ERR_INVALID_ARG; so do tunings that set a K split or a
   * long-stream variant whose sum order differs.  0 = default. */
  int32_t deterministic;
} moe_fused_args_t;

/* Host-only: workspace bytes needed by moe_fused_forward for these sizes (in
 * either mode). */
size_t moe_fused_workspace_size(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, moe_dtype_t dtype);

/* Host-only: block size and sorted_ids capacity of the sort-and-pad step of
 * moe_fused_forward for these sizes and modes (E and top_k counting shared
 * experts, as for moe_fused_workspace_size; deterministic and
 * weight_scale_mode as in moe_fused_args_t): block 128 on the prefill path
 * (fp8, M*top_k >= 8192, not deterministic, not block-scaled), else 16;
 * capacity as moe_align_capacity.  Errors as moe_fused_forward's shape
 * checks, and MOE_ERR_INVALID_ARG for unknown modes or NULL outputs. */
moe_status_t moe_fused_align_shape(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, moe_dtype_t dtype,
                                   int32_t deterministic, int32_t weight_scale_mode, int32_t* block,
                                   int64_t* capacity);

moe_status_t moe_fused_forward(const moe_fused_args_t* args, void* stream);

/*
 * Profiling support: when `events` (host array of hipEvent_t, passed as
 * void*) is non-NULL, moe_fused_forward_profiled records events[2*s] before
 * and events[2*s+1] after each of its MOE_NUM_STAGES launches on `stream`
 * (stage order: route (preceded by the router logits product when router_w is
 * given), align, gate/up product, down product, finalize).
 * A stage that is not launched still records both events back to back.
 * NULL entries of `events` are skipped, so a caller can time only the stages
 * it needs without adding markers between the others.
 */
#define MOE_NUM_STAGES 5
moe_status_t moe_fused_forward_profiled(const moe_fused_args_t* args, void* stream, void* const* events);

/*
 * The launch sequence a moe_fused_forward call on `args` takes.  Its stage
 * events (moe_fused_forward_profiled) bracket these launches:
 *   MOE_PATH_NONE               M = 0: nothing is launched
 *   MOE_PATH_PREFILL            tiled prefill products: route, align with the
 *                               x quantisation, gate/up, down (preceded in its
 *                               stage by the h quantisation with a dynamic fp8
 *                               h scale), finalize
 *   MOE_PATH_DECODE             route, align (one launch for both at most 1024
 *                               pairs), gate/up, down per expert, finalize
 *   MOE_PATH_DECODE_TOKEN_DOWN  as MOE_PATH_DECODE up to the gate/up product,
 *                               then the down product with the weighted
 *                               combine per token (its down stage; the
 *                               finalize stage is empty)
 *   MOE_PATH_TWO_LAUNCHES       the routing, sort-and-pad and gate/up product
 *                               in one launch (the gate/up stage; route and
 *                               align are empty), then the per-token down
 *                               product with the combine
 *   MOE_PATH_SINGLE_LAUNCH      the whole layer in one launch (the route
 *                               stage; the others are empty)
 * A given router_w adds its logits product at the start of the route stage.
 * The call validates `args` exactly as moe_fused_forward does, except that
 * y and the workspace may be NULL and the workspace size is not checked, and
 * returns the status moe_fused_forward would return before enqueuing
 * anything; *path is written on MOE_OK only.  It enqueues nothing, reads no
 * memory through the device pointers in `args` and needs no GPU.  path NULL:
 * MOE_ERR_INVALID_ARG.
 */
#define MOE_PATH_NONE 0
#define MOE_PATH_PREFILL 1
#define MOE_PATH_DECODE 2
#define MOE_PATH_DECODE_TOKEN_DOWN 3
#define MOE_PATH_TWO_LAUNCHES 4
#define MOE_PATH_SINGLE_LAUNCH 5
moe_status_t moe_fused_path(const moe_fused_args_t* args, int32_t* path);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the fused
 * layer exactly as moe_fused_forward computes it (same kernels, same plan,
 * same bits), with the workspace taken from a scratch array that the library
 * holds on each GPU it runs on, MOE_NOALLOC_SCRATCH_BYTES bytes, from the
 * first call on that GPU until the process ends.  args->workspace must be
 * NULL and args->workspace_bytes 0 (else MOE_ERR_INVALID_ARG); the caller
 * still passes every input and output.  Calls whose workspace would exceed
 * the array (the down product's partial sums are sized here for the plan's
 * K slices only; decode-sized layers fit, the fp8 prefill layer of 4096
 * tokens does not) return MOE_ERR_UNSUPPORTED before anything is enqueued.
 * The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  The first call on a GPU looks up the array's device address
 * (hipGetSymbolAddress); a failure there is MOE_ERR_DEVICE.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; nothing in it needs to start at zero.  Calls that overlap on one
 * GPU (other streams, other threads) race on the array: the caller must
 * order them, e.g. on one stream.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_fused_forward_noalloc(const moe_fused_args_t* args, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
