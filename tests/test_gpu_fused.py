"""GPU parity of the fused layer (moe_fused_forward) against the CPU oracle.

Every case checks: topk ids and per-expert counts bit-exact, topk weights
within 1e-6, the fp8 activation scale s_x bit-exact and s_h within 1e-4
(h differs by summation order), and the output within
max|y - y_ref| / max|y_ref| <= 1e-2 (bf16) or 3e-2 (fp8), y_ref being the
oracle's output before bf16 rounding.

Every case also checks the call's sort-and-pad outputs (counts, offsets,
sorted ids, block map, padded total) bit-exact against the oracle's align for
the call's block size, the output per token (max |dy_m| / max |y_ref_m|)
against the same bound, and canaries on both sides of every output.

Shapes: small layers that span several weight tiles, token tiles and token
passes with ragged tails, the tiny workload, and the four full-size workloads
at every token count of their sweeps.  Every output element of every case is
compared (the oracle evaluates all tokens, the M=4096 prefill layer
included).
"""
import numpy as np
import pytest
import torch

import moe_layer_align_amd as moe
import oracle
from gpu_common import DEV, TOL, compare, run_gpu, say
from synth import (CONFIGS, MoEConfig, gen_logits, gen_router_weights, gen_weights, gen_weights_block,
                   gen_weights_per_channel, gen_weights_per_expert, gen_x)

pytestmark = pytest.mark.gpu


def cfg_of(dtype, E, k, H, I, logits="normal"):
    return MoEConfig("small", E=E, k=k, H=H, I=I, dtype=dtype, ms=(1,), logits=logits)


# ---------------------------------------------------------------- small layers, whole output compared
@pytest.mark.parametrize("dtype,xs,hs", [("bf16", None, None), ("fp8", None, None), ("fp8", 0.02, 0.02)])
@pytest.mark.parametrize("M", [1, 5, 17, 40, 100, 600])
def test_small_layer(dtype, xs, hs, M):
    # M*k <= 1024 takes the one-workgroup prologue, M = 600 (1200 pairs) the router + align launches
    cfg = cfg_of(dtype, 6, 2, 512, 384)
    compare(cfg, M, seed=M, x_scale=xs, h_scale=hs)


# Routing inside the fused call: the one-workgroup prologue holds ceil(E/16)
# logits per lane (1, 2, 4, 8 or 16 keys, E <= 256), beyond that the
# multi-workgroup router; M spans several 64-token routing passes and ends
# with a partial wave of token rows.
@pytest.mark.parametrize("E,k", [(17, 3), (33, 5), (64, 8), (65, 2), (200, 8), (256, 16), (300, 4)])
def test_fused_routing_key_widths(E, k):
    compare(cfg_of("bf16", E, k, 256, 128), 61, seed=E)


def test_fused_one_workgroup_align_with_router():
    # fp8 with M*H above the prologue's quantisation limit but M*k <= 1024:
    # multi-workgroup router (x amax in fixed chunks), one-workgroup align
    # whose other workgroups quantise x
    compare(cfg_of("fp8", 64, 4, 4096, 128), 40, seed=21)
    compare(cfg_of("fp8", 64, 4, 4096, 128), 40, seed=22, x_scale=0.02, h_scale=0.02)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_single_expert_top1(dtype):
    compare(cfg_of(dtype, 1, 1, 256, 256), 9, seed=3)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_all_experts_selected(dtype):
    compare(cfg_of(dtype, 4, 4, 256, 128), 21, seed=4)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_many_tokens_one_expert(dtype):
    # every token picks expert 2 first: one expert holds 150 pairs (3 token passes)
    cfg = cfg_of(dtype, 5, 2, 256, 256)
    lg = gen_logits(cfg, 150, sub=150)
    lg[:, 2] += 100.0
    compare(cfg, 150, seed=5, logits=lg)


def test_max_experts_and_topk():
    compare(cfg_of("fp8", 512, 16, 256, 256), 11, seed=6)


def test_tuning_variants_agree():
    cfg = cfg_of("bf16", 8, 2, 1024, 512)
    w = gen_weights(cfg, 7, device=DEV)
    for t in [moe.Tuning(gemm1_ksplit=1, gemm2_ksplit=1, token_tiles=1, unroll=2, gemm2_wave_ksplit=4),
              moe.Tuning(gemm1_ksplit=2, gemm2_ksplit=4, token_tiles=2, unroll=4, gemm2_wave_ksplit=2),
              moe.Tuning(gemm1_ksplit=4, gemm2_ksplit=16, token_tiles=4, unroll=2, gemm2_wave_ksplit=1),
              moe.Tuning(gemm1_ksplit=4, gemm2_ksplit=2, token_tiles=3, unroll=2, gemm2_wave_ksplit=4),
              # long-stream variants in bf16
              moe.Tuning(gemm1_stream_tiles=3, gemm2_stream_tiles=5, token_tiles=2, unroll=2),
              moe.Tuning(gemm1_stream_tiles=1, gemm2_stream_tiles=16, token_tiles=4, unroll=4, gemm2_ksplit=4)]:
        compare(cfg, 33, seed=7, weights=w, tuning=t)
    cfg8 = cfg_of("fp8", 8, 2, 1024, 512)
    w8 = gen_weights(cfg8, 7, device=DEV)
    for t in [moe.Tuning(gemm1_ksplit=1, gemm2_ksplit=1, token_tiles=1, unroll=1, gemm2_wave_ksplit=4),
              moe.Tuning(gemm1_ksplit=2, gemm2_ksplit=2, token_tiles=2, unroll=2, gemm2_wave_ksplit=2),
              moe.Tuning(gemm1_ksplit=4, gemm2_ksplit=4, token_tiles=4, unroll=1, gemm2_wave_ksplit=1)]:
        compare(cfg8, 33, seed=7, weights=w8, tuning=t)
        compare(cfg8, 33, seed=7, weights=w8, tuning=t, x_scale=0.03, h_scale=0.02)
    # long-stream variants (fp8): tile counts that leave partial chunks and idle waves, K slices, unrolls
    for t in [moe.Tuning(gemm1_stream_tiles=1, gemm2_stream_tiles=1, token_tiles=1, unroll=1),
              moe.Tuning(gemm1_stream_tiles=3, gemm2_stream_tiles=5, token_tiles=2, unroll=2, gemm2_ksplit=2),
              moe.Tuning(gemm1_stream_tiles=16, gemm2_stream_tiles=16, token_tiles=4, unroll=1, gemm2_ksplit=4),
              moe.Tuning(gemm1_stream_tiles=-1, gemm2_stream_tiles=-1, token_tiles=4)]:
        compare(cfg8, 33, seed=7, weights=w8, tuning=t)
        compare(cfg8, 33, seed=7, weights=w8, tuning=t, x_scale=0.03, h_scale=0.02)


def test_m0_is_noop():
    cfg = cfg_of("bf16", 4, 2, 128, 128)
    w13, w2, _, _ = gen_weights(cfg, 0, device=DEV)
    y = moe.fused_forward(torch.empty(0, 128, dtype=torch.bfloat16, device=DEV),
                          torch.empty(0, 4, device=DEV), w13, w2, 2)
    assert y.shape == (0, 128)


def test_repeat_calls_reuse_workspace():
    cfg = cfg_of("fp8", 16, 4, 512, 256)
    w = gen_weights(cfg, 8, device=DEV)
    x = gen_x(cfg.H, 40, 8, sub=40)
    lg = gen_logits(cfg, 40, 8, sub=40)
    ws = torch.empty(moe.workspace_size(40, 16, 512, 256, 4, "fp8"), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # stale contents must not matter
    s13 = torch.tensor([w[2]], device=DEV)
    s2 = torch.tensor([w[3]], device=DEV)
    ys = [moe.fused_forward(x.to(DEV), lg.to(DEV), w[0], w[1], 4, "fp8", s13, s2, workspace=ws).clone()
          for _ in range(3)]
    assert torch.equal(ys[0].isfinite(), torch.ones_like(ys[0], dtype=torch.bool))
    for y in ys[1:]:
        # the top-k combine sums in a fixed order: repeated calls are bitwise identical
        assert torch.equal(y, ys[0])


def test_bf16_batch_invariance_with_fixed_splits():
    # With the K splits fixed by the caller, a bf16 token's output depends on
    # that token alone: each MFMA output column is one token, routing is per
    # token, and the combine adds in a fixed order.  The same token alone, and
    # at two positions of batches of 17 and 64 other tokens, gives the same bits.
    cfg = cfg_of("bf16", 8, 2, 512, 384)
    w13, w2, _, _ = gen_weights(cfg, 9, device=DEV)
    t = moe.Tuning(gemm1_ksplit=4, gemm2_ksplit=3, gemm2_wave_ksplit=4, token_tiles=2, single_launch=-1)
    x1 = gen_x(cfg.H, 1, 9, sub=1)
    lg1 = gen_logits(cfg, 1, 9, sub=1)
    y1 = moe.fused_forward(x1.to(DEV), lg1.to(DEV), w13, w2, cfg.k, tuning=t)
    for M, pos in ((17, 0), (17, 16), (64, 5), (64, 63)):
        x = gen_x(cfg.H, M, 10 + M, sub=M)
        lg = gen_logits(cfg, M, 10 + M, sub=M)
        x[pos] = x1[0]
        lg[pos] = lg1[0]
        y = moe.fused_forward(x.to(DEV), lg.to(DEV), w13, w2, cfg.k, tuning=t)
        torch.cuda.synchronize()
        assert torch.equal(y[pos], y1[0]), (M, pos)


# ---------------------------------------------------------------- the single-launch layer
# At most 16 tokens and 64 pairs the layer can run as one launch (tuning
# single_launch = 1, which fails rather than falls back where it does not
# fit); the default (0) and -1 take the multi-launch path, which the cases
# below also run at the same sizes.
ONE = moe.Tuning(single_launch=1)
MULTI = moe.Tuning(single_launch=-1)


@pytest.mark.parametrize("dtype,xs,hs", [("bf16", None, None), ("fp8", None, None), ("fp8", 0.02, 0.02)])
@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("path", ["single", "multi"])
def test_small_layer_both_paths(dtype, xs, hs, M, path):
    cfg = cfg_of(dtype, 6, 2, 512, 384)
    compare(cfg, M, seed=60 + M, x_scale=xs, h_scale=hs, tuning=ONE if path == "single" else MULTI)


@pytest.mark.parametrize("S", [1, 2])
def test_single_launch_shared_experts(S):
    for dtype, xs, hs in (("bf16", None, None), ("fp8", None, None), ("fp8", 0.02, 0.004)):
        compare(cfg_of(dtype, 6, 2, 512, 384), 7, seed=61 + S, x_scale=xs, h_scale=hs, n_shared=S, tuning=ONE)


def test_single_launch_weight_scale_modes():
    cfg = cfg_of("fp8", 16, 4, 512, 384)
    compare(cfg, 9, seed=62, weights=gen_weights_per_channel(cfg, 62, device=DEV), tuning=ONE)
    compare(cfg, 9, seed=63, weights=gen_weights_per_expert(cfg, 63, device=DEV), tuning=ONE)
    compare(cfg, 9, seed=63, weights=gen_weights_per_expert(cfg, 63, device=DEV), tuning=ONE, x_scale=0.015,
            h_scale=0.004)


def test_single_launch_down_wave_splits():
    # I of 3, 2 and 4 fp8 K-steps: the down product split over 1, 2 and 4 waves
    for I in (384, 256, 512):
        compare(cfg_of("fp8", 8, 2, 512, I), 6, seed=64 + I, tuning=ONE)


def test_single_launch_refused_where_it_does_not_fit():
    cfg = cfg_of("bf16", 8, 2, 256, 256)
    w13, w2, _, _ = gen_weights(cfg, 65, device=DEV)
    for M in (17, 40):  # more than 16 tokens, more than 64 pairs
        x = gen_x(cfg.H, M, 65, sub=M).to(DEV)
        lg = gen_logits(cfg, M, 65, sub=M).to(DEV)
        with pytest.raises(moe.MoEError) as e:
            moe.fused_forward(x, lg, w13, w2, cfg.k, tuning=ONE)
        assert e.value.code == 2


def test_single_launch_repeat_calls_bitwise():
    cfg = cfg_of("fp8", 16, 4, 512, 256)
    w = gen_weights(cfg, 66, device=DEV)
    x = gen_x(cfg.H, 12, 66, sub=12).to(DEV)
    lg = gen_logits(cfg, 12, 66, sub=12).to(DEV)
    ws = torch.empty(moe.workspace_size(12, 16, 512, 256, 4, "fp8"), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # stale contents must not matter
    s13, s2 = torch.tensor([w[2]], device=DEV), torch.tensor([w[3]], device=DEV)
    ys = [moe.fused_forward(x, lg, w[0], w[1], 4, "fp8", s13, s2, workspace=ws, tuning=ONE).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


# ---------------------------------------------------------------- the workloads
def test_tiny():
    cfg = CONFIGS["tiny"]
    compare(cfg, 4, seed=0)
    compare(cfg, 4, seed=0, tuning=ONE)


@pytest.fixture(scope="module")
def mixtral_w():
    w = gen_weights(CONFIGS["mixtral"], 0, device=DEV)
    yield w
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", CONFIGS["mixtral"].ms)
def test_mixtral(mixtral_w, M):
    compare(CONFIGS["mixtral"], M, seed=0, weights=mixtral_w)
    if M <= 16:  # the single-launch layer too
        compare(CONFIGS["mixtral"], M, seed=0, weights=mixtral_w, tuning=ONE)


@pytest.fixture(scope="module")
def qwen3_w():
    w = gen_weights(CONFIGS["qwen3"], 0, device=DEV)
    yield w
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", CONFIGS["qwen3"].ms)
def test_qwen3(qwen3_w, M):
    compare(CONFIGS["qwen3"], M, seed=0, weights=qwen3_w)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_qwen3_single_launch(qwen3_w, M):
    compare(CONFIGS["qwen3"], M, seed=0, weights=qwen3_w, tuning=ONE)
    compare(CONFIGS["qwen3"], M, seed=0, weights=qwen3_w, tuning=ONE, x_scale=0.02, h_scale=0.01)


@pytest.fixture(scope="module")
def deepseek_w():
    w = gen_weights(CONFIGS["deepseek"], 0, device=DEV)
    yield w
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", CONFIGS["deepseek"].ms)
def test_deepseek(deepseek_w, M):
    compare(CONFIGS["deepseek"], M, seed=0, weights=deepseek_w)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_deepseek_single_launch(deepseek_w, M):
    compare(CONFIGS["deepseek"], M, seed=0, weights=deepseek_w, tuning=ONE)


@pytest.fixture(scope="module")
def prefill_w():
    w = gen_weights(CONFIGS["prefill"], 0, device=DEV)
    yield w
    del w
    torch.cuda.empty_cache()


# Tiled prefill products (fp8 with at least 8192 pairs) at sizes the oracle
# evaluates quickly: Zipf routing leaves experts empty and blocks partial.
def test_prefill_path_dynamic_scales_all_tokens():
    # smallest prefill shapes: four 128-byte K-steps in both products, two
    # 256-row tiles in the down product
    cfg = MoEConfig("pf_small", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="zipf")
    compare(cfg, 1100, seed=11)


def test_prefill_path_shortest_down_k():
    # down product of four K-steps (no steady-state iteration: every step is
    # a tail step that may load the next item), gate/up of 12
    cfg = MoEConfig("pf_k4", E=16, k=8, H=1536, I=512, dtype="fp8", ms=(1100,), logits="zipf")
    compare(cfg, 1100, seed=13)


def test_prefill_path_many_items_per_workgroup():
    # several hundred (tile, block) items in both products: every persistent
    # workgroup walks more than one with the LDS ring running across items
    cfg = MoEConfig("pf_items", E=8, k=2, H=1024, I=1024, dtype="fp8", ms=(8192,), logits="zipf")
    compare(cfg, 8192, seed=14)


def test_prefill_path_static_scales_long_k():
    cfg = MoEConfig("pf_long", E=16, k=8, H=1024, I=512, dtype="fp8", ms=(1100,), logits="zipf")
    compare(cfg, 1100, seed=12, x_scale=0.012, h_scale=0.01)


@pytest.mark.timeout(900)
def test_prefill_full_static_scales(prefill_w):
    M = 4096
    compare(CONFIGS["prefill"], M, seed=0, weights=prefill_w, x_scale=0.011, h_scale=0.02)


@pytest.mark.timeout(900)
def test_prefill_full_dynamic_scales(prefill_w):
    # the measured launch: M = 4096 with dynamic x and h scales; the oracle
    # takes s_h over all 32768 pairs and y of every token
    M = 4096
    compare(CONFIGS["prefill"], M, seed=0, weights=prefill_w)


def test_prefill_path_repeat_calls_bitwise():
    # persistent products, LDS-transposed down epilogue and the fixed-order
    # combine: repeated calls on a stale workspace give the same bits
    cfg = MoEConfig("pf_rep", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="zipf")
    w = gen_weights(cfg, 15, device=DEV)
    x = gen_x(cfg.H, 1100, 15, sub=1100).to(DEV)
    lg = gen_logits(cfg, 1100, 15, sub=1100).to(DEV)
    ws = torch.empty(moe.workspace_size(1100, cfg.E, cfg.H, cfg.I, cfg.k, "fp8"), dtype=torch.uint8, device=DEV)
    ws.fill_(0x7F)
    s13 = torch.tensor([w[2]], device=DEV)
    s2 = torch.tensor([w[3]], device=DEV)
    ys = [moe.fused_forward(x, lg, w[0], w[1], cfg.k, "fp8", s13, s2, workspace=ws).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert bool(ys[0].float().isfinite().all())
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


# ---------------------------------------------------------------- one weight scale per row
@pytest.mark.parametrize("variant", ["ksplit", "stream"])
@pytest.mark.parametrize("xs,hs", [(None, None), (0.015, 0.004)])
@pytest.mark.parametrize("M", [5, 40])
def test_per_channel_small_layer(variant, xs, hs, M):
    cfg = cfg_of("fp8", 16, 4, 512, 384)
    w = gen_weights_per_channel(cfg, 21, device=DEV)
    t = moe.Tuning(gemm1_stream_tiles=-1, gemm2_stream_tiles=-1) if variant == "ksplit" else \
        moe.Tuning(gemm1_stream_tiles=2, gemm2_stream_tiles=2)
    compare(cfg, M, seed=21, weights=w, x_scale=xs, h_scale=hs, tuning=t)


def test_per_channel_equal_rows_match_per_tensor():
    # per-row scales all equal to the tensor's scale: the same bits as one
    # scale per tensor, on the decode and on the prefill path
    for cfg, M in ((cfg_of("fp8", 16, 4, 512, 384), 40),
                   (MoEConfig("pf_pc", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="zipf"), 1100)):
        w13, w2, s13, s2 = gen_weights(cfg, 22, device=DEV)
        x = gen_x(cfg.H, M, 22, sub=M).to(DEV)
        lg = gen_logits(cfg, M, 22, sub=M).to(DEV)
        t13 = torch.tensor([s13], device=DEV)
        t2 = torch.tensor([s2], device=DEV)
        r13 = torch.full((cfg.E, 2 * cfg.I), s13, dtype=torch.float32, device=DEV)
        r2 = torch.full((cfg.E, cfg.H), s2, dtype=torch.float32, device=DEV)
        a = moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", t13, t2)
        b = moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", r13, r2)
        torch.cuda.synchronize()
        assert torch.equal(a, b), cfg.name


def test_per_channel_qwen3_shape():
    cfg = CONFIGS["qwen3"]
    w = gen_weights_per_channel(cfg, 0, device=DEV)
    compare(cfg, 32, seed=0, weights=w)


@pytest.mark.parametrize("xs,hs", [(None, None), (0.012, 0.003)])
def test_per_channel_prefill_path(xs, hs):
    cfg = MoEConfig("pf_pc", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="zipf")
    w = gen_weights_per_channel(cfg, 23, device=DEV)
    compare(cfg, 1100, seed=23, weights=w, x_scale=xs, h_scale=hs)


@pytest.mark.timeout(900)
def test_per_channel_prefill_full_static_scales():
    cfg = CONFIGS["prefill"]
    w = gen_weights_per_channel(cfg, 0, device=DEV)
    compare(cfg, 4096, seed=0, weights=w, x_scale=0.011, h_scale=0.02)
    del w
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- router logits inside the layer
@pytest.mark.parametrize("cfg,M", [
    (MoEConfig("r_bf16", E=8, k=2, H=256, I=512, dtype="bf16", ms=(4,), logits="normal"), 4),
    (CONFIGS["qwen3"], 8),
    (MoEConfig("r_pf", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="normal"), 1100),
])
def test_fused_with_router_weights(cfg, M):
    # the layer computes the logits itself: they agree with the oracle's
    # within fp32 summation error, the routing taken on them is the oracle's
    # bit for bit, and y is the oracle's layer on those logits
    say("fused with router weights %s M=%d" % (cfg.name, M))
    w = gen_weights(cfg, 24, device=DEV)
    x = gen_x(cfg.H, M, 24, sub=M)
    wg = gen_router_weights(cfg.E, cfg.H, 24)
    fp8 = cfg.dtype == "fp8"
    lo = torch.empty(M, cfg.E, dtype=torch.float32, device=DEV)
    ids = torch.empty(M, cfg.k, dtype=torch.int32, device=DEV)
    sc = (lambda v: torch.tensor([v], device=DEV)) if fp8 else (lambda v: None)
    y = moe.fused_forward(x.to(DEV), None, w[0], w[1], cfg.k, cfg.dtype, sc(w[2]), sc(w[3]), topk_ids=ids,
                          router_w=wg.to(DEV), logits_out=lo)
    torch.cuda.synchronize()
    lg = lo.cpu()
    ref_lg = oracle.router_logits(x, wg)
    assert np.abs(lg.numpy() - ref_lg).max() <= 1e-5 * np.abs(ref_lg).max() + 1e-6
    ref_ids, _ = oracle.route(lg, cfg.k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    e, _, _ = compare(cfg, M, seed=24, weights=w, logits=lg, x=x)
    # the same layer on the given logits gives the same bits (on the same
    # path: with router weights the layer never takes the single launch)
    y2 = moe.fused_forward(x.to(DEV), lo, w[0], w[1], cfg.k, cfg.dtype, sc(w[2]), sc(w[3]), tuning=MULTI)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("M", [6, 1100])
def test_router_weights_with_per_channel_scales(M):
    # the two optional inputs together, on the decode and on the prefill path:
    # logits from router weights, one weight scale per row, static x scale
    cfg = MoEConfig("r_pc", E=16, k=8, H=512, I=512, dtype="fp8", ms=(M,), logits="normal")
    w = gen_weights_per_channel(cfg, 25, device=DEV)
    x = gen_x(cfg.H, M, 25, sub=M)
    wg = gen_router_weights(cfg.E, cfg.H, 25)
    lo = torch.empty(M, cfg.E, dtype=torch.float32, device=DEV)
    xs = torch.tensor([0.013], device=DEV)
    y = moe.fused_forward(x.to(DEV), None, w[0], w[1], cfg.k, "fp8", w[2], w[3], x_scale=xs, router_w=wg.to(DEV),
                          logits_out=lo)
    torch.cuda.synchronize()
    _, gpu, _ = compare(cfg, M, seed=25, weights=w, logits=lo.cpu(), x=x, x_scale=0.013, tuning=MULTI)
    assert torch.equal(y.float().cpu(), torch.from_numpy(gpu["y"]).float())


def test_prefill_dynamic_scales(prefill_w):
    compare(CONFIGS["prefill"], 256, seed=0, weights=prefill_w)


# ---------------------------------------------------------------- shared experts
# Every token also passes through the S experts stacked after the E routed
# ones, with weight one: slots k..k+S-1 of the routing.  The cases cover the
# one-wave align (M*(k+S) <= 64), the one-workgroup align, the router + align
# launches with (k+S a power of two) and without the router's histograms, and
# the tiled prefill products.
@pytest.mark.parametrize("dtype,xs,hs", [("bf16", None, None), ("fp8", None, None), ("fp8", 0.02, 0.004)])
@pytest.mark.parametrize("M,S", [(5, 1), (40, 1), (40, 2), (600, 1), (600, 2)])
def test_shared_experts_small_layer(dtype, xs, hs, M, S):
    compare(cfg_of(dtype, 6, 2, 512, 384), M, seed=30 + M + S, x_scale=xs, h_scale=hs, n_shared=S)


def test_shared_expert_qwen3_shape():
    compare(CONFIGS["qwen3"], 16, seed=31, n_shared=1)


@pytest.mark.parametrize("k,S", [(8, 1), (7, 1)])
def test_shared_expert_prefill_path(k, S):
    cfg = MoEConfig("pf_shared", E=16, k=k, H=512, I=512, dtype="fp8", ms=(1100,), logits="zipf")
    compare(cfg, 1100, seed=32 + k, n_shared=S)


def test_shared_expert_per_channel_with_router_weights():
    # per-row weight scales (the shared expert's rows after the routed ones)
    # and logits computed from router weights inside the call; the same layer
    # on those logits, given, gives the same bits and the oracle's output
    cfg = cfg_of("fp8", 16, 4, 512, 384)
    M, S = 24, 1
    w13, w2, s13, s2 = gen_weights_per_channel(cfg_of("fp8", 16 + S, 4, 512, 384), 33, device=DEV)
    x = gen_x(cfg.H, M, 33, sub=M)
    rw = gen_router_weights(cfg.E, cfg.H, 33, device=DEV)
    lo = torch.empty(M, cfg.E, dtype=torch.float32, device=DEV)
    b = moe.fused_forward(x.to(DEV), None, w13, w2, cfg.k, "fp8", s13, s2, router_w=rw, logits_out=lo, n_shared=S)
    a = moe.fused_forward(x.to(DEV), lo, w13, w2, cfg.k, "fp8", s13, s2, n_shared=S)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    compare(cfg, M, seed=33, weights=(w13, w2, s13, s2), x=x, logits=lo.cpu(), n_shared=S)



# ---------------------------------------------------------------- one weight scale per expert
# Experts' scales up to 4x apart, so that a wrong expert's scale fails the
# tolerance; both decode variants, the prefill path, and with shared experts.
@pytest.mark.parametrize("variant", ["ksplit", "stream"])
@pytest.mark.parametrize("xs,hs", [(None, None), (0.015, 0.004)])
@pytest.mark.parametrize("M", [5, 40])
def test_per_expert_small_layer(variant, xs, hs, M):
    cfg = cfg_of("fp8", 16, 4, 512, 384)
    w = gen_weights_per_expert(cfg, 41, device=DEV)
    t = moe.Tuning(gemm1_stream_tiles=-1, gemm2_stream_tiles=-1) if variant == "ksplit" else \
        moe.Tuning(gemm1_stream_tiles=2, gemm2_stream_tiles=2)
    compare(cfg, M, seed=41, weights=w, x_scale=xs, h_scale=hs, tuning=t)


@pytest.mark.parametrize("xs,hs", [(None, None), (0.012, 0.003)])
def test_per_expert_prefill_path(xs, hs):
    cfg = MoEConfig("pf_pe", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="zipf")
    w = gen_weights_per_expert(cfg, 42, device=DEV)
    compare(cfg, 1100, seed=42, weights=w, x_scale=xs, h_scale=hs)


def test_per_expert_equal_scales_match_per_tensor():
    # per-expert scales all equal to the tensor's: the same bits as one scale
    # per tensor, on the decode and on the prefill path
    for cfg, M in ((cfg_of("fp8", 16, 4, 512, 384), 40),
                   (MoEConfig("pf_pe", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="zipf"), 1100)):
        w13, w2, s13, s2 = gen_weights(cfg, 43, device=DEV)
        x = gen_x(cfg.H, M, 43, sub=M).to(DEV)
        lg = gen_logits(cfg, M, 43, sub=M).to(DEV)
        a = moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", torch.tensor([s13], device=DEV),
                              torch.tensor([s2], device=DEV))
        b = moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", torch.full((cfg.E,), s13, device=DEV),
                              torch.full((cfg.E,), s2, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(a, b), cfg.name


@pytest.mark.parametrize("M", [24, 1100])
def test_per_expert_scales_with_shared_expert(M):
    cfg = MoEConfig("pe_shared", E=16, k=7, H=512, I=512, dtype="fp8", ms=(M,), logits="zipf")
    w = gen_weights_per_expert(cfg, 44, device=DEV, E=17)
    compare(cfg, M, seed=44, weights=w, n_shared=1)


@pytest.mark.parametrize("S", [0, 1])
def test_reverse_grid_order_is_bitwise_neutral(S):
    # the workgroup order of the products does not enter the arithmetic: the
    # reversed and the in-order grid give the same bits, in both variants
    cfg = CONFIGS["qwen3"]
    M = 40
    w13, w2, s13, s2 = gen_weights(cfg, 45, device=DEV, E=cfg.E + S)
    x = gen_x(cfg.H, M, 45, sub=M).to(DEV)
    lg = gen_logits(cfg, M, 45, sub=M).to(DEV)
    t13, t2 = torch.tensor([s13], device=DEV), torch.tensor([s2], device=DEV)
    for st in (-1, 2):
        ys = [moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", t13, t2, n_shared=S,
                                tuning=moe.Tuning(reverse_order=r, gemm1_stream_tiles=st, gemm2_stream_tiles=st))
              for r in (1, -1)]
        torch.cuda.synchronize()
        assert torch.equal(ys[0], ys[1]), st


def test_shared_expert_stream_variants():
    t = moe.Tuning(gemm1_stream_tiles=2, gemm2_stream_tiles=2)
    compare(CONFIGS["qwen3"], 40, seed=46, n_shared=1, tuning=t)


# ---------------------------------------------------------------- down product + combine per token
# Layers of at most 64 pairs take, by default, the down product with the
# weighted top-k combine in one launch: a workgroup per (16 output rows,
# token) sums the token's pairs itself (tuning down_per_token; -1 takes the
# per-expert down product and the finalize).  Both paths against the oracle,
# over K chunk counts with an odd number of units per wave, shared experts,
# every weight-scale mode, and repeated calls.
TOK = moe.Tuning(down_per_token=1, single_launch=-1)
EXP = moe.Tuning(down_per_token=-1, single_launch=-1)


@pytest.mark.parametrize("dtype,xs,hs", [("bf16", None, None), ("fp8", None, None), ("fp8", 0.02, 0.02)])
@pytest.mark.parametrize("M", [1, 5, 32])
@pytest.mark.parametrize("path", ["token", "expert"])
def test_down_per_token_small_layers(dtype, xs, hs, M, path):
    compare(cfg_of(dtype, 8, 2, 512, 384), M, seed=80 + M, x_scale=xs, h_scale=hs,
            tuning=TOK if path == "token" else EXP)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("E,k,I", [(1, 1, 1024), (6, 3, 512), (16, 7, 256), (16, 16, 512)])
def test_down_per_token_unit_splits(dtype, E, k, I):
    # pairs per token 1..16 with the K chunks the plan picks for them: paired
    # units and a single unit left over per wave, idle waves (k = 1: one pair
    # in eight chunks), one unit per wave (k = 16 in fp8 gets one chunk)
    M = max(1, 64 // k)
    compare(cfg_of(dtype, E, k, 256, I), M, seed=90 + k, tuning=TOK)


def test_down_per_token_shared_experts_and_scale_modes():
    cfg = cfg_of("fp8", 16, 7, 512, 512, logits="zipf")
    M = 8  # 8 x (7 + 1) = 64 pairs
    compare(cfg, M, seed=95, weights=gen_weights_per_channel(cfg_of("fp8", 17, 7, 512, 512), 95, device=DEV),
            n_shared=1, tuning=TOK)
    compare(cfg, M, seed=96, weights=gen_weights_per_expert(cfg, 96, device=DEV, E=17), n_shared=1, tuning=TOK)
    compare(cfg, M, seed=97, n_shared=1, x_scale=0.015, h_scale=0.004, tuning=TOK)


def test_down_per_token_is_the_default_and_repeats_bitwise():
    # with no tuning a 64-pair layer takes the per-token path (same bits as
    # requiring it), and repeated calls on a stale workspace give the same bits
    cfg = CONFIGS["qwen3"]
    M = 8
    w13, w2, s13, s2 = gen_weights(cfg, 98, device=DEV)
    x = gen_x(cfg.H, M, 98, sub=M).to(DEV)
    lg = gen_logits(cfg, M, 98, sub=M).to(DEV)
    t13, t2 = torch.tensor([s13], device=DEV), torch.tensor([s2], device=DEV)
    ws = torch.empty(moe.workspace_size(M, cfg.E, cfg.H, cfg.I, cfg.k, "fp8"), dtype=torch.uint8, device=DEV)
    ys = [moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", t13, t2, workspace=ws, tuning=t)
          for t in (None, TOK, None, TOK)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


# ---------------------------------------------------------------- router logits at larger M
# With router weights the layer's logits are moe_router_logits' bits (the
# same kernel, every 16 x 16 tile summed in one fixed order), the routing is
# the oracle's on them and y the oracle's layer, at token counts past the
# one-workgroup prologue and not a multiple of the router's 64-token tiles:
# E = 8..256, shared experts, fp8 with a dynamic x scale, and the prefill path.
@pytest.mark.parametrize("cfg,M,S", [
    (MoEConfig("rg_bf16", E=8, k=2, H=256, I=512, dtype="bf16", ms=(300,), logits="normal"), 300, 0),
    (MoEConfig("rg_fp8", E=64, k=6, H=1024, I=512, dtype="fp8", ms=(301,), logits="normal"), 301, 1),
    (MoEConfig("rg_e256", E=256, k=8, H=512, I=256, dtype="fp8", ms=(257,), logits="normal"), 257, 0),
    (MoEConfig("rg_pf", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1100,), logits="normal"), 1100, 0),
])
def test_router_logits_at_larger_token_counts(cfg, M, S):
    say("router weights %s M=%d S=%d" % (cfg.name, M, S))
    w = gen_weights(cfg, 26, device=DEV, E=cfg.E + S)
    x = gen_x(cfg.H, M, 26, sub=M)
    wg = gen_router_weights(cfg.E, cfg.H, 26)
    fp8 = cfg.dtype == "fp8"
    sc = (lambda v: torch.tensor([v], device=DEV)) if fp8 else (lambda v: None)
    lo = torch.empty(M, cfg.E, dtype=torch.float32, device=DEV)
    ids = torch.empty(M, cfg.k + S, dtype=torch.int32, device=DEV)
    y = moe.fused_forward(x.to(DEV), None, w[0], w[1], cfg.k, cfg.dtype, sc(w[2]), sc(w[3]), topk_ids=ids,
                          router_w=wg.to(DEV), logits_out=lo, n_shared=S)
    alone = moe.router_logits(x.to(DEV), wg.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(lo.view(torch.int32), alone.view(torch.int32)), "logits differ from moe_router_logits"
    ref_ids, _ = oracle.route(lo.cpu(), cfg.k)
    assert np.array_equal(ids[:, :cfg.k].cpu().numpy(), ref_ids)
    compare(cfg, M, seed=26, weights=w, logits=lo.cpu(), x=x, n_shared=S)
    y2 = moe.fused_forward(x.to(DEV), lo, w[0], w[1], cfg.k, cfg.dtype, sc(w[2]), sc(w[3]), n_shared=S)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "the layer on its own logits, given, gives other bits"


# ---------------------------------------------------------------- bf16 prefill path
# bf16 layers with at least 8192 pairs take the tiled prefill products too
# (four 32x32x16 bf16 MFMAs per 128-byte K-step, bf16 h between the products,
# no scales).  Every token against the oracle: the smallest shapes (four
# K-steps in both products at H = I = 256 elements), a long K, many items per
# workgroup, shared experts, an align histogram-free top-k (k = 9), and
# repeated calls bitwise.
@pytest.mark.parametrize("E,k,H,I,M,S", [(16, 8, 256, 256, 1100, 0), (16, 8, 1024, 512, 1100, 0),
                                         (8, 2, 1024, 1024, 8192, 0), (16, 7, 512, 512, 1100, 1),
                                         (16, 9, 512, 256, 1000, 0)])
def test_prefill_path_bf16(E, k, H, I, M, S):
    cfg = MoEConfig("pf_bf16", E=E, k=k, H=H, I=I, dtype="bf16", ms=(M,), logits="zipf")
    assert moe.fused_align_shape(M, E + S, H, I, k + S, "bf16")[0] == 128  # the prefill path's block
    compare(cfg, M, seed=60 + k, n_shared=S)


def test_prefill_path_bf16_repeat_calls_bitwise():
    cfg = MoEConfig("pf_bf16_rep", E=16, k=8, H=512, I=512, dtype="bf16", ms=(1100,), logits="zipf")
    w = gen_weights(cfg, 16, device=DEV)
    x = gen_x(cfg.H, 1100, 16, sub=1100).to(DEV)
    lg = gen_logits(cfg, 1100, 16, sub=1100).to(DEV)
    ws = torch.empty(moe.workspace_size(1100, cfg.E, cfg.H, cfg.I, cfg.k, "bf16"), dtype=torch.uint8, device=DEV)
    ws.fill_(0x7F)
    ys = [moe.fused_forward(x, lg, w[0], w[1], cfg.k, "bf16", workspace=ws).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert bool(ys[0].float().isfinite().all())
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


# ---------------------------------------------------------------- two launches for tiny layers
# At most 16 tokens and 64 pairs (fp8 x of at most 8192 elements) with the
# per-token down product: every gate/up workgroup routes, quantises and sorts
# the few tokens itself, so the layer is two launches.  Its arithmetic is the
# three-launch path's: the same bits where that path's gate/up takes the same
# plan (M < 8 in fp8; bf16), and the oracle's outputs everywhere, with the
# call's routing and sort-and-pad outputs (checked by compare).
TWO = moe.Tuning(routing_in_gate_up=1, single_launch=-1)
THREE = moe.Tuning(routing_in_gate_up=-1, single_launch=-1)


@pytest.mark.parametrize("dtype,xs,hs", [("bf16", None, None), ("fp8", None, None), ("fp8", 0.02, 0.004)])
@pytest.mark.parametrize("M", [1, 3, 7])
def test_two_launches_match_three(dtype, xs, hs, M):
    cfg = cfg_of(dtype, 16, 4, 512, 384)
    w13, w2, s13, s2 = gen_weights(cfg, 100 + M, device=DEV)
    x = gen_x(cfg.H, M, 100 + M, sub=M).to(DEV)
    lg = gen_logits(cfg, M, 100 + M, sub=M).to(DEV)
    fp8 = dtype == "fp8"
    sc = (lambda v: torch.tensor([v], device=DEV)) if fp8 else (lambda v: None)
    kw = dict(x_scale=sc(xs) if xs else None, h_scale=sc(hs) if hs else None)
    so = [torch.empty(2, device=DEV) if fp8 else None for _ in range(2)]
    ys = [moe.fused_forward(x, lg, w13, w2, cfg.k, dtype, sc(s13), sc(s2), tuning=t, scales_out=so[i], **kw)
          for i, t in enumerate((TWO, THREE))]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]), "two launches and three differ"
    if fp8:
        assert torch.equal(so[0], so[1])
    compare(cfg, M, seed=100 + M, weights=(w13, w2, s13, s2), x=x.cpu(), logits=lg.cpu(), x_scale=xs, h_scale=hs,
            tuning=TWO)


@pytest.mark.parametrize("xs,hs", [(None, None), (0.02, 0.004)])
@pytest.mark.parametrize("M", [5, 7])
def test_two_launches_match_three_wide_x(xs, hs, M):
    # an fp8 x of 10240 and 14336 elements (four register chunks per thread in
    # the gate/up workgroups), below 8 tokens: the same bits as three launches
    cfg = cfg_of("fp8", 16, 4, 2048, 256)
    w13, w2, s13, s2 = gen_weights(cfg, 110 + M, device=DEV)
    x = gen_x(cfg.H, M, 110 + M, sub=M).to(DEV)
    lg = gen_logits(cfg, M, 110 + M, sub=M).to(DEV)
    sc = lambda v: torch.tensor([v], device=DEV)
    kw = dict(x_scale=sc(xs) if xs else None, h_scale=sc(hs) if hs else None)
    so = [torch.empty(2, device=DEV) for _ in range(2)]
    ys = [moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", sc(s13), sc(s2), tuning=t, scales_out=so[i], **kw)
          for i, t in enumerate((TWO, THREE))]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]), "two launches and three differ"
    assert torch.equal(so[0], so[1])
    compare(cfg, M, seed=110 + M, weights=(w13, w2, s13, s2), x=x.cpu(), logits=lg.cpu(), x_scale=xs, h_scale=hs,
            tuning=TWO)


def test_two_launches_workload_shapes(qwen3_w, deepseek_w):
    compare(CONFIGS["qwen3"], 1, seed=0, weights=qwen3_w, tuning=TWO)
    compare(CONFIGS["qwen3"], 4, seed=0, weights=qwen3_w, tuning=TWO)
    compare(CONFIGS["qwen3"], 8, seed=0, weights=qwen3_w, tuning=TWO)  # x in four register chunks per thread
    compare(CONFIGS["deepseek"], 1, seed=0, weights=deepseek_w, tuning=TWO)
    compare(CONFIGS["tiny"], 4, seed=0, tuning=TWO)


def test_two_launches_shared_experts_and_scale_modes():
    cfg = cfg_of("fp8", 16, 7, 512, 512, logits="zipf")
    M = 8  # 64 pairs with the shared expert; x of 4096 elements
    compare(cfg, M, seed=101, weights=gen_weights_per_channel(cfg_of("fp8", 17, 7, 512, 512), 101, device=DEV),
            n_shared=1, tuning=TWO)
    compare(cfg, M, seed=102, weights=gen_weights_per_expert(cfg, 102, device=DEV, E=17), n_shared=1, tuning=TWO)
    compare(cfg_of("bf16", 8, 2, 512, 384), 16, seed=103, n_shared=1, tuning=TWO)


def test_two_launches_are_the_default_for_tiny_layers():
    cfg = CONFIGS["qwen3"]
    w13, w2, s13, s2 = gen_weights(cfg, 104, device=DEV)
    x = gen_x(cfg.H, 1, 104, sub=1).to(DEV)
    lg = gen_logits(cfg, 1, 104, sub=1).to(DEV)
    t13, t2 = torch.tensor([s13], device=DEV), torch.tensor([s2], device=DEV)
    a = moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", t13, t2)
    b = moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", t13, t2, tuning=TWO)
    c = moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", t13, t2, tuning=THREE)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


# ---- two groups per wave in the K-split products (gemm1_feature_tiles = 2:
# 16-feature groups of the gate/up product; gemm2_row_tiles = 2: 32-row
# groups of the down product): every output's k-steps and K-split sum keep
# their order, so the layer's output is that of one group per wave, bit for
# bit
@pytest.mark.parametrize("dtype,scales", [("bf16", "-"), ("fp8", "dynamic"), ("fp8", "static"),
                                          ("fp8", "per-row"), ("fp8", "per-expert"), ("fp8", "block")])
def test_two_groups_per_wave_match_one(dtype, scales):
    # the down product's K slices are pinned (their default count follows the
    # number of workgroups, which two row groups halve); variants whose LDS
    # does not fit a workgroup are refused by the plan and skipped here
    cfg = cfg_of(dtype, 16, 4, 512, 512)
    fp8 = dtype == "fp8"
    seed = 120
    if scales == "per-row":
        w13, w2, s13, s2 = gen_weights_per_channel(cfg, seed, device=DEV)
    elif scales == "per-expert":
        w13, w2, s13, s2 = gen_weights_per_expert(cfg, seed, device=DEV)
    elif scales == "block":
        w13, w2, s13, s2 = gen_weights_block(cfg, seed, device=DEV)
    else:
        w13, w2, s13, s2 = gen_weights(cfg, seed, device=DEV)
    sc = lambda v: v if isinstance(v, torch.Tensor) else torch.tensor([v], device=DEV)
    kw = dict(x_scale=sc(0.02), h_scale=sc(0.004)) if scales == "static" else {}
    ran, refused = 0, 0
    for M in (20, 45):
        x = gen_x(cfg.H, M, seed, sub=M).to(DEV)
        lg = gen_logits(cfg, M, seed, sub=M).to(DEV)
        for ks in (1, 2, 4):
            for tt, u in ((1, 0), (2, 0), (4, 0), (2, 1 if fp8 else 2)):
                def run(ft, fr):
                    t = moe.Tuning(gemm1_ksplit=ks, gemm2_ksplit=1, gemm2_wave_ksplit=ks, token_tiles=tt, unroll=u,
                                   gemm1_stream_tiles=-1, gemm2_stream_tiles=-1, gemm1_feature_tiles=ft,
                                   gemm2_row_tiles=fr)
                    return moe.fused_forward(x, lg, w13, w2, cfg.k, dtype, sc(s13) if fp8 else None,
                                             sc(s2) if fp8 else None, tuning=t, **kw)
                say("%s %s M=%d ksplit=%d token_tiles=%d unroll=%d" % (dtype, scales, M, ks, tt, u))
                y0 = run(1, 1)
                for ft, fr in ((2, 1), (1, 2), (2, 2)):
                    try:
                        y = run(ft, fr)
                    except moe.MoEError as ex:
                        assert fr == 2 and "UNSUPPORTED" in str(ex), ex  # only the down product's LDS can refuse
                        refused += 1
                        continue
                    torch.cuda.synchronize()
                    assert torch.equal(y0, y), (M, ks, tt, u, ft, fr)
                    ran += 1
    say("  %d variants equal, %d refused" % (ran, refused))
    assert refused <= ran // 4


def test_two_groups_per_wave_parity():
    # both products with two groups per wave against the oracle, on a
    # Mixtral-like expert count (more than 16 tokens per expert, two token
    # tiles) and an fp8 layer
    t = moe.Tuning(gemm1_feature_tiles=2, gemm2_row_tiles=2, gemm1_stream_tiles=-1, gemm2_stream_tiles=-1)
    compare(cfg_of("bf16", 8, 2, 512, 384), 63, seed=121, tuning=t)
    compare(cfg_of("fp8", 16, 4, 512, 384), 60, seed=122, tuning=t)
