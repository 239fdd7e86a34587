"""Pins of the oracle's layer output.

* E=1, k=1 reduces the layer to a plain SwiGLU MLP y = W2 (SiLU(W1 x) * W3 x)
  with the layer's storage roundings; it is recomputed here with float64
  torch matmuls (a library routine), in bf16 and in fp8.
* E=k with equal logits gives weights 1/k, so y is the mean of the expert
  outputs.
* Two experts with unequal logits: y is the softmax-weighted sum of the two
  expert MLPs, with the weights from the closed form.
* A token repeated M times gives identical rows.
* The dynamic fp8 scales are amax/448 of x and of h.
* One weight scale per row (output channel): E=1, k=1 against the same
  float64 SwiGLU with per-row rescaling; per-row scales all equal to the
  tensor's scale give the per-tensor result bit for bit; with several experts
  each pair uses its own expert's rows (static activation scales, dense
  per-token sum of per-expert MLPs).
* One weight scale per expert: scales all equal to the tensor's give the
  per-tensor output bit for bit; unequal scales (up to 4x apart): the dense
  per-token sum of float64 per-expert MLPs, each with its expert's scales.
* Shared experts (experts E.. that every token passes through with weight
  one): with the routed down weights zeroed, y is the shared expert's SwiGLU
  (float64 torch); with S shared experts, y equals the routed-only layer plus
  each shared expert run alone as an E=1, k=1 layer, bit for bit; a dynamic h
  scale is the larger of the routed-only and the shared-only scales.
* A hand-derived fixture in tests/golden.
Plausible mistakes (gate and up swapped, a sign in SiLU, a transposed W2, a
dropped routing weight, the scale applied twice) each fail one of these.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, MoEConfig, gen_weights, gen_weights_per_channel, gen_weights_per_expert, gen_x

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def mlp_ref_bf16(x_bf16: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor) -> torch.Tensor:
    """SwiGLU of one expert: gate rows [0,I), up rows [I,2I); h stored as bf16."""
    I = w13.shape[0] // 2
    x = x_bf16.double()
    gu = x @ w13.double().T
    g, u = gu[:, :I], gu[:, I:]
    h = g / (1 + torch.exp(-g)) * u
    hq = h.float().to(torch.bfloat16).double()
    return hq @ w2.double().T


def dq(codes: torch.Tensor) -> torch.Tensor:
    return codes.view(torch.float8_e4m3fn).double()


def mlp_ref_fp8(x_bf16, w13q, w2q, s13, s2, sx=None, sh=None):
    """fp8 SwiGLU with per-tensor scales; activation scales amax/448 when None."""
    I = w13q.shape[0] // 2
    xf = x_bf16.float()
    if sx is None:
        sx = float(torch.tensor(xf.abs().max().item() / 448.0, dtype=torch.float32))
    sx = float(np.float32(sx))  # scales are fp32 parameters
    rx = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(sx, dtype=torch.float32)
    xq = (xf * rx).clamp(-448, 448).to(torch.float8_e4m3fn).double()  # saturating cast
    gu = (xq @ dq(w13q).T) * (sx * s13)
    g, u = gu[:, :I], gu[:, I:]
    h = (g / (1 + torch.exp(-g)) * u).float()
    if sh is None:
        sh = float(torch.tensor(h.abs().max().item() / 448.0, dtype=torch.float32))
    sh = float(np.float32(sh))
    rh = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(sh, dtype=torch.float32)
    hq = (h * rh).clamp(-448, 448).to(torch.float8_e4m3fn).double()
    return (hq @ dq(w2q).T) * (sh * s2), sx, sh


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def small_cfg(dtype, E, k, H=128, I=96):
    return MoEConfig("t", E=E, k=k, H=H, I=I, dtype=dtype, ms=(1,), logits="normal")


def test_single_expert_is_swiglu_bf16():
    cfg = small_cfg("bf16", 1, 1)
    x = gen_x(cfg.H, 5, seed=1)
    w13, w2, _, _ = gen_weights(cfg, seed=1)
    lg = torch.zeros(5, 1)
    out = oracle.layer(x, lg, w13, w2, 1, "bf16")
    ref = mlp_ref_bf16(x, w13[0], w2[0]).numpy()
    assert (out["ids"] == 0).all() and (out["weights"] == 1.0).all()
    assert rel_err(out["y"], ref) < 1e-12


def test_single_expert_is_swiglu_fp8_dynamic():
    cfg = small_cfg("fp8", 1, 1)
    x = gen_x(cfg.H, 6, seed=2)
    w13, w2, s13, s2 = gen_weights(cfg, seed=2)
    out = oracle.layer(x, torch.zeros(6, 1), w13, w2, 1, "fp8", s13, s2)
    ref, sx, sh = mlp_ref_fp8(x, w13[0], w2[0], s13, s2)
    assert out["s_x"] == sx and out["s_h"] == sh
    assert rel_err(out["y"], ref.numpy()) < 1e-12


def test_single_expert_is_swiglu_fp8_static():
    cfg = small_cfg("fp8", 1, 1)
    x = gen_x(cfg.H, 3, seed=3)
    w13, w2, s13, s2 = gen_weights(cfg, seed=3)
    out = oracle.layer(x, torch.zeros(3, 1), w13, w2, 1, "fp8", s13, s2, x_scale=0.01, h_scale=0.002)
    ref, _, _ = mlp_ref_fp8(x, w13[0], w2[0], s13, s2, sx=0.01, sh=0.002)
    assert out["s_x"] == np.float32(0.01) and out["s_h"] == np.float32(0.002)
    assert rel_err(out["y"], ref.numpy()) < 1e-12


@pytest.mark.parametrize("static", [False, True])
def test_single_expert_is_swiglu_fp8_per_channel(static):
    cfg = small_cfg("fp8", 1, 1)
    x = gen_x(cfg.H, 7, seed=4)
    w13, w2, s13, s2 = gen_weights_per_channel(cfg, seed=4)
    assert len(set(s13[0].tolist())) > cfg.I and len(set(s2[0].tolist())) > cfg.H // 2  # rows differ
    xs, hs = (0.01, 0.002) if static else (None, None)
    out = oracle.layer(x, torch.zeros(7, 1), w13, w2, 1, "fp8", s13, s2, x_scale=xs, h_scale=hs)
    ref, sx, sh = mlp_ref_fp8(x, w13[0], w2[0], s13[0].double(), s2[0].double(), sx=xs, sh=hs)
    assert out["s_x"] == np.float32(sx) and out["s_h"] == np.float32(sh)
    assert rel_err(out["y"], ref.numpy()) < 1e-12


def test_per_channel_equal_rows_is_per_tensor():
    cfg = small_cfg("fp8", 4, 2)
    x = gen_x(cfg.H, 9, seed=5)
    lg = torch.randn(9, 4, generator=torch.Generator().manual_seed(5))
    w13, w2, s13, s2 = gen_weights(cfg, seed=5)
    r13 = torch.full((4, 2 * cfg.I), s13, dtype=torch.float32)
    r2 = torch.full((4, cfg.H), s2, dtype=torch.float32)
    a = oracle.layer(x, lg, w13, w2, 2, "fp8", s13, s2)
    b = oracle.layer(x, lg, w13, w2, 2, "fp8", r13, r2)
    assert np.array_equal(a["y"], b["y"]) and a["s_h"] == b["s_h"]


def test_per_channel_rows_follow_each_pairs_expert():
    cfg = small_cfg("fp8", 4, 2)
    M = 6
    x = gen_x(cfg.H, M, seed=6)
    lg = torch.randn(M, 4, generator=torch.Generator().manual_seed(6))
    w13, w2, s13, s2 = gen_weights_per_channel(cfg, seed=6)
    out = oracle.layer(x, lg, w13, w2, 2, "fp8", s13, s2, x_scale=0.02, h_scale=0.004)
    ref = np.zeros((M, cfg.H))
    for m in range(M):
        for j in range(2):
            e = int(out["ids"][m, j])
            o, _, _ = mlp_ref_fp8(x[m:m + 1], w13[e], w2[e], s13[e].double(), s2[e].double(), sx=0.02, sh=0.004)
            ref[m] += float(out["weights"][m, j]) * o[0].numpy()
    assert rel_err(out["y"], ref) < 1e-12


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_equal_logits_give_mean_of_experts(dtype):
    E = 4
    cfg = small_cfg(dtype, E, E)
    x = gen_x(cfg.H, 2, seed=4)
    w13, w2, s13, s2 = gen_weights(cfg, seed=4)
    out = oracle.layer(x, torch.full((2, E), 0.5), w13, w2, E, dtype, s13, s2,
                       x_scale=0.01 if dtype == "fp8" else None, h_scale=0.001 if dtype == "fp8" else None)
    assert (out["weights"] == 0.25).all()
    if dtype == "bf16":
        per = [mlp_ref_bf16(x, w13[e], w2[e]) for e in range(E)]
    else:
        per = [mlp_ref_fp8(x, w13[e], w2[e], s13, s2, sx=0.01, sh=0.001)[0] for e in range(E)]
    ref = sum(per) / E
    assert rel_err(out["y"], ref.numpy()) < 1e-12


def test_two_experts_weighted_sum_bf16():
    cfg = small_cfg("bf16", 3, 2)
    x = gen_x(cfg.H, 1, seed=5)
    w13, w2, _, _ = gen_weights(cfg, seed=5)
    lg = torch.tensor([[0.1, 1.3, 0.7]], dtype=torch.float32)
    out = oracle.layer(x, lg, w13, w2, 2, "bf16")
    assert out["ids"].tolist() == [[1, 2]]
    l1, l2 = float(lg[0, 1]), float(lg[0, 2])
    w1 = 1 / (1 + math.exp(l2 - l1))
    w = [np.float32(w1), np.float32(1 - w1)]
    ref = float(w[0]) * mlp_ref_bf16(x, w13[1], w2[1]) + float(w[1]) * mlp_ref_bf16(x, w13[2], w2[2])
    assert abs(float(out["weights"][0, 0]) - w1) <= 2 ** -24
    assert rel_err(out["y"], ref.numpy()) < 1e-6


def test_repeated_token_gives_identical_rows():
    cfg = small_cfg("fp8", 8, 2)
    x1 = gen_x(cfg.H, 1, seed=6)
    x = x1.repeat(7, 1)
    lg = torch.randn(1, 8, generator=torch.Generator().manual_seed(6)).repeat(7, 1)
    w13, w2, s13, s2 = gen_weights(cfg, seed=6)
    out = oracle.layer(x, lg, w13, w2, 2, "fp8", s13, s2)
    y = out["y"]
    assert (y == y[0:1]).all()


def test_subset_of_tokens_and_expert_dict_agree_with_full():
    cfg = small_cfg("bf16", 6, 2)
    x = gen_x(cfg.H, 9, seed=7)
    lg = torch.randn(9, 6, generator=torch.Generator().manual_seed(7))
    w13, w2, _, _ = gen_weights(cfg, seed=7)
    full = oracle.layer(x, lg, w13, w2, 2, "bf16")
    need = set(full["ids"][[2, 5]].ravel().tolist())
    part = oracle.layer(x, lg, None, None, 2, "bf16", tokens=[2, 5],
                        experts={e: (w13[e], w2[e]) for e in need})
    assert np.array_equal(part["y"], full["y"][[2, 5]])


def test_golden_hand_example():
    with open(os.path.join(GOLDEN, "layer_hand.json")) as f:
        g = json.load(f)
    x = torch.tensor(g["x"], dtype=torch.float32).to(torch.bfloat16)
    w13 = torch.tensor(g["w13"], dtype=torch.float32).to(torch.bfloat16)
    w2 = torch.tensor(g["w2"], dtype=torch.float32).to(torch.bfloat16)
    lg = torch.tensor(g["logits"], dtype=torch.float32)
    out = oracle.layer(x, lg, w13, w2, g["k"], "bf16")
    assert out["ids"].tolist() == g["ids"]
    assert np.array_equal(out["y"], np.array(g["y"], dtype=np.float64))


def test_shared_expert_alone_is_swiglu_bf16():
    cfg = small_cfg("bf16", 4, 2)
    M = 5
    x = gen_x(cfg.H, M, seed=11)
    w13, w2, _, _ = gen_weights(cfg, seed=11, E=5)
    w2[:4] = 0  # routed experts contribute exactly zero
    lg = torch.randn(M, 4, generator=torch.Generator().manual_seed(11))
    out = oracle.layer(x, lg, w13, w2, 2, "bf16", n_shared=1)
    assert out["ids"].shape == (M, 2) and (out["ids"] < 4).all()
    assert rel_err(out["y"], mlp_ref_bf16(x, w13[4], w2[4]).numpy()) < 1e-12


@pytest.mark.parametrize("dtype,S", [("bf16", 1), ("bf16", 2), ("fp8", 1), ("fp8", 2)])
def test_shared_experts_add_to_routed_output(dtype, S):
    cfg = small_cfg(dtype, 4, 2)
    M = 7
    x = gen_x(cfg.H, M, seed=12)
    w13, w2, s13, s2 = gen_weights(cfg, seed=12, E=4 + S)
    lg = torch.randn(M, 4, generator=torch.Generator().manual_seed(12))
    kw = dict(x_scale=0.02, h_scale=0.004) if dtype == "fp8" else {}
    full = oracle.layer(x, lg, w13, w2, 2, dtype, s13, s2, n_shared=S, **kw)
    ref = oracle.layer(x, lg, w13[:4], w2[:4], 2, dtype, s13, s2, **kw)
    assert np.array_equal(full["ids"], ref["ids"]) and np.array_equal(full["weights"], ref["weights"])
    y = ref["y"]
    for s in range(S):
        alone = oracle.layer(x, torch.zeros(M, 1), w13[4 + s:5 + s], w2[4 + s:5 + s], 1, dtype, s13, s2, **kw)
        y = y + alone["y"]
    assert np.array_equal(full["y"], y)


def test_dynamic_h_scale_covers_shared_pairs():
    cfg = small_cfg("fp8", 4, 2)
    M = 6
    x = gen_x(cfg.H, M, seed=13)
    w13, w2, s13, s2 = gen_weights_per_channel(cfg, seed=13)
    w13s, w2s, s13s, s2s = gen_weights_per_channel(cfg, seed=14)
    w13 = torch.cat([w13, w13s[:1]])
    w2 = torch.cat([w2, w2s[:1]])
    r13 = torch.cat([s13, s13s[:1] * 8])  # the shared expert's h dominates
    r2 = torch.cat([s2, s2s[:1]])
    lg = torch.randn(M, 4, generator=torch.Generator().manual_seed(13))
    full = oracle.layer(x, lg, w13, w2, 2, "fp8", r13, r2, n_shared=1)
    routed = oracle.layer(x, lg, w13[:4], w2[:4], 2, "fp8", r13[:4], r2[:4])
    alone = oracle.layer(x, torch.zeros(M, 1), w13[4:], w2[4:], 1, "fp8", r13[4:], r2[4:])
    assert alone["s_h"] > routed["s_h"]
    assert full["s_h"] == alone["s_h"] and full["s_x"] == routed["s_x"]


def test_per_expert_equal_scales_is_per_tensor():
    cfg = small_cfg("fp8", 4, 2)
    x = gen_x(cfg.H, 9, seed=15)
    lg = torch.randn(9, 4, generator=torch.Generator().manual_seed(15))
    w13, w2, s13, s2 = gen_weights(cfg, seed=15)
    a = oracle.layer(x, lg, w13, w2, 2, "fp8", s13, s2)
    b = oracle.layer(x, lg, w13, w2, 2, "fp8", torch.full((4,), s13), torch.full((4,), s2))
    assert np.array_equal(a["y"], b["y"]) and a["s_h"] == b["s_h"]


@pytest.mark.parametrize("static", [False, True])
def test_per_expert_scales_follow_each_pairs_expert(static):
    cfg = small_cfg("fp8", 4, 2)
    M = 6
    x = gen_x(cfg.H, M, seed=16)
    lg = torch.randn(M, 4, generator=torch.Generator().manual_seed(16))
    w13, w2, s13, s2 = gen_weights_per_expert(cfg, seed=16)
    assert float(s13.max() / s13.min()) > 3
    xs, hs = (0.02, 0.004) if static else (None, None)
    out = oracle.layer(x, lg, w13, w2, 2, "fp8", s13, s2, x_scale=xs, h_scale=hs)
    if not static:  # the scales the oracle took, checked on their own by the E = 1 pins
        xs, hs = out["s_x"], out["s_h"]
    ref = np.zeros((M, cfg.H))
    for m in range(M):
        for j in range(2):
            e = int(out["ids"][m, j])
            o, _, _ = mlp_ref_fp8(x[m:m + 1], w13[e], w2[e], float(s13[e]), float(s2[e]), sx=xs, sh=hs)
            ref[m] += float(out["weights"][m, j]) * o[0].numpy()
    assert rel_err(out["y"], ref) < 1e-12
