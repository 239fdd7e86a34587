"""Seeded synthetic inputs for the fused MoE layer.

This module only draws random inputs of the shapes and value laws of the
workloads; it holds none of the layer's arithmetic (no routing, no sorting,
no activation quantisation, no GEMM).  Both the CPU oracle and the GPU path
read the tensors it returns.

Workloads (sizes and laws as stated for the Mixtral-, Qwen3-MoE- and
DeepSeek-V3-shaped layers and the prefill case; the web pages on the subject
only say that decode batches hold one token per user, M = 1..63, and that the
layer works on FP8 per-tensor-quantised or bf16 experts):

* x      : hidden states, N(0, 1), stored as bf16 [M, H]
* logits : router logits, fp32 [M, E]
    - "normal": N(0, 1)
    - "biased": N(0, 1) + b_e, one bias per expert, b_e ~ N(0, 0.5**2)
    - "zipf"  : N(0, 1) + ln p_r(e), p_r proportional to r**-1.1 for a seeded
                rank permutation r of the experts; the 4 lowest-ranked experts
                get -1e4 so that some experts receive no token at all
* W13    : [E, 2I, H], rows [0, I) gate, [I, 2I) up, N(0, 1/H)
* W2     : [E, H, I], N(0, 1/I)
  bf16 layers store the weights as bf16 (round to nearest even, torch cast);
  fp8 layers store OCP e4m3fn codes (torch cast) with one fp32 scale per
  tensor, scale = amax(|W|)/448 over all experts of that tensor.

Every tensor is drawn from its own torch.Generator whose seed is derived from
(seed, tensor id, expert), so a tensor never depends on the order in which the
others were drawn.  Weights may be drawn directly on the GPU (fast for the
multi-GB layers); x and logits are always drawn on the host so that routing
inputs are byte-identical for both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, List, Optional, Tuple

import torch

__all__ = ["MoEConfig", "CONFIGS", "gen_x", "gen_logits", "gen_weights", "gen_weights_block", "gen_x_varied",
           "LayerInputs", "make_layer"]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    E: int
    k: int
    H: int
    I: int
    dtype: str  # "bf16" or "fp8"
    ms: Tuple[int, ...]
    logits: str  # "normal", "biased", "zipf"


# The five workloads, by shape.
CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", E=8, k=2, H=256, I=512, dtype="bf16", ms=(4,), logits="normal"),
    "mixtral": MoEConfig("mixtral", E=8, k=2, H=4096, I=14336, dtype="bf16", ms=(1, 4, 16, 32, 63), logits="normal"),
    "qwen3": MoEConfig("qwen3", E=128, k=8, H=2048, I=768, dtype="fp8", ms=(1, 8, 32, 64), logits="normal"),
    "deepseek": MoEConfig("deepseek", E=256, k=8, H=7168, I=2048, dtype="fp8", ms=(1, 16, 64, 128), logits="biased"),
    "prefill": MoEConfig("prefill", E=128, k=8, H=4096, I=1536, dtype="fp8", ms=(4096,), logits="zipf"),
}

_T_X, _T_LOGITS, _T_BIAS, _T_PERM, _T_W13, _T_W2, _T_WG = 1, 2, 3, 4, 5, 6, 7
E4M3_MAX = 448.0


def _gen(seed: int, tensor: int, sub: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed & 0xFFFFFFFF) << 24) ^ (tensor << 16) ^ (sub & 0xFFFF) ^ 0x5DEECE66D)
    return g


def gen_x(H: int, M: int, seed: int = 0, sub: int = 0) -> torch.Tensor:
    """Hidden states x ~ N(0,1), bf16 [M, H], on the host."""
    g = _gen(seed, _T_X, sub, "cpu")
    return torch.randn(M, H, generator=g, dtype=torch.float32).to(torch.bfloat16)


def gen_logits(cfg: MoEConfig, M: int, seed: int = 0, sub: int = 0) -> torch.Tensor:
    """Router logits, fp32 [M, E], on the host, following cfg.logits."""
    E = cfg.E
    g = _gen(seed, _T_LOGITS, sub, "cpu")
    z = torch.randn(M, E, generator=g, dtype=torch.float64)
    if cfg.logits == "normal":
        out = z
    elif cfg.logits == "biased":
        gb = _gen(seed, _T_BIAS, 0, "cpu")
        bias = torch.randn(E, generator=gb, dtype=torch.float64) * 0.5
        out = z + bias[None, :]
    elif cfg.logits == "zipf":
        gp = _gen(seed, _T_PERM, 0, "cpu")
        rank = torch.randperm(E, generator=gp) + 1  # rank of expert e, 1 = most popular
        p = rank.to(torch.float64) ** -1.1
        p = p / p.sum()
        out = z + torch.log(p)[None, :]
        cold = rank > E - 4
        out[:, cold] = -1.0e4
    else:
        raise ValueError(cfg.logits)
    return out.to(torch.float32).contiguous()


def _expert_normal(seed: int, tensor: int, e: int, rows: int, cols: int, std: float, device) -> torch.Tensor:
    g = _gen(seed, tensor, e, device)
    w = torch.randn(rows, cols, generator=g, dtype=torch.float32, device=device)
    return w * std


def gen_weights(cfg: MoEConfig, seed: int = 0, device="cpu", H: Optional[int] = None, I: Optional[int] = None,
                E: Optional[int] = None):
    """Expert weights.

    Returns (w13, w2, s13, s2): bf16 tensors and None scales for bf16 layers,
    uint8 e4m3fn codes and python-float fp32 scales for fp8 layers.
    """
    E = cfg.E if E is None else E
    H = cfg.H if H is None else H
    I = cfg.I if I is None else I
    s13_std, s2_std = 1.0 / math.sqrt(H), 1.0 / math.sqrt(I)
    if cfg.dtype == "bf16":
        w13 = torch.empty(E, 2 * I, H, dtype=torch.bfloat16, device=device)
        w2 = torch.empty(E, H, I, dtype=torch.bfloat16, device=device)
        for e in range(E):
            w13[e] = _expert_normal(seed, _T_W13, e, 2 * I, H, s13_std, device).to(torch.bfloat16)
            w2[e] = _expert_normal(seed, _T_W2, e, H, I, s2_std, device).to(torch.bfloat16)
        return w13, w2, None, None
    if cfg.dtype != "fp8":
        raise ValueError(cfg.dtype)
    # pass 1: per-tensor amax over all experts; pass 2: redraw and cast.
    a13 = torch.zeros((), dtype=torch.float32, device=device)
    a2 = torch.zeros((), dtype=torch.float32, device=device)
    for e in range(E):
        a13 = torch.maximum(a13, _expert_normal(seed, _T_W13, e, 2 * I, H, s13_std, device).abs().amax())
        a2 = torch.maximum(a2, _expert_normal(seed, _T_W2, e, H, I, s2_std, device).abs().amax())
    s13 = float((a13 / E4M3_MAX).item())
    s2 = float((a2 / E4M3_MAX).item())
    w13 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device=device)
    r13 = torch.tensor(s13, dtype=torch.float32, device=device)
    r2 = torch.tensor(s2, dtype=torch.float32, device=device)
    for e in range(E):
        q = (_expert_normal(seed, _T_W13, e, 2 * I, H, s13_std, device) / r13).clamp_(-E4M3_MAX, E4M3_MAX)
        w13[e] = q.to(torch.float8_e4m3fn).view(torch.uint8)
        q = (_expert_normal(seed, _T_W2, e, H, I, s2_std, device) / r2).clamp_(-E4M3_MAX, E4M3_MAX)
        w2[e] = q.to(torch.float8_e4m3fn).view(torch.uint8)
    return w13, w2, s13, s2


def gen_router_weights(E: int, H: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router weights W_g [E,H] bf16 ~ N(0, 1/H): logits x . W_g^T of N(0,1)
    hidden states are then about N(0,1), the law of the given-logit workloads."""
    g = _gen(seed, _T_WG, 0, device)
    w = torch.randn(E, H, generator=g, dtype=torch.float32, device=device) / math.sqrt(H)
    return w.to(torch.bfloat16).contiguous()


def gen_weights_per_channel(cfg: MoEConfig, seed: int = 0, device="cpu", E: Optional[int] = None):
    """fp8 expert weights with one scale per weight row (output channel).

    The same normal draws as gen_weights; row n of W13[e] and of W2[e] is
    stored as e4m3fn codes of W/s with s = amax(|row|)/448 (1.0 for an all-zero
    row).  Returns (w13, w2, s13, s2): uint8 codes and fp32 tensors s13 [E,2I],
    s2 [E,H] on `device`.
    """
    if cfg.dtype != "fp8":
        raise ValueError("per-channel scales are for fp8 layers")
    E = cfg.E if E is None else E
    H, I = cfg.H, cfg.I
    s13_std, s2_std = 1.0 / math.sqrt(H), 1.0 / math.sqrt(I)
    w13 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device=device)
    s13 = torch.empty(E, 2 * I, dtype=torch.float32, device=device)
    s2 = torch.empty(E, H, dtype=torch.float32, device=device)
    for e in range(E):
        for w, s, t, rows, cols, std in ((w13, s13, _T_W13, 2 * I, H, s13_std), (w2, s2, _T_W2, H, I, s2_std)):
            v = _expert_normal(seed, t, e, rows, cols, std, device)
            a = v.abs().amax(dim=1)
            sc = torch.where(a > 0, a / E4M3_MAX, torch.ones_like(a))
            s[e] = sc
            w[e] = (v / sc[:, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return w13, w2, s13, s2


def gen_weights_per_expert(cfg: MoEConfig, seed: int = 0, device="cpu", E: Optional[int] = None):
    """fp8 expert weights with one scale per expert and weight tensor.

    The normal draws of gen_weights with expert e's standard deviation
    multiplied by 0.5 * (1 + e % 4), so that the experts' scales differ by up
    to 4x; W13[e] and W2[e] are stored as e4m3fn codes of W/s with
    s = amax(|W|)/448 over that expert's tensor.  Returns (w13, w2, s13, s2):
    uint8 codes and fp32 tensors s13 [E], s2 [E] on `device`.
    """
    if cfg.dtype != "fp8":
        raise ValueError("per-expert scales are for fp8 layers")
    E = cfg.E if E is None else E
    H, I = cfg.H, cfg.I
    w13 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device=device)
    s13 = torch.empty(E, dtype=torch.float32, device=device)
    s2 = torch.empty(E, dtype=torch.float32, device=device)
    for e in range(E):
        f = 0.5 * (1 + e % 4)
        for w, s, t, rows, cols, std in ((w13, s13, _T_W13, 2 * I, H, f / math.sqrt(H)),
                                         (w2, s2, _T_W2, H, I, f / math.sqrt(I))):
            v = _expert_normal(seed, t, e, rows, cols, std, device)
            sc = v.abs().amax() / E4M3_MAX
            s[e] = sc
            w[e] = (v / sc).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return w13, w2, s13, s2


_T_BLK, _T_XV = 8, 9


def gen_weights_block(cfg: MoEConfig, seed: int = 0, device="cpu", E: Optional[int] = None):
    """fp8 expert weights with one power-of-two (E8M0) scale per 128 x 128 block.

    The normal draws of gen_weights, each 128 x 128 block multiplied by 2^r
    with r drawn uniformly from -3..3 per block (so neighbouring blocks'
    scales differ by up to 64x and a scale taken from a wrong block shows);
    the block's E8M0 code is c = max(floor(log2 amax) + 127 - 8, 0) and its
    values are stored as e4m3fn codes of W * 2^(127 - c) (below 512, clamped
    to 448).  Returns (w13, w2, b13, b2): uint8 codes [E,2I,H] / [E,H,I] and
    uint8 E8M0 codes [E,2I/128,H/128] / [E,H/128,I/128] on `device`.
    """
    if cfg.dtype != "fp8":
        raise ValueError("block scales are for fp8 layers")
    E = cfg.E if E is None else E
    H, I = cfg.H, cfg.I
    w13 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device=device)
    b13 = torch.empty(E, 2 * I // 128, H // 128, dtype=torch.uint8, device=device)
    b2 = torch.empty(E, H // 128, I // 128, dtype=torch.uint8, device=device)
    for e in range(E):
        for w, b, t, rows, cols, std in ((w13, b13, _T_W13, 2 * I, H, 1.0 / math.sqrt(H)),
                                         (w2, b2, _T_W2, H, I, 1.0 / math.sqrt(I))):
            v = _expert_normal(seed, t, e, rows, cols, std, device)
            gr = _gen(seed, _T_BLK, e * 2 + (t == _T_W2), device)
            r = torch.randint(-3, 4, (rows // 128, cols // 128), generator=gr, device=device).to(torch.float32)
            blocks = v.view(rows // 128, 128, cols // 128, 128) * torch.exp2(r)[:, None, :, None]
            amax = blocks.abs().amax(dim=(1, 3))
            _, ex = torch.frexp(amax)  # amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
            c = torch.clamp(ex - 1 + 127 - 8, 0, 254)
            b[e] = c.to(torch.uint8)
            q = blocks * torch.exp2((127 - c).to(torch.float32))[:, None, :, None]
            w[e] = q.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8).view(rows, cols)
    return w13, w2, b13, b2


def gen_x_varied(H: int, M: int, seed: int = 0, sub: int = 0) -> torch.Tensor:
    """Hidden states whose tokens and 128-element groups differ in magnitude:
    N(0,1) times 2^a per token and 2^b per group, a and b drawn from -4..4, so
    that per-group activation scales differ.  bf16 [M, H] on the host."""
    x = gen_x(H, M, seed, sub).to(torch.float32)
    g = _gen(seed, _T_XV, sub, "cpu")
    a = torch.randint(-4, 5, (M, 1), generator=g).to(torch.float32)
    b = torch.randint(-4, 5, (M, H // 128), generator=g).to(torch.float32)
    f = torch.exp2(a + torch.repeat_interleave(b, 128, dim=1))
    return (x * f).to(torch.bfloat16)


@dataclasses.dataclass
class LayerInputs:
    cfg: MoEConfig
    M: int
    x: torch.Tensor        # bf16 [M,H] host
    logits: torch.Tensor   # fp32 [M,E] host
    w13: torch.Tensor      # bf16 or uint8 [E,2I,H]
    w2: torch.Tensor       # bf16 or uint8 [E,H,I]
    s13: Optional[float]
    s2: Optional[float]


def make_layer(cfg: MoEConfig, M: int, seed: int = 0, device="cpu", weights=None) -> LayerInputs:
    """All inputs of one layer call.  `weights` may be passed to reuse a draw."""
    x = gen_x(cfg.H, M, seed, sub=M)
    logits = gen_logits(cfg, M, seed, sub=M)
    if weights is None:
        weights = gen_weights(cfg, seed, device)
    w13, w2, s13, s2 = weights
    return LayerInputs(cfg, M, x, logits, w13, w2, s13, s2)
