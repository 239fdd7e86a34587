"""Seeded random layer shapes against the oracle.

The other GPU tests pin the shapes of the five workloads and the edges of
each path one at a time; these cases draw every knob at once from a fixed
seed: the expert count and top-k (with and without shared experts), H and I
(any multiple of 128), the token count (from one token to past the 8192
pairs where fp8 layers take the tiled prefill products; a second set holds
decode-sized layers of 1 to 64 tokens with H up to 8192 and I up to 4096), the logits'
distribution, the weight-scale mode (per tensor, per row, per expert,
128 x 128 blocks), static or dynamic activation scales, and the
deterministic mode.  So the default path choice (single workgroup routing
or the router launches, two or three launches, per-token or per-expert down
product, decode or prefill products, the K-split and stream variants the
plan picks) meets shapes no other test names.  Each case is a full
`compare`: bit-exact routing and sort-and-pad, outputs within the tolerance.
The oracle's work per case is capped so that the whole file runs in minutes.
"""
import math

import numpy as np
import pytest
import torch

import moe_layer_align_amd as moe

import oracle
from gpu_common import DEV, TOL, TOL_TOKEN_FP8, compare, err_norm, row_errs, run_oracle, say
from synth import (MoEConfig, gen_router_weights, gen_weights, gen_weights_block, gen_weights_per_channel,
                   gen_weights_per_expert, gen_x)

pytestmark = pytest.mark.gpu

N_CASES = 40
MAX_MACS = 2.5e10  # multiply-adds of the oracle's expert products per case
MAX_MACS_BLOCK = 6e9  # the same for 128 x 128 block scales, which the oracle applies block by block
PREFILL_PAIRS = 8192  # fp8 layers with at least this many pairs take the tiled products


def _draw(rng: np.random.Generator, i: int) -> dict:
    dtype = "fp8" if rng.random() < 0.6 else "bf16"
    E = int(rng.choice([1, 2, 3, 5, 8, 16, 31, 64, 100, 128, 200, 256, 300]))
    S = int(rng.choice([0, 0, 0, 1, 2]))
    k = int(rng.integers(1, min(E, 16 - S) + 1))
    H = 128 * int(rng.integers(1, 17))
    I = 128 * int(rng.integers(1, 13))
    logits = str(rng.choice(["normal", "biased", "zipf"]))
    if logits == "zipf" and E < k + 8:
        logits = "normal"  # zipf gives four experts the same logit; keep them out of every top-k
    mode, xs, hs, det = 0, None, None, False
    if dtype == "fp8":
        mode = int(rng.choice([0, 0, 1, 2, 3]))
        if mode != 3 and rng.random() < 0.4:
            xs, hs = 0.02, float(rng.choice([0.004, 0.02, 0.06]))
    if mode != 3 and rng.random() < 0.15:
        det = True
        if dtype == "fp8":
            xs, hs = 0.02, 0.02
    KS = k + S
    if dtype == "fp8" and not det and rng.random() < 0.3:
        M = -(-PREFILL_PAIRS // KS) + int(rng.integers(0, 300))
    else:
        M = int(round(math.exp(rng.uniform(0.0, math.log(1200.0)))))
    # keep the oracle's products under the cap: shrink I, then H
    cap = MAX_MACS_BLOCK if mode == 3 else MAX_MACS
    while M * KS * 3 * H * I > cap and I > 128:
        I -= 128
    while M * KS * 3 * H * I > cap and H > 128:
        H -= 128
    return dict(i=i, dtype=dtype, E=E, S=S, k=k, H=H, I=I, M=M, logits=logits, mode=mode, xs=xs, hs=hs, det=det)


_RNG = np.random.default_rng(20261203)
CASES = [_draw(_RNG, i) for i in range(N_CASES)]


def _draw_decode(rng: np.random.Generator, i: int) -> dict:
    # decode-sized layers with wide matrices: M 1..64, H up to 8192, I up to 4096
    dtype = "fp8" if rng.random() < 0.6 else "bf16"
    E = int(rng.choice([1, 2, 4, 8, 16, 64, 128, 256]))
    S = int(rng.choice([0, 0, 0, 1]))
    k = int(rng.integers(1, min(E, 16 - S) + 1))
    H = 128 * int(rng.integers(1, 65))
    I = 128 * int(rng.integers(1, 33))
    M = int(round(math.exp(rng.uniform(0.0, math.log(64.0)))))
    logits = "biased" if rng.random() < 0.5 else "normal"
    mode, xs, hs, det = 0, None, None, False
    if dtype == "fp8":
        mode = int(rng.choice([0, 0, 1, 2, 3]))
        if mode != 3 and rng.random() < 0.4:
            xs, hs = 0.02, float(rng.choice([0.004, 0.02, 0.06]))
    if mode != 3 and rng.random() < 0.15:
        det = True
        if dtype == "fp8":
            xs, hs = 0.02, 0.02
    cap = MAX_MACS_BLOCK if mode == 3 else MAX_MACS
    while M * (k + S) * 3 * H * I > cap and I > 128:
        I -= 128
    return dict(i=i, dtype=dtype, E=E, S=S, k=k, H=H, I=I, M=M, logits=logits, mode=mode, xs=xs, hs=hs, det=det)


CASES += [_draw_decode(_RNG, N_CASES + i) for i in range(N_CASES)]

# Logits from a few integer values, so that most top-k selections break ties
# (toward the lower expert index): the ids must still match bit for bit on
# every routing variant the fused call picks (one wave, one workgroup, the
# multi-workgroup router).
_TIE_RNG = np.random.default_rng(977)
TIE_CASES = []
for _i in range(16):
    _c = (_draw if _i % 2 else _draw_decode)(_TIE_RNG, 2 * N_CASES + _i)
    _c["logits"] = "ties%d" % int(_TIE_RNG.integers(2, 6))
    TIE_CASES.append(_c)


def _id(c: dict) -> str:
    sc = "" if c["dtype"] == "bf16" else "-m%d-%s" % (c["mode"], "dyn" if c["xs"] is None else "hs%g" % c["hs"])
    return "%d-%s-E%dk%dS%d-H%dI%d-M%d-%s%s%s" % (c["i"], c["dtype"], c["E"], c["k"], c["S"], c["H"], c["I"],
                                                 c["M"], c["logits"], sc, "-det" if c["det"] else "")


def test_cases_cover_the_paths():
    # the draw reaches every path it is meant to exercise
    fp8 = [c for c in CASES if c["dtype"] == "fp8"]
    assert any(c["M"] * (c["k"] + c["S"]) >= PREFILL_PAIRS and not c["det"] and c["mode"] != 3 for c in fp8)
    assert any(c["M"] * (c["k"] + c["S"]) <= 64 for c in CASES)
    assert any(c["S"] > 0 for c in CASES) and any(c["det"] for c in CASES)
    assert {c["mode"] for c in fp8} == {0, 1, 2, 3}
    assert any(c["xs"] is not None for c in fp8) and any(c["xs"] is None for c in fp8)
    assert any(c["H"] > 4096 and c["M"] <= 64 for c in CASES) and any(c["I"] > 2048 and c["M"] <= 64 for c in CASES)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("c", CASES + TIE_CASES, ids=_id)
def test_random_shape(c):
    ties = c["logits"].startswith("ties")
    cfg = MoEConfig("rand%d" % c["i"], E=c["E"], k=c["k"], H=c["H"], I=c["I"], dtype=c["dtype"], ms=(c["M"],),
                    logits="normal" if ties else c["logits"])
    seed = 7000 + c["i"]
    ES = c["E"] + c["S"]
    gen = {0: gen_weights, 1: gen_weights_per_channel, 2: gen_weights_per_expert, 3: gen_weights_block}[c["mode"]]
    w = gen(cfg, seed, device=DEV, E=ES)
    logits = None
    if ties:
        levels = int(c["logits"][4:])
        g = np.random.default_rng(seed)
        logits = torch.from_numpy(g.integers(0, levels, (c["M"], c["E"])).astype(np.float32) * 0.5)
    compare(cfg, c["M"], seed=seed, weights=w, x_scale=c["xs"], h_scale=c["hs"], n_shared=c["S"],
            deterministic=c["det"], logits=logits)


def _draw_router(rng: np.random.Generator, i: int) -> dict:
    dtype = "fp8" if rng.random() < 0.6 else "bf16"
    E = int(rng.choice([2, 8, 16, 64, 128, 256, 384, 512]))
    k = int(rng.integers(1, min(E, 16) + 1))
    H = 128 * int(rng.integers(1, 33))
    I = 128 * int(rng.integers(1, 13))
    mode = int(rng.choice([0, 1, 2])) if dtype == "fp8" else 0
    if dtype == "fp8" and rng.random() < 0.3:
        M = -(-PREFILL_PAIRS // k) + int(rng.integers(0, 200))
    else:
        M = int(round(math.exp(rng.uniform(0.0, math.log(1200.0)))))
    while M * k * 3 * H * I > MAX_MACS and I > 128:
        I -= 128
    while M * k * 3 * H * I > MAX_MACS and H > 128:
        H -= 128
    return dict(i=i, dtype=dtype, E=E, S=0, k=k, H=H, I=I, M=M, logits="router", mode=mode, xs=None, hs=None,
                det=False)


_ROUTER_RNG = np.random.default_rng(31337)
ROUTER_CASES = [_draw_router(_ROUTER_RNG, 3 * N_CASES + i) for i in range(12)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("c", ROUTER_CASES, ids=_id)
def test_random_router_weights(c):
    # the layer computes its logits from router weights: they agree with the
    # oracle's within fp32 summation error, the routing on them is the
    # oracle's bit for bit, and y is the oracle's layer on those logits
    M, E, k, H = c["M"], c["E"], c["k"], c["H"]
    cfg = MoEConfig("router%d" % c["i"], E=E, k=k, H=H, I=c["I"], dtype=c["dtype"], ms=(M,), logits="normal")
    seed = 7000 + c["i"]
    gen = {0: gen_weights, 1: gen_weights_per_channel, 2: gen_weights_per_expert}[c["mode"]]
    w = gen(cfg, seed, device=DEV)
    x = gen_x(H, M, seed, sub=M)
    wg = gen_router_weights(E, H, seed)
    fp8 = c["dtype"] == "fp8"
    sc = (lambda v: v.to(DEV) if isinstance(v, torch.Tensor) else torch.tensor([v], device=DEV)) if fp8 else \
        (lambda v: None)
    lo = torch.empty(M, E, dtype=torch.float32, device=DEV)
    ids = torch.empty(M, k, dtype=torch.int32, device=DEV)
    say("router weights %s" % _id(c))
    y = moe.fused_forward(x.to(DEV), None, w[0], w[1], k, c["dtype"], sc(w[2]), sc(w[3]), topk_ids=ids,
                          router_w=wg.to(DEV), logits_out=lo)
    torch.cuda.synchronize()
    lg = lo.cpu()
    ref_lg = oracle.router_logits(x, wg)
    assert np.abs(lg.numpy() - ref_lg).max() <= 1e-5 * np.abs(ref_lg).max() + 1e-6
    ref = run_oracle(cfg, x, lg, w)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    yg = y.float().cpu().numpy().astype(np.float64)
    e, er = err_norm(yg, ref["y"]), float(row_errs(yg, ref["y"]).max())
    say("  err=%.3e per-token %.3e" % (e, er))
    assert np.isfinite(yg).all()
    assert e <= TOL[c["dtype"]] and er <= (TOL_TOKEN_FP8 if fp8 else TOL["bf16"]), (e, er)
