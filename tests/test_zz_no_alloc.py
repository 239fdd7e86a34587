"""GPU test of moe_fused_forward_noalloc, the fused layer for callers that
cannot allocate device memory, called through the C ABI binding.

Its output equals the workspace entry point's (moe_fused_forward) bit for
bit, and the oracle's within the stated tolerance, on two calls in a row, the
second with a smaller input (the scratch array keeps the first call's
contents); calls beyond the scratch array, or that pass a workspace, are
refused before anything runs.  The seeded random layers of the parity
tests that fit the array give the same bits through both entry points.
"""
import numpy as np
import pytest
import torch

import moe_layer_align_amd as moe
from gpu_common import DEV, TOL, err_norm, run_gpu, run_oracle, say
from synth import (MoEConfig, gen_logits, gen_weights, gen_weights_block, gen_weights_per_channel,
                   gen_weights_per_expert, gen_x)

pytestmark = pytest.mark.gpu


def _pair(cfg, w, M, seed, x_scale=None, h_scale=None):
    """(workspace entry point, no-alloc entry point) outputs on the same inputs."""
    w13, w2, s13, s2 = w
    fp8 = cfg.dtype == "fp8"
    t = lambda v: None if v is None else torch.tensor([v], dtype=torch.float32, device=DEV)
    x = gen_x(cfg.H, M, seed, sub=M)
    lg = gen_logits(cfg, M, seed, sub=M)
    res = []
    for noalloc in (False, True):
        y = torch.full((M, cfg.H), float("nan"), dtype=torch.bfloat16, device=DEV)
        ids = torch.full((M, cfg.k), -1, dtype=torch.int32, device=DEV)
        wts = torch.zeros(M, cfg.k, dtype=torch.float32, device=DEV)
        counts = torch.full((cfg.E,), -1, dtype=torch.int32, device=DEV)
        moe.fused_forward(x.to(DEV), lg.to(DEV), w13, w2, cfg.k, cfg.dtype, t(s13) if fp8 else None,
                          t(s2) if fp8 else None, x_scale=t(x_scale), h_scale=t(h_scale), out=y, topk_ids=ids,
                          topk_weights=wts, expert_counts=counts, noalloc=noalloc)
        torch.cuda.synchronize()
        res.append(dict(y=y.view(torch.int16).cpu(), ids=ids.cpu(), w=wts.cpu(), counts=counts.cpu(),
                        yf=y.float().cpu().numpy().astype(np.float64)))
    return x, lg, res[0], res[1]


@pytest.mark.parametrize("cfg,ms,scales", [
    (MoEConfig("na_fp8", E=64, k=8, H=1024, I=768, dtype="fp8", ms=(1,), logits="normal"), (64, 9), (None, None)),
    (MoEConfig("na_fp8s", E=64, k=8, H=1024, I=768, dtype="fp8", ms=(1,), logits="normal"), (40, 3), (0.02, 0.004)),
    (MoEConfig("na_bf16", E=8, k=2, H=1024, I=2048, dtype="bf16", ms=(1,), logits="normal"), (63, 1), (None, None)),
], ids=["fp8_dynamic", "fp8_static", "bf16"])
def test_noalloc_matches_workspace_entry_point(cfg, ms, scales):
    w = gen_weights(cfg, 71, device=DEV)
    for i, M in enumerate(ms):
        say("no-alloc %s call %d M=%d" % (cfg.name, i, M))
        x, lg, ref, got = _pair(cfg, w, M, 71 + M, *scales)
        assert torch.equal(got["ids"], ref["ids"]) and torch.equal(got["counts"], ref["counts"])
        assert torch.equal(got["w"].view(torch.int32), ref["w"].view(torch.int32))
        assert torch.equal(got["y"], ref["y"]), "no-alloc output differs from the workspace entry point's"
        orc = run_oracle(cfg, x, lg, w, x_scale=scales[0], h_scale=scales[1])
        assert np.array_equal(got["ids"].numpy(), orc["ids"])
        e = err_norm(got["yf"], orc["y"])
        say("  err vs oracle %.3e" % e)
        assert e <= TOL[cfg.dtype]


def test_noalloc_refuses_oversized_calls_and_workspaces():
    cfg = MoEConfig("na_big", E=16, k=8, H=1024, I=1024, dtype="fp8", ms=(1,), logits="normal")
    w13, w2, s13, s2 = gen_weights(cfg, 72, device=DEV)
    t = lambda v: torch.tensor([v], dtype=torch.float32, device=DEV)
    M = 4096  # 32768 pairs: fp32 h alone is 128 MB, beyond the 64 MB scratch array
    x = torch.zeros(M, cfg.H, dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros(M, cfg.E, dtype=torch.float32, device=DEV)
    y = torch.empty(M, cfg.H, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoEError) as e:
        moe.fused_forward(x, lg, w13, w2, cfg.k, "fp8", t(s13), t(s2), out=y, noalloc=True)
    assert e.value.code == 2
    args = moe._FusedArgs(M=4, E=cfg.E, H=cfg.H, I=cfg.I, top_k=cfg.k, dtype=1, x=x.data_ptr(), logits=lg.data_ptr(),
                          w13=w13.data_ptr(), w2=w2.data_ptr(), w13_scale=t(s13).data_ptr(),
                          w2_scale=t(s2).data_ptr(), y=y.data_ptr(), workspace=y.data_ptr(), workspace_bytes=1 << 20)
    import ctypes
    assert moe.load().moe_fused_forward_noalloc(ctypes.byref(args), None) == 1


@pytest.mark.timeout(600)
def test_noalloc_random_shapes_match_workspace_entry_point():
    # every output of every random layer that fits the scratch array, bit for
    # bit, the calls one after another on the one array (larger after smaller
    # and the reverse)
    import test_gpu_random_shapes as rs
    fit = 0
    for c in rs.CASES + rs.TIE_CASES:
        ties = c["logits"].startswith("ties")
        cfg = MoEConfig("na%d" % c["i"], E=c["E"], k=c["k"], H=c["H"], I=c["I"], dtype=c["dtype"], ms=(c["M"],),
                        logits="normal" if ties else c["logits"])
        M, seed = c["M"], 7000 + c["i"]
        if c["M"] * (c["k"] + c["S"]) > 2048:
            continue  # the larger layers need more than the array
        gen = {0: gen_weights, 1: gen_weights_per_channel, 2: gen_weights_per_expert, 3: gen_weights_block}[c["mode"]]
        w = gen(cfg, seed, device=DEV, E=c["E"] + c["S"])
        x = gen_x(cfg.H, M, seed, sub=M)
        lg = (torch.from_numpy(np.random.default_rng(seed).integers(0, int(c["logits"][4:]), (M, c["E"]))
                               .astype(np.float32) * 0.5) if ties else gen_logits(cfg, M, seed, sub=M))
        say("no-alloc random %s" % rs._id(c))
        kw = dict(x_scale=c["xs"], h_scale=c["hs"], n_shared=c["S"], deterministic=c["det"])
        ref = run_gpu(cfg, x, lg, w, **kw)
        try:
            got = run_gpu(cfg, x, lg, w, noalloc=True, **kw)
        except moe.MoEError as e:
            assert e.code == 2, e.code  # beyond the array: refused before anything runs
            continue
        fit += 1
        for name in ("y_bits", "ids", "weights", "counts", "offsets", "sorted_ids", "block_expert", "num_padded",
                     "scales"):
            a, b = ref[name], got[name]
            if name == "sorted_ids":
                n = int(ref["num_padded"][0])
                a, b = a[:n], b[:n]
            assert (a is None and b is None) or np.array_equal(np.asarray(a).view(np.uint8),
                                                               np.asarray(b).view(np.uint8)), (rs._id(c), name)
        del w
    say("no-alloc: %d random layers fit the array" % fit)
    assert fit >= 40
