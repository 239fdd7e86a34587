"""GPU tests of the deterministic mode (moe_fused_args_t.deterministic = 1).

A token's routing, routing weights and output are the same bits whatever
batch it is in and wherever it sits there: alone, in batches of 17 and 64,
and in a batch of 1100 tokens whose pairs would send the default mode to the
tiled prefill products; in bf16 and in fp8 with static activation scales.
Two separate processes, one after the other, produce byte-identical files.
The mode's outputs also match the oracle within the usual tolerance.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import moe_layer_align_amd as moe
from gpu_common import DEV, compare, say
from synth import MoEConfig, gen_logits, gen_weights, gen_x

pytestmark = pytest.mark.gpu

BF16 = MoEConfig("det_bf16", E=16, k=4, H=512, I=384, dtype="bf16", ms=(1,), logits="normal")
FP8 = MoEConfig("det_fp8", E=64, k=8, H=1024, I=768, dtype="fp8", ms=(1,), logits="normal")
XS, HS = 0.013, 0.004


def _run(cfg, w, x, lg):
    w13, w2, s13, s2 = w
    M = x.shape[0]
    ids = torch.empty(M, cfg.k, dtype=torch.int32, device=DEV)
    wts = torch.empty(M, cfg.k, dtype=torch.float32, device=DEV)
    kw = {}
    if cfg.dtype == "fp8":
        t = lambda v: torch.tensor([v], dtype=torch.float32, device=DEV)
        kw = dict(w13_scale=t(s13), w2_scale=t(s2), x_scale=t(XS), h_scale=t(HS))
    y = moe.fused_forward(x.to(DEV), lg.to(DEV), w13, w2, cfg.k, cfg.dtype, topk_ids=ids, topk_weights=wts,
                          deterministic=True, **kw)
    torch.cuda.synchronize()
    return ids.cpu(), wts.cpu(), y.view(torch.int16).cpu()


@pytest.mark.parametrize("cfg", [BF16, FP8], ids=["bf16", "fp8_static"])
def test_token_bits_independent_of_batch(cfg):
    w = gen_weights(cfg, 51, device=DEV)
    x1 = gen_x(cfg.H, 1, 51, sub=1)
    lg1 = gen_logits(cfg, 1, 51, sub=1)
    ids1, w1, y1 = _run(cfg, w, x1, lg1)
    for M, pos in ((17, 0), (17, 16), (64, 5), (64, 63), (1100, 0), (1100, 777), (1100, 1099)):
        say("deterministic %s token at %d of %d" % (cfg.name, pos, M))
        x = gen_x(cfg.H, M, 52 + M, sub=M)
        lg = gen_logits(cfg, M, 52 + M, sub=M)
        x[pos] = x1[0]
        lg[pos] = lg1[0]
        ids, wts, y = _run(cfg, w, x, lg)
        assert torch.equal(ids[pos], ids1[0]), (M, pos)
        assert torch.equal(wts[pos].view(torch.int32), w1[0].view(torch.int32)), (M, pos)
        assert torch.equal(y[pos], y1[0]), (M, pos)


@pytest.mark.parametrize("cfg,M", [(BF16, 70), (FP8, 40), (FP8, 1100)], ids=["bf16_70", "fp8_40", "fp8_1100"])
def test_deterministic_mode_matches_oracle(cfg, M):
    kw = dict(x_scale=XS, h_scale=HS) if cfg.dtype == "fp8" else {}
    compare(cfg, M, seed=53, deterministic=True, **kw)


def test_deterministic_mode_with_shared_expert():
    compare(FP8, 300, seed=54, deterministic=True, x_scale=XS, h_scale=HS, n_shared=1)


def test_two_processes_write_the_same_bytes(tmp_path):
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "det_child.py")
    files = []
    for i in range(2):
        out = str(tmp_path / ("run%d.npz" % i))
        say("deterministic child process %d" % i)
        subprocess.run([sys.executable, child, out], check=True, timeout=300)
        files.append(np.load(out))
    a, b = files
    assert sorted(a.files) == sorted(b.files)
    for key in a.files:
        assert a[key].tobytes() == b[key].tobytes(), key
