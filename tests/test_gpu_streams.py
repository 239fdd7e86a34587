"""Fused calls on side streams, and two at once on two streams with their own
workspaces and outputs.

The library keeps nothing between calls outside the caller's workspace (the
single-launch layer's barrier counters and the no-alloc scratch array are
the documented exceptions, and neither runs here), so each call gives on a
side stream, and while another layer of another launch sequence runs beside
it, the bits it gives alone on the default stream: y, the routing outputs,
the expert counts and the fp8 scales.
"""
import itertools

import pytest
import torch

import moe_layer_align_amd as moe
from gpu_common import DEV, say
from synth import MoEConfig, gen_logits, gen_weights, gen_x

pytestmark = pytest.mark.gpu

# one layer per launch sequence the default plan picks
LAYERS = {
    "decode_bf16": (MoEConfig("s_dec_bf16", E=16, k=4, H=1024, I=768, dtype="bf16", ms=(1,), logits="normal"), 40),
    "decode_fp8": (MoEConfig("s_dec_fp8", E=64, k=8, H=1024, I=512, dtype="fp8", ms=(1,), logits="normal"), 40),
    "two_launches": (MoEConfig("s_two", E=16, k=4, H=1024, I=512, dtype="fp8", ms=(1,), logits="normal"), 3),
    "decode_token_down": (MoEConfig("s_tok", E=4, k=2, H=2048, I=8320, dtype="bf16", ms=(1,), logits="normal"), 1),
    "prefill": (MoEConfig("s_pf", E=16, k=8, H=512, I=512, dtype="fp8", ms=(1,), logits="zipf"), 1100),
}


class Layer:
    """Inputs, weights, workspace and outputs of one layer call; run() enqueues
    it on a stream and reads nothing back."""

    def __init__(self, name: str, seed: int):
        cfg, M = LAYERS[name]
        self.name, self.cfg, self.M = name, cfg, M
        fp8 = cfg.dtype == "fp8"
        assert moe.fused_path(M, cfg.E, cfg.H, cfg.I, cfg.k, cfg.dtype) == name.replace("_bf16", "").replace(
            "_fp8", ""), name
        self.w13, self.w2, s13, s2 = gen_weights(cfg, seed, device=DEV)
        t = lambda v: torch.tensor([v], dtype=torch.float32, device=DEV)
        self.s13, self.s2 = (t(s13), t(s2)) if fp8 else (None, None)
        self.x = gen_x(cfg.H, M, seed, sub=M).to(DEV)
        self.lg = gen_logits(cfg, M, seed, sub=M).to(DEV)
        self.ws = torch.empty(moe.workspace_size(M, cfg.E, cfg.H, cfg.I, cfg.k, cfg.dtype), dtype=torch.uint8,
                              device=DEV)
        self.y = torch.empty(M, cfg.H, dtype=torch.bfloat16, device=DEV)
        self.ids = torch.empty(M, cfg.k, dtype=torch.int32, device=DEV)
        self.wts = torch.empty(M, cfg.k, dtype=torch.float32, device=DEV)
        self.counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
        self.scales = torch.empty(2, dtype=torch.float32, device=DEV) if fp8 else None

    def run(self, stream):
        c = self.cfg
        moe.fused_forward(self.x, self.lg, self.w13, self.w2, c.k, c.dtype, self.s13, self.s2, out=self.y,
                          workspace=self.ws, topk_ids=self.ids, topk_weights=self.wts, expert_counts=self.counts,
                          scales_out=self.scales, stream=stream)

    def clear(self):
        for t in (self.y, self.ids, self.wts, self.counts, self.scales):
            if t is not None:
                t.fill_(-1) if t.dtype == torch.int32 else t.fill_(float("nan"))

    def bits(self):
        out = [self.y.view(torch.int16), self.ids, self.wts.view(torch.int32), self.counts]
        if self.scales is not None:
            out.append(self.scales.view(torch.int32))
        return [t.cpu().clone() for t in out]


@pytest.fixture(scope="module")
def layers():
    ls = {name: Layer(name, 90 + i) for i, name in enumerate(LAYERS)}
    ref = {}
    for name, l in ls.items():
        l.run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref[name] = l.bits()
    return ls, ref


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def test_side_stream_matches_default_stream(layers):
    ls, ref = layers
    s = torch.cuda.Stream()
    for name, l in ls.items():
        l.clear()
        torch.cuda.synchronize()
        l.run(s)
        s.synchronize()
        assert _same(l.bits(), ref[name]), name


@pytest.mark.parametrize("a,b", list(itertools.combinations(LAYERS, 2)))
def test_two_layers_at_once_on_two_streams(layers, a, b):
    ls, ref = layers
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    la, lb = ls[a], ls[b]
    for rep in range(3):
        say("streams %s | %s rep %d" % (a, b, rep))
        la.clear()
        lb.clear()
        torch.cuda.synchronize()
        # several calls of each queued back to back on its own stream, the
        # two streams free to interleave; the last call of each is checked
        for _ in range(3):
            (la if rep % 2 else lb).run(s1 if rep % 2 else s2)
            (lb if rep % 2 else la).run(s2 if rep % 2 else s1)
        torch.cuda.synchronize()
        assert _same(la.bits(), ref[a]), (a, "beside", b, rep)
        assert _same(lb.bits(), ref[b]), (b, "beside", a, rep)


def test_side_stream_with_the_bindings_own_workspace(layers):
    # no workspace given: the binding allocates one on the current stream and
    # drops it when the call returns, while the call still runs on the side
    # stream; the default stream meanwhile allocates and fills memory of the
    # same size, which must not land on the workspace in use
    ls, ref = layers
    s = torch.cuda.Stream()
    for name, l in ls.items():
        c = l.cfg
        outs = []
        for _ in range(4):
            y = torch.empty_like(l.y)
            moe.fused_forward(l.x, l.lg, l.w13, l.w2, c.k, c.dtype, l.s13, l.s2, out=y, stream=s)
            junk = torch.empty_like(l.ws)
            junk.fill_(0x5A)
            outs.append(y)
        torch.cuda.synchronize()
        for y in outs:
            assert torch.equal(y.view(torch.int16).cpu(), ref[name][0]), name
