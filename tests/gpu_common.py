"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import moe_layer_align_amd as moe
import oracle
from synth import MoEConfig, gen_logits, gen_weights, gen_x

DEV = torch.device("cuda:0")
TOL = {"bf16": 1e-2, "fp8": 3e-2}
GUARD = 64  # canary elements before and after every caller-visible output


class Guarded:
    """A GPU output with GUARD canary elements on both sides.  The interior is
    pre-filled with the same pattern, so every element the call must write
    is checked to have been written (by the comparisons that follow) and
    nothing past either end may change."""

    def __init__(self, shape, dtype, pattern: int):
        n = int(np.prod(shape))
        raw = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.int32: torch.int32}[dtype]
        self.n, self.pattern = n, pattern
        self.buf = torch.full((n + 2 * GUARD,), pattern, dtype=raw, device=DEV)
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(*shape)

    def check(self, name: str):
        b = self.buf.cpu()
        assert bool((b[:GUARD] == self.pattern).all()), "%s: canary before the output overwritten" % name
        assert bool((b[GUARD + self.n:] == self.pattern).all()), "%s: canary after the output overwritten" % name


def say(msg: str):
    sys.__stderr__.write("[gpu-test] %s\n" % msg)
    sys.__stderr__.flush()


def err_norm(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """max |y_gpu - y_ref| / max |y_ref| over the compared rows."""
    return float(np.abs(y_gpu - y_ref).max() / max(np.abs(y_ref).max(), 1e-30))


def row_errs(y_gpu: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per token max_n |dy_m| / max_n |y_ref_m|, so that rows of small
    magnitude are held to the same bound."""
    num = np.abs(y_gpu - y_ref).max(axis=1)
    den = np.maximum(np.abs(y_ref).max(axis=1), 1e-30)
    return num / den


# Per-token bound of the fp8 modes.  The fp8 matrix instructions of gfx950
# do not sum their products at fp32 precision: against exact sums of random
# e4m3 operands spread over the format's range, their results are off by up
# to about 2^-13 of the sum of |products| (both the 16x16x128 and the
# 16x16x32 forms; narrow-range operands and the fp32 accumulator add are
# exact).  So the kernel's fp32 h differs from the definition's by ~1e-4 of
# its row and some of h's e4m3 rounding decisions come out on the other side
# of a midpoint.  A step in the format's top binades is 1/8 to 1/16 of the
# value, so one such decision on a large h element moves its token's outputs
# by a few percent of their largest value, more often the more tokens and
# the smaller I.  Block scaling puts every 128-element group's largest values
# in the top binade: its per-token maximum is about 1.3e-2 at 600 tokens,
# 2.4e-2 at 1100 and 3.0e-2 at 4096.  With one h scale per layer, a layer of
# 2780 tokens, top-3 of 31 experts, H = 896, I = 384 reaches 3.1e-2 on one
# token (whole output 1.1e-2), every one of its worst tokens' differences
# made of such flips.  The whole-output bound TOL holds in every mode.
TOL_TOKEN_FP8 = 5e-2


def run_gpu(cfg: MoEConfig, x, logits, weights, x_scale=None, h_scale=None, tuning=None, n_shared=0,
            deterministic=False, noalloc=False):
    """One fused forward on the GPU (the no-alloc entry point with noalloc);
    returns host copies of y and intermediates (ids/weights [M,k+n_shared],
    counts [E+n_shared], the sort-and-pad outputs).  Every output sits
    between canaries, checked after the call."""
    w13, w2, s13, s2 = weights
    M = x.shape[0]
    fp8 = cfg.dtype == "fp8"
    ES, KS = cfg.E + n_shared, cfg.k + n_shared
    # activation scales and per-tensor weight scales are floats; per-row
    # weight scales are [E,rows] tensors, passed as they are
    # (uint8 block-scale codes pass unchanged)
    sc = lambda v: (None if v is None else v.to(DEV).contiguous() if isinstance(v, torch.Tensor) and
                    v.dtype == torch.uint8 else v.to(DEV, torch.float32).contiguous() if isinstance(v, torch.Tensor)
                    else torch.tensor([v], dtype=torch.float32, device=DEV))
    block_scaled = isinstance(s13, torch.Tensor) and s13.dtype == torch.uint8
    blk, cap = moe.fused_align_shape(M, ES, cfg.H, cfg.I, KS, cfg.dtype, deterministic, 3 if block_scaled else 0)
    out = dict(y=Guarded((M, cfg.H), torch.bfloat16, 0x7FC1), ids=Guarded((M, KS), torch.int32, -7),
               weights=Guarded((M, KS), torch.float32, 0x7FC00007), counts=Guarded((ES,), torch.int32, -7),
               offsets=Guarded((ES + 1,), torch.int32, -7), sorted_ids=Guarded((cap,), torch.int32, -7),
               block_expert=Guarded((cap // blk,), torch.int32, -7), num_padded=Guarded((1,), torch.int32, -7))
    if fp8:
        out["scales"] = Guarded((2,), torch.float32, 0x7FC00007)
    y = moe.fused_forward(x.to(DEV), logits.to(DEV), w13, w2, cfg.k, cfg.dtype,
                          w13_scale=sc(s13) if fp8 else None, w2_scale=sc(s2) if fp8 else None,
                          x_scale=sc(x_scale), h_scale=sc(h_scale), out=out["y"].t, topk_ids=out["ids"].t,
                          topk_weights=out["weights"].t, expert_counts=out["counts"].t,
                          scales_out=out["scales"].t if fp8 else None, tuning=tuning, n_shared=n_shared,
                          align_out={key: out[key].t for key in ("offsets", "sorted_ids", "block_expert",
                                                                  "num_padded")},
                          deterministic=deterministic, noalloc=noalloc)
    torch.cuda.synchronize()
    assert y.data_ptr() == out["y"].t.data_ptr()
    for name, g in out.items():
        g.check(name)
    res = {name: g.t.cpu().numpy() for name, g in out.items() if name != "y"}
    res["y"] = out["y"].t.float().cpu().numpy().astype(np.float64)
    res["y_bits"] = out["y"].t.view(torch.int16).cpu().numpy()
    res.setdefault("scales", None)
    res["block"] = blk
    return res


def check_align(gpu: dict, ids_full: np.ndarray, E: int):
    """The fused call's sort-and-pad outputs equal the oracle's for its block
    size, bit for bit (entries of sorted_ids past the padded total are
    unspecified and not compared)."""
    ref = oracle.align(ids_full, E, gpu["block"])
    n = int(gpu["num_padded"][0])
    assert n == ref["num_padded"], (n, ref["num_padded"])
    assert np.array_equal(gpu["counts"], ref["counts"]), "expert counts differ"
    assert np.array_equal(gpu["offsets"], ref["offsets"]), "expert offsets differ"
    assert np.array_equal(gpu["sorted_ids"][:n], ref["sorted_ids"][:n]), "sorted ids differ"
    assert np.array_equal(gpu["block_expert"], ref["block_expert"]), "block map differs"


def run_oracle(cfg: MoEConfig, x, logits, weights, tokens=None, x_scale=None, h_scale=None, n_shared=0):
    """Oracle on the same inputs; copies only the experts it needs to the host."""
    w13, w2, s13, s2 = weights
    ids, _ = oracle.route(logits, cfg.k)
    if tokens is None:
        tokens = list(range(x.shape[0]))
    fp8 = cfg.dtype == "fp8"
    # uint8 weight scales: E8M0 codes of 128 x 128 blocks (block-scaled mode),
    # whose activation scales are per group (no h amax over all pairs)
    blk = isinstance(s13, torch.Tensor) and s13.dtype == torch.uint8
    all_h = fp8 and h_scale is None and not blk
    need = sorted(set(ids.ravel().tolist()) if all_h else set(ids[tokens].ravel().tolist()))
    need += [cfg.E + s for s in range(n_shared)]
    experts = {e: (w13[e].cpu(), w2[e].cpu()) for e in need}
    t0 = time.time()
    if blk:
        out = oracle.layer(x, logits, None, None, cfg.k, cfg.dtype, x_scale=x_scale, h_scale=h_scale, tokens=tokens,
                           experts=experts, n_shared=n_shared, w13_block=s13.cpu(), w2_block=s2.cpu())
    else:
        out = oracle.layer(x, logits, None, None, cfg.k, cfg.dtype, s13, s2, x_scale=x_scale, h_scale=h_scale,
                           tokens=tokens, experts=experts, n_shared=n_shared)
    out["seconds"] = time.time() - t0
    return out


def compare(cfg: MoEConfig, M: int, seed: int = 0, weights=None, tokens=None, x_scale=None, h_scale=None,
            tuning=None, logits=None, x=None, n_shared=0, deterministic=False):
    """Full parity check of one layer call; returns (err, gpu, ref).  With
    n_shared, `weights` (default: drawn for E+n_shared experts) hold the shared
    experts after the routed ones."""
    if x is None:
        x = gen_x(cfg.H, M, seed, sub=M)
    if logits is None:
        logits = gen_logits(cfg, M, seed, sub=M)
    if weights is None:
        weights = gen_weights(cfg, seed, device=DEV, E=cfg.E + n_shared)
    say("%s M=%d dtype=%s xs=%s hs=%s shared=%d" % (cfg.name, M, cfg.dtype, x_scale, h_scale, n_shared))
    gpu = run_gpu(cfg, x, logits, weights, x_scale, h_scale, tuning, n_shared, deterministic)
    ref = run_oracle(cfg, x, logits, weights, tokens, x_scale, h_scale, n_shared)
    # routing: bit-exact ids and counts; the shared slots name E+s with weight one
    k = cfg.k
    assert np.array_equal(gpu["ids"][:, :k], ref["ids"]), "topk ids differ"
    counts = np.bincount(ref["ids"].ravel(), minlength=cfg.E)
    ids_full = ref["ids"]
    if n_shared:
        assert (gpu["ids"][:, k:] == cfg.E + np.arange(n_shared)).all(), "shared slots differ"
        assert (gpu["weights"][:, k:] == 1.0).all(), "shared weights differ"
        counts = np.concatenate([counts, np.full(n_shared, M)])
        ids_full = np.concatenate([ref["ids"], np.tile(cfg.E + np.arange(n_shared, dtype=np.int32), (M, 1))], axis=1)
    assert np.array_equal(gpu["counts"], counts), "expert counts differ"
    check_align(gpu, np.ascontiguousarray(ids_full, dtype=np.int32), cfg.E + n_shared)
    assert np.allclose(gpu["weights"][:, :k], ref["weights"], rtol=1e-6, atol=1e-6), "topk weights differ"
    if cfg.dtype == "fp8":
        assert gpu["scales"][0] == np.float32(ref["s_x"]), (gpu["scales"][0], ref["s_x"])
        if ref["s_h"] == 0.0:  # block-scaled: no tensor scales, both reported as 0
            assert gpu["scales"][1] == 0.0, gpu["scales"][1]
        else:
            assert abs(gpu["scales"][1] / ref["s_h"] - 1) < 1e-4, (gpu["scales"][1], ref["s_h"])
    rows = list(range(M)) if tokens is None else list(tokens)
    e = err_norm(gpu["y"][rows], ref["y"])
    er = float(row_errs(gpu["y"][rows], ref["y"]).max()) if rows else 0.0
    tol_tok = TOL_TOKEN_FP8 if cfg.dtype == "fp8" else TOL[cfg.dtype]
    say("  err=%.3e per-token %.3e (tol %.0e, per token %.0e) on %s tokens, oracle %.1fs"
        % (e, er, TOL[cfg.dtype], tol_tok, "all" if tokens is None else len(rows), ref["seconds"]))
    assert np.isfinite(gpu["y"]).all()
    assert e <= TOL[cfg.dtype], "output error %.3e above %.0e" % (e, TOL[cfg.dtype])
    assert er <= tol_tok, "per-token output error %.3e above %.0e" % (er, tol_tok)
    return e, gpu, ref
