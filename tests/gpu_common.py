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


def say(msg: str):
    sys.__stderr__.write("[gpu-test] %s\n" % msg)
    sys.__stderr__.flush()


def err_norm(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """max |y_gpu - y_ref| / max |y_ref| over the compared rows."""
    return float(np.abs(y_gpu - y_ref).max() / max(np.abs(y_ref).max(), 1e-30))


def run_gpu(cfg: MoEConfig, x, logits, weights, x_scale=None, h_scale=None, tuning=None, n_shared=0):
    """One fused forward on the GPU; returns host copies of y and intermediates
    (ids/weights [M,k+n_shared], counts [E+n_shared])."""
    w13, w2, s13, s2 = weights
    M = x.shape[0]
    fp8 = cfg.dtype == "fp8"
    # activation scales and per-tensor weight scales are floats; per-row
    # weight scales are [E,rows] tensors, passed as they are
    sc = lambda v: (None if v is None else v.to(DEV, torch.float32).contiguous() if isinstance(v, torch.Tensor)
                    else torch.tensor([v], dtype=torch.float32, device=DEV))
    ids = torch.full((M, cfg.k + n_shared), -1, dtype=torch.int32, device=DEV)
    wts = torch.zeros((M, cfg.k + n_shared), dtype=torch.float32, device=DEV)
    counts = torch.full((cfg.E + n_shared,), -1, dtype=torch.int32, device=DEV)
    scales = torch.zeros(2, dtype=torch.float32, device=DEV) if fp8 else None
    y = moe.fused_forward(x.to(DEV), logits.to(DEV), w13, w2, cfg.k, cfg.dtype,
                          w13_scale=sc(s13) if fp8 else None, w2_scale=sc(s2) if fp8 else None,
                          x_scale=sc(x_scale), h_scale=sc(h_scale), topk_ids=ids, topk_weights=wts,
                          expert_counts=counts, scales_out=scales, tuning=tuning, n_shared=n_shared)
    torch.cuda.synchronize()
    return dict(y=y.float().cpu().numpy().astype(np.float64), ids=ids.cpu().numpy(), weights=wts.cpu().numpy(),
                counts=counts.cpu().numpy(), scales=None if scales is None else scales.cpu().numpy())


def run_oracle(cfg: MoEConfig, x, logits, weights, tokens=None, x_scale=None, h_scale=None, n_shared=0):
    """Oracle on the same inputs; copies only the experts it needs to the host."""
    w13, w2, s13, s2 = weights
    ids, _ = oracle.route(logits, cfg.k)
    if tokens is None:
        tokens = list(range(x.shape[0]))
    fp8 = cfg.dtype == "fp8"
    all_h = fp8 and h_scale is None
    need = sorted(set(ids.ravel().tolist()) if all_h else set(ids[tokens].ravel().tolist()))
    need += [cfg.E + s for s in range(n_shared)]
    experts = {e: (w13[e].cpu(), w2[e].cpu()) for e in need}
    t0 = time.time()
    out = oracle.layer(x, logits, None, None, cfg.k, cfg.dtype, s13, s2, x_scale=x_scale, h_scale=h_scale,
                       tokens=tokens, experts=experts, n_shared=n_shared)
    out["seconds"] = time.time() - t0
    return out


def compare(cfg: MoEConfig, M: int, seed: int = 0, weights=None, tokens=None, x_scale=None, h_scale=None,
            tuning=None, logits=None, x=None, n_shared=0):
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
    gpu = run_gpu(cfg, x, logits, weights, x_scale, h_scale, tuning, n_shared)
    ref = run_oracle(cfg, x, logits, weights, tokens, x_scale, h_scale, n_shared)
    # routing: bit-exact ids and counts; the shared slots name E+s with weight one
    k = cfg.k
    assert np.array_equal(gpu["ids"][:, :k], ref["ids"]), "topk ids differ"
    counts = np.bincount(ref["ids"].ravel(), minlength=cfg.E)
    if n_shared:
        assert (gpu["ids"][:, k:] == cfg.E + np.arange(n_shared)).all(), "shared slots differ"
        assert (gpu["weights"][:, k:] == 1.0).all(), "shared weights differ"
        counts = np.concatenate([counts, np.full(n_shared, M)])
    assert np.array_equal(gpu["counts"], counts), "expert counts differ"
    assert np.allclose(gpu["weights"][:, :k], ref["weights"], rtol=1e-6, atol=1e-6), "topk weights differ"
    if cfg.dtype == "fp8":
        assert gpu["scales"][0] == np.float32(ref["s_x"]), (gpu["scales"][0], ref["s_x"])
        assert abs(gpu["scales"][1] / ref["s_h"] - 1) < 1e-4, (gpu["scales"][1], ref["s_h"])
    rows = list(range(M)) if tokens is None else list(tokens)
    e = err_norm(gpu["y"][rows], ref["y"])
    say("  err=%.3e (tol %.0e) oracle %.1fs" % (e, TOL[cfg.dtype], ref["seconds"]))
    assert np.isfinite(gpu["y"]).all()
    assert e <= TOL[cfg.dtype], "output error %.3e above %.0e" % (e, TOL[cfg.dtype])
    return e, gpu, ref
