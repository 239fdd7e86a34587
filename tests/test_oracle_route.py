"""Pins of the oracle's routing: brute-force sorts and closed forms.

Routing selects, per token, the k experts with the largest router logits
(ties to the lower expert index, slot order by decreasing logit) and weights
them with the softmax over the selected logits.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, gen_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_topk(logits: np.ndarray, k: int) -> np.ndarray:
    out = []
    for row in logits:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("name,M", [("tiny", 4), ("mixtral", 63), ("qwen3", 64), ("deepseek", 128), ("prefill", 256)])
def test_topk_matches_stable_sort(name, M):
    cfg = CONFIGS[name]
    lg = gen_logits(cfg, M, seed=0, sub=M).numpy()
    ids, w = oracle.route(lg, cfg.k)
    assert np.array_equal(ids, brute_topk(lg, cfg.k))
    # weights: non-increasing in slot order, sum to one within k ulps
    assert (np.diff(w.astype(np.float64), axis=1) <= 0).all()
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() <= cfg.k * 2.0 ** -24


def test_weights_equal_renormalised_full_softmax():
    g = torch.Generator().manual_seed(3)
    lg = torch.randn(50, 16, generator=g, dtype=torch.float32)
    ids, w = oracle.route(lg.numpy(), 5)
    full = torch.softmax(lg.double(), dim=1).numpy()
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    ref = sel / sel.sum(1, keepdims=True)
    assert np.abs(w - ref).max() <= 2.0 ** -24 * 2


def test_k_equals_E_is_softmax():
    g = torch.Generator().manual_seed(4)
    lg = torch.randn(20, 8, generator=g, dtype=torch.float32)
    ids, w = oracle.route(lg.numpy(), 8)
    ref = torch.softmax(lg.double(), dim=1).numpy()
    back = np.take_along_axis(ref, ids.astype(np.int64), 1).astype(np.float32)
    ulp = np.spacing(np.abs(back))
    assert (np.abs(w - back) <= ulp).all()


def test_top1_weight_is_exactly_one():
    g = torch.Generator().manual_seed(5)
    lg = torch.randn(30, 64, generator=g, dtype=torch.float32).numpy()
    ids, w = oracle.route(lg, 1)
    assert (w == 1.0).all()
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))  # numpy argmax: first maximal index


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_all_equal_logits(k):
    lg = np.full((3, 16), 0.25, dtype=np.float32)
    ids, w = oracle.route(lg, k)
    assert (ids == np.arange(k)).all()
    assert (w == np.float32(1.0 / k)).all()  # exact for powers of two


def test_ties_at_kth_boundary_and_signed_zero():
    lg = np.array([
        [1.0, 3.0, 2.0, 2.0, 2.0, 0.0],   # k=3: 1, then 2 and 3 (lower indices among the tied 2.0s)
        [-0.0, 0.0, -1.0, -0.0, 0.0, -2.0],  # all zeros tie: 0, 1, 3
        [5.0, 5.0, 5.0, 5.0, 5.0, 5.0],
    ], dtype=np.float32)
    ids, _ = oracle.route(lg, 3)
    assert ids.tolist() == [[1, 2, 3], [0, 1, 3], [0, 1, 2]]
    assert np.array_equal(ids, brute_topk(lg, 3))


def test_nonfinite_rejected():
    lg = np.zeros((2, 4), dtype=np.float32)
    lg[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.route(lg, 2)


def test_golden_route_example():
    with open(os.path.join(GOLDEN, "route_ties.json")) as f:
        g = json.load(f)
    lg = np.array(g["logits"], dtype=np.float32)
    ids, w = oracle.route(lg, g["k"])
    assert ids.tolist() == g["ids"]
    # closed form written in the fixture: softmax over {0.5, 0.5, 0}
    d = 2 + math.exp(-0.5)
    expect = np.array([[1 / d, 1 / d, math.exp(-0.5) / d]])
    assert np.allclose(w.astype(np.float64), expect, rtol=2.0 ** -23, atol=0)


def test_zipf_logits_leave_experts_empty():
    cfg = CONFIGS["prefill"]
    lg = gen_logits(cfg, 4096, seed=0, sub=4096).numpy()
    ids, _ = oracle.route(lg, cfg.k)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    assert (counts == 0).sum() >= 4
    assert counts.sum() == 4096 * cfg.k
