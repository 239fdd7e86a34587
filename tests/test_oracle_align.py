"""Pins of the oracle's sort-and-pad step.

The (token, slot) pairs f = m*k + j are grouped by expert, in increasing f
inside each group, and each group is padded with the sentinel P up to a
multiple of the block B; block_expert names the expert of every block.
Checked here against a comparison sort on the key (expert, f) and against the
invariants of the layout, not against a second counting sort.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, gen_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_layout(ids: np.ndarray, E: int, B: int, out: dict):
    f = ids.ravel()
    P = f.size
    counts, offsets, sid, be, total = (out["counts"], out["offsets"], out["sorted_ids"], out["block_expert"],
                                       out["num_padded"])
    assert np.array_equal(counts, np.bincount(f, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == total
    sizes = np.diff(offsets)
    assert (sizes % B == 0).all()
    assert ((sizes - counts >= 0) & (sizes - counts < B)).all()
    assert ((sizes == 0) == (counts == 0)).all()
    by_key = sorted(range(P), key=lambda i: (int(f[i]), i))
    got = [int(v) for v in sid[:total] if v != P]
    assert got == by_key  # stable grouping, all pairs exactly once
    for e in range(E):
        seg = sid[offsets[e]:offsets[e + 1]]
        assert (seg[:counts[e]] != P).all() and (seg[counts[e]:] == P).all()
        assert (f[seg[:counts[e]]] == e).all()
    nb = total // B
    for b in range(nb):
        e = be[b]
        assert offsets[e] <= b * B < offsets[e + 1]
    assert (be[nb:] == -1).all()


@pytest.mark.parametrize("B", [1, 4, 16, 32, 64, 128])
@pytest.mark.parametrize("name,M", [("tiny", 4), ("qwen3", 64), ("deepseek", 128), ("prefill", 512)])
def test_align_layout(name, M, B):
    cfg = CONFIGS[name]
    ids, _ = oracle.route(gen_logits(cfg, M, sub=M), cfg.k)
    out = oracle.align(ids, cfg.E, B)
    check_layout(ids, cfg.E, B, out)
    assert out["sorted_ids"].size == oracle.align_capacity(ids.size, cfg.E, B)


def test_align_random_ids_with_empty_experts():
    g = torch.Generator().manual_seed(11)
    ids = torch.randint(0, 5, (300, 3), generator=g).numpy().astype(np.int32) * 3  # only experts 0,3,..,12 of 16
    for B in (1, 2, 8, 16):
        check_layout(ids, 16, B, oracle.align(ids, 16, B))


def test_align_empty_input():
    out = oracle.align(np.zeros((0, 2), dtype=np.int32), 8, 16)
    assert out["num_padded"] == 0 and (out["counts"] == 0).all() and (out["offsets"] == 0).all()


def test_align_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 9]], dtype=np.int32), 8, 16)


def test_golden_align_example():
    with open(os.path.join(GOLDEN, "align_small.json")) as f:
        g = json.load(f)
    ids = np.array(g["ids"], dtype=np.int32)
    out = oracle.align(ids, g["E"], g["B"])
    assert out["counts"].tolist() == g["counts"]
    assert out["offsets"].tolist() == g["offsets"]
    assert out["sorted_ids"][:g["num_padded"]].tolist() == g["sorted_ids_prefix"]
    assert out["sorted_ids"].size == g["capacity"]
    assert out["block_expert"].tolist() == g["block_expert"]
    assert out["num_padded"] == g["num_padded"]
