"""GPU parity of the single-step entry points against the CPU oracle:
e4m3 quantisation (bit-exact codes), router logits (within fp32 summation
error, bitwise the same for a token in any batch), router top-k (bit-exact
ids), align (bit-exact counts, offsets, sorted ids, block map), on fixed and on seeded random shapes."""
import numpy as np
import pytest
import torch

import moe_layer_align_amd as moe
import oracle
from gpu_common import DEV, say
from synth import CONFIGS, gen_logits, gen_router_weights, gen_x

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ e4m3
def _codec_inputs():
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    eps = np.spacing(mids.astype(np.float32))
    g = np.random.default_rng(0)
    rnd = (g.standard_normal(50001) * np.exp(g.standard_normal(50001) * 3)).astype(np.float32)
    v = np.concatenate([pos, -pos, mids, -mids, mids + eps, mids - eps, -(mids + eps),
                        [447.9, 448.0, 448.1, 463.9, 464.0, 500.0, 1e10, -1e10, 2.0 ** -11, -2.0 ** -11], rnd])
    return v.astype(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.37, 5.0e-3, 81.0])
def test_quant_e4m3_bit_exact(scale):
    v = _codec_inputs()
    say("quant n=%d scale=%g" % (v.size, scale))
    out = moe.quant_e4m3(torch.from_numpy(v).to(DEV), torch.tensor([scale], dtype=torch.float32, device=DEV))
    got = out.cpu().numpy()
    r = np.float32(1.0) / np.float32(scale)
    t = (v * r).astype(np.float32)
    ref = oracle.e4m3_encode(t)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(t[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_quant_e4m3_tail_sizes():
    for n in (1, 3, 5, 1023, 1025):
        v = np.linspace(-600, 600, n).astype(np.float32)
        out = moe.quant_e4m3(torch.from_numpy(v).to(DEV), torch.ones(1, device=DEV))
        assert np.array_equal(out.cpu().numpy(), oracle.e4m3_encode(v))


# ------------------------------------------------------------------ router
def _route_case(lg: np.ndarray, k: int):
    ids, w = moe.route_topk(torch.from_numpy(lg).to(DEV), k)
    torch.cuda.synchronize()
    rid, rw = oracle.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen3", "deepseek", "prefill"])
def test_route_configs(name):
    cfg = CONFIGS[name]
    for M in sorted(set(cfg.ms) | {1, 63, 64, 65}):
        say("route %s M=%d" % (name, M))
        _route_case(gen_logits(cfg, M, sub=M).numpy(), cfg.k)


@pytest.mark.parametrize("E,k", [(1, 1), (2, 2), (8, 8), (64, 16), (65, 3), (130, 7), (256, 16), (512, 16), (512, 1)])
def test_route_shapes(E, k):
    g = np.random.default_rng(E * 100 + k)
    lg = g.standard_normal((37, E)).astype(np.float32)
    _route_case(lg, k)


def test_route_ties_and_signed_zero():
    E = 200
    lg = np.zeros((6, E), dtype=np.float32)
    lg[0] = 1.0                               # all equal
    lg[1, ::2] = -0.0                         # -0 and +0 tie
    lg[2] = np.repeat(np.arange(E // 8), 8)   # runs of 8 equal values
    lg[3, 150:] = 5.0                         # ties beyond the first 64-lane slice
    lg[4] = np.float32(-3.0)
    lg[4, [199, 64, 128, 0]] = 2.0
    lg[5] = np.random.default_rng(1).integers(-2, 3, E).astype(np.float32)
    for k in (1, 4, 8, 16):
        _route_case(lg, k)


def _random_route_cases(n=30, seed=4242):
    # seeded (M, E, k, levels): M across the one-wave, one-workgroup and
    # multi-workgroup sizes, E up to 512, logits continuous (levels 0) or from
    # a few values, so that ties decide most selections
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(g.choice([1, 2, 3, 7, 8, 16, 33, 64, 100, 128, 255, 256, 257, 384, 512]))
        k = int(g.integers(1, min(E, 16) + 1))
        M = int(round(np.exp(g.uniform(0, np.log(5000)))))
        out.append((M, E, k, int(g.choice([0, 0, 2, 3, 7]))))
    return out


@pytest.mark.parametrize("M,E,k,levels", _random_route_cases())
def test_route_random(M, E, k, levels):
    g = np.random.default_rng(M * 1000003 + E * 17 + k)
    if levels:
        lg = (g.integers(0, levels, (M, E)) * 0.25 - 0.5).astype(np.float32)
    else:
        lg = g.standard_normal((M, E)).astype(np.float32)
    _route_case(lg, k)


# ------------------------------------------------------------------ align
def _align_case(ids: np.ndarray, E: int, B: int):
    dev = moe.align(torch.from_numpy(ids).to(DEV), E, B)
    torch.cuda.synchronize()
    ref = oracle.align(ids, E, B)
    n = int(dev["num_padded"].item())
    assert n == ref["num_padded"]
    assert np.array_equal(dev["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(dev["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(dev["sorted_ids"].cpu().numpy()[:n], ref["sorted_ids"][:n])
    assert np.array_equal(dev["block_expert"].cpu().numpy(), ref["block_expert"])
    return dev


@pytest.mark.parametrize("P,E,B", [(0, 8, 16), (1, 8, 16), (8, 8, 1), (63, 8, 16), (1023, 8, 64), (1024, 128, 16),
                                   (1025, 128, 16), (4096, 256, 32), (32768, 128, 64), (5000, 512, 256),
                                   (3000, 1, 16), (777, 3, 128)])
def test_align_random(P, E, B):
    say("align P=%d E=%d B=%d" % (P, E, B))
    g = np.random.default_rng(P + E + B)
    ids = g.integers(0, E, P).astype(np.int32).reshape(-1, 1)
    _align_case(ids, E, B)


def _random_align_cases(n=30, seed=4343):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(g.choice([1, 2, 5, 8, 31, 64, 128, 200, 256, 300, 512]))
        k = int(g.integers(1, min(E, 16) + 1))
        M = int(round(np.exp(g.uniform(0, np.log(6000)))))
        B = int(2 ** g.integers(0, 9))
        out.append((M, E, k, B))
    return out


@pytest.mark.parametrize("M,E,k,B", _random_align_cases())
def test_align_random_shapes(M, E, k, B):
    # ids as routing gives them (distinct experts per token), some experts
    # far more popular than others
    g = np.random.default_rng(M * 7919 + E * 31 + k * 7 + B)
    lg = (g.standard_normal((M, E)) + np.log(np.arange(1, E + 1))[g.permutation(E)] * -1.5).astype(np.float32)
    ids, _ = oracle.route(lg, k)
    _align_case(ids, E, B)


def test_align_skewed_and_empty_experts():
    cfg = CONFIGS["prefill"]
    rid, _ = oracle.route(gen_logits(cfg, 4096, sub=4096).numpy(), cfg.k)
    for B in (16, 64, 128):
        _align_case(rid, cfg.E, B)


def test_align_deterministic():
    ids = np.random.default_rng(5).integers(0, 64, (4096, 8)).astype(np.int32)
    t = torch.from_numpy(ids).to(DEV)
    a = moe.align(t, 64, 16)
    n = int(a["num_padded"].item())
    for _ in range(100):
        b = moe.align(t, 64, 16)
        assert int(b["num_padded"].item()) == n
        assert torch.equal(a["sorted_ids"][:n], b["sorted_ids"][:n])  # entries past num_padded are unspecified


def test_align_out_of_range_ids_flagged():
    ids = np.array([[0, 1], [9, 2], [-1, 3]], dtype=np.int32)
    dev = moe.align(torch.from_numpy(ids).to(DEV), 8, 16)
    torch.cuda.synchronize()
    assert int(dev["num_padded"].item()) == -1
    assert dev["counts"].cpu().numpy().tolist() == [1, 1, 1, 1, 0, 0, 0, 0]


# ------------------------------------------------------------------ router logits
@pytest.mark.parametrize("M,E,H", [(1, 8, 4096), (5, 128, 2048), (63, 256, 7168), (300, 128, 4096), (17, 7, 256),
                                   (4096, 128, 4096)])
def test_router_logits(M, E, H):
    say("router logits M=%d E=%d H=%d" % (M, E, H))
    x = gen_x(H, M, 40 + E, sub=M)
    w = gen_router_weights(E, H, 40 + E)
    out = moe.router_logits(x.to(DEV), w.to(DEV)).cpu().numpy()
    ref = oracle.router_logits(x, w)
    # fp32 sums of H bf16 products in another order: far below 1e-5 of the
    # logits' scale
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max() + 1e-6
    # a token's logits do not depend on the batch it is in
    one = moe.router_logits(x[:1].to(DEV), w.to(DEV)).cpu().numpy()
    assert np.array_equal(one[0], out[0])
