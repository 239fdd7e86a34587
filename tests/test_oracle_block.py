"""Pins of the oracle's block-scaled FP8 mode (CPU only).

Block quantisation (oracle_block_quant) is checked by brute force and by
properties that a mistake in the exponent rule, the rounding or the
saturation breaks: every element maps to the nearest of all 256 E4M3 codes
times the block scale (ties to the even code, saturation at 448), the
largest element lands in the format's top octave [256, 512), scaling a block
by 2^j moves only its scale code, and zero or tiny blocks take the smallest
scale.  The layer in block mode with one expert and top-1 equals a float64
SwiGLU of the dequantised operands (weights times their 128 x 128 block
scales, activations quantised per 128 elements), evaluated with library
matmuls; and a token's output does not depend on the other tokens of the
batch (no per-tensor amax).
"""
import numpy as np
import pytest
import torch

import oracle

E4M3 = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))


def nearest_code(t: float) -> int:
    """Brute force: the E4M3 code nearest to t (finite codes only), ties to
    the even code; beyond 448 the largest magnitude."""
    finite = [c for c in range(256) if np.isfinite(E4M3[c])]
    if abs(t) >= 448:
        return 0x7E | (0x80 if t < 0 else 0)
    d = np.array([abs(E4M3[c] - t) for c in finite])
    best = d.min()
    cands = [c for c, dd in zip(finite, d) if dd == best]
    if len(cands) > 1:  # a tie between two neighbours (or +-0): the even mantissa
        even = [c for c in cands if c % 2 == 0]
        cands = even or cands
        if t >= 0:
            cands = [c for c in cands if c < 0x80] or cands
        else:
            cands = [c for c in cands if c >= 0x80] or cands
    return cands[0]


def test_e8m0_values():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert oracle.e8m0_value(130) == 8.0
    assert np.isnan(oracle.e8m0_value(255))


@pytest.mark.parametrize("seed", range(6))
def test_block_quant_is_nearest_code_times_scale(seed):
    g = np.random.default_rng(seed)
    v = (g.standard_normal(128) * np.exp(g.standard_normal(128) * 2) * 10.0 ** g.integers(-6, 6)).astype(np.float32)
    codes, c = oracle.block_quant(v)
    scale = 2.0 ** (c - 127)
    for x, q in zip(v, codes):
        t = np.float32(x) * np.float32(1.0 / scale)  # exact: a power of two
        assert q == nearest_code(float(t)) or E4M3[q] == E4M3[nearest_code(float(t))], (x, q)


@pytest.mark.parametrize("seed", range(6))
def test_block_quant_exponent_window(seed):
    g = np.random.default_rng(100 + seed)
    v = (g.standard_normal(128) * 10.0 ** g.integers(-30, 30)).astype(np.float32)
    codes, c = oracle.block_quant(v)
    amax = float(np.abs(v).max())
    # the largest magnitude lands in [256, 512) after division by the scale
    t = amax * 2.0 ** (127 - c)
    assert 256.0 <= t < 512.0
    # its dequantised value is within half an E4M3 step (32 at that octave) or saturates at 448
    i = int(np.abs(v).argmax())
    deq = E4M3[codes[i]] * 2.0 ** (c - 127)
    assert abs(abs(deq) - min(t, 448.0) * 2.0 ** (c - 127)) <= 16.0 * 2.0 ** (c - 127)


def test_block_quant_power_of_two_shift():
    g = np.random.default_rng(7)
    v = g.standard_normal(128).astype(np.float32)
    codes, c = oracle.block_quant(v)
    for j in (-20, -3, -1, 1, 5, 40):
        codes2, c2 = oracle.block_quant((v * np.float32(2.0 ** j)).astype(np.float32))
        assert c2 == c + j and np.array_equal(codes2, codes)


def test_block_quant_zero_and_tiny_blocks():
    codes, c = oracle.block_quant(np.zeros(128, dtype=np.float32))
    assert c == 0 and not codes.any()
    # subnormal: the smallest scale 2^-127, at which 1e-40 is still an E4M3
    # value (about 0.017, within half a step)
    tiny = np.full(128, 1e-40, dtype=np.float32)
    codes, c = oracle.block_quant(tiny)
    deq = E4M3[codes] * 2.0 ** -127
    assert c == 0 and (np.abs(deq - np.float64(np.float32(1e-40))) <= 0.0625 * 1e-40).all()
    small = np.full(16, 2.0 ** -110, dtype=np.float32)
    codes, c = oracle.block_quant(small)
    assert c == (127 - 110) - 8 and (E4M3[codes] * 2.0 ** (c - 127) == 2.0 ** -110).all()


def _block_weights(E, rows, cols, seed):
    """e4m3 codes and E8M0 block codes [E, rows/128, cols/128], the blocks'
    scales spread over a factor 64 so that a scale taken from a wrong block
    shows."""
    g = np.random.default_rng(seed)
    codes = g.integers(0, 256, size=(E, rows, cols), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x01  # no NaN codes
    blocks = g.integers(118, 124, size=(E, rows // 128, cols // 128), dtype=np.uint8)
    return codes, blocks


def _dequant_weights(codes, blocks):
    e, rows, cols = codes.shape
    scale = np.repeat(np.repeat(2.0 ** (blocks.astype(np.float64) - 127), 128, axis=1), 128, axis=2)
    return E4M3[codes.ravel()].reshape(codes.shape) * scale


def _dequant_rows(a: np.ndarray) -> np.ndarray:
    """Per-128-element block quantisation of each row, dequantised (float64)."""
    out = np.empty(a.shape, dtype=np.float64)
    for r in range(a.shape[0]):
        for g in range(0, a.shape[1], 128):
            codes, c = oracle.block_quant(a[r, g:g + 128])
            out[r, g:g + 128] = E4M3[codes] * 2.0 ** (c - 127)
    return out


def test_block_layer_single_expert_is_swiglu_of_dequantised_operands():
    H, I, M = 256, 384, 5
    w13, b13 = _block_weights(1, 2 * I, H, 1)
    w2, b2 = _block_weights(1, H, I, 2)
    g = np.random.default_rng(3)
    # tokens and their 128-element groups at different magnitudes
    xf = g.standard_normal((M, H)) * (2.0 ** np.arange(M))[:, None] * np.repeat([1.0, 40.0], 128)[None, :]
    x = torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16)
    lg = torch.zeros(M, 1)
    ref = oracle.layer(x, lg, torch.from_numpy(w13), torch.from_numpy(w2), 1, "fp8", w13_block=b13, w2_block=b2)
    xhat = _dequant_rows(x.float().numpy())
    W13 = torch.from_numpy(_dequant_weights(w13, b13)[0])
    W2 = torch.from_numpy(_dequant_weights(w2, b2)[0])
    gu = torch.from_numpy(xhat) @ W13.T
    h = (torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]).numpy().astype(np.float32)
    y = (torch.from_numpy(_dequant_rows(h)) @ W2.T).numpy()
    assert np.abs(ref["y"] - y).max() <= 1e-9 * np.abs(y).max()
    assert ref["s_x"] == 0.0 and ref["s_h"] == 0.0


def test_block_layer_token_independent_of_batch():
    # block scales are per token and group: a token alone and inside a batch
    # of other tokens gets the same output bits
    E, k, H, I = 6, 2, 256, 256
    w13, b13 = _block_weights(E, 2 * I, H, 4)
    w2, b2 = _block_weights(E, H, I, 5)
    g = np.random.default_rng(6)
    x = torch.from_numpy(g.standard_normal((9, H)).astype(np.float32)).to(torch.bfloat16)
    x[3] *= 1000.0
    lg = torch.from_numpy(g.standard_normal((9, E)).astype(np.float32))
    full = oracle.layer(x, lg, torch.from_numpy(w13), torch.from_numpy(w2), k, "fp8", w13_block=b13, w2_block=b2)
    for m in (0, 3, 8):
        one = oracle.layer(x[m:m + 1], lg[m:m + 1], torch.from_numpy(w13), torch.from_numpy(w2), k, "fp8",
                           w13_block=b13, w2_block=b2)
        assert np.array_equal(one["y"][0], full["y"][m])


def test_block_layer_rejects_bad_shapes():
    w13, b13 = _block_weights(2, 256, 128, 8)
    w2, b2 = _block_weights(2, 128, 128, 9)
    x = torch.zeros(2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # bf16 with block scales
        oracle.layer(x, torch.zeros(2, 2), torch.zeros(2, 256, 128, dtype=torch.bfloat16),
                     torch.zeros(2, 128, 128, dtype=torch.bfloat16), 1, "bf16", w13_block=b13, w2_block=b2)
    with pytest.raises(ValueError):  # wrong block-scale shape
        oracle.layer(x, torch.zeros(2, 2), torch.from_numpy(w13), torch.from_numpy(w2), 1, "fp8",
                     w13_block=b13[:, :1], w2_block=b2)
