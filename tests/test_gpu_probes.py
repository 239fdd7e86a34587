"""GPU checks of the measurement probes (include/moe_probes.h).

Each probe's result is checked against what it must compute, so that the
figures bench.py reports from them measure real work: the streaming read's
per-workgroup XORs fold to the XOR of the buffer; the MFMA loop's
accumulators hold 64 * iters (operands 1.0), or iters times one round
(pseudo-random operands); the publish probe writes every workgroup's values
and counts every workgroup once in each of its modes (their timings printed); the fp8 dot agrees with exact sums where the
instructions are exact (operands of one binade, power-of-two scales, the
fp32 accumulator add) and stays within 2^-12 of the sum of |products| for
operands spread over the whole e4m3 range, where the instructions' own
summation drops low-order bits of small products (the measured figure is
printed).
"""
import numpy as np
import pytest
import torch

from moe_layer_align_amd import probes

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def exact_dot(A, B, sa=127, sb=127, c0=0.0):
    v = e4m3_values()
    a, b = v[A.cpu().numpy()], v[B.cpu().numpy()]
    prod = a[:, None, :] * b[None, :, :] * 2.0 ** (sa - 127) * 2.0 ** (sb - 127)
    return c0 + prod.sum(axis=2), np.abs(prod).sum(axis=2) + abs(c0)


def finite_codes(g, shape, lo=0, hi=256):
    c = torch.randint(lo, hi, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def test_hbm_read_folds_the_buffer():
    n = (64 << 20) + 48  # not a multiple of the grid's stride: the tail loop runs
    g = torch.Generator().manual_seed(1)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    want = np.bitwise_xor.reduce(buf.numpy().view(np.uint32))
    d = buf.to(DEV)
    for grid in (1, 7, 1024):
        sink = torch.zeros(grid, dtype=torch.int32, device=DEV)
        probes.hbm_read(d, sink, grid)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, grid


def test_mfma_loop_accumulates():
    grid, iters = 300, 1000
    out = torch.full((grid * 16,), -1.0, dtype=torch.float32, device=DEV)
    probes.mfma_fp8_loop(out, grid, iters)
    torch.cuda.synchronize()
    assert torch.all(out == 64.0 * iters)


def test_mfma_loop_random_operands_accumulate():
    # the same product every round: iters rounds give iters times one round
    grid = 40
    one = torch.empty(grid * 16, dtype=torch.float32, device=DEV)
    many = torch.empty_like(one)
    probes.mfma_fp8_loop(one, grid, 1, random_operands=True)
    probes.mfma_fp8_loop(many, grid, 64, random_operands=True)
    torch.cuda.synchronize()
    o1, o64 = one.cpu().double(), many.cpu().double()
    assert torch.all(torch.isfinite(o1)) and o1.abs().max() > 0
    assert torch.allclose(o64, 64 * o1, rtol=1e-5, atol=1e-6 * float(o1.abs().max()))
    # every wave holds the same operands, so its four accumulators agree
    assert torch.all(o1.view(-1, 4) == o1.view(-1, 4)[:, :1])


@pytest.mark.parametrize("form", [0, 1])
def test_fp8_dot_exact_within_a_binade(form):
    # operands in [1, 2) and [0.5, 1): every product and partial sum is a
    # multiple of 2^-7 below 2^10, which the instructions sum exactly
    g = torch.Generator().manual_seed(2 + form)
    A = (0x38 + torch.randint(0, 8, (16, 128), generator=g)).to(torch.uint8)
    B = (0x30 + torch.randint(0, 8, (16, 128), generator=g)).to(torch.uint8)
    C = probes.fp8_dot(A.to(DEV), B.to(DEV), form=form).cpu().numpy()
    want, _ = exact_dot(A, B)
    assert np.array_equal(C.astype(np.float64), want)


def test_fp8_dot_scales_are_powers_of_two():
    g = torch.Generator().manual_seed(4)
    A = (0x38 + torch.randint(0, 8, (16, 128), generator=g)).to(torch.uint8)
    B = (0x38 + torch.randint(0, 8, (16, 128), generator=g)).to(torch.uint8)
    for sa, sb in ((127, 127), (100, 150), (140, 110), (127, 90)):
        C = probes.fp8_dot(A.to(DEV), B.to(DEV), sa, sb).cpu().numpy()
        want, _ = exact_dot(A, B, sa, sb)
        assert np.array_equal(C.astype(np.float64), want), (sa, sb)


def test_fp8_dot_accumulator_add_is_fp32():
    g = torch.Generator().manual_seed(5)
    A = finite_codes(g, (16, 128), 0, 128)  # positive operands over the whole range
    B = torch.full((16, 128), 0x38, dtype=torch.uint8)
    c0 = float(2 ** 20)
    C = probes.fp8_dot(A.to(DEV), B.to(DEV), c0=c0).cpu().numpy().astype(np.float64)
    want, mag = exact_dot(A, B, c0=c0)
    # one fp32 rounding of a sum near 2^20 (half an ulp is 2^-4), plus the
    # products' own summation error
    assert np.all(np.abs(C - want) <= 2.0 ** -4 + 2.0 ** -12 * (mag - c0))


@pytest.mark.parametrize("form", [0, 1])
def test_fp8_dot_summation_precision(form):
    g = torch.Generator().manual_seed(6 + form)
    worst = 0.0
    for _ in range(8):
        A, B = finite_codes(g, (16, 128)), finite_codes(g, (16, 128))
        C = probes.fp8_dot(A.to(DEV), B.to(DEV), form=form).cpu().numpy().astype(np.float64)
        want, mag = exact_dot(A, B)
        worst = max(worst, float((np.abs(C - want) / mag).max()))
    print("fp8 dot form %d: max |C - exact| / sum|a*b| = %.3e (2^%.1f)"
          % (form, worst, np.log2(worst) if worst > 0 else -np.inf))
    assert worst <= 2.0 ** -12


def test_publish_probe_writes_and_counts():
    # every mode writes the same values and counts every workgroup once; the
    # durations (best of five calls, 2048 workgroups x 32 KB) are printed
    grid = 2048
    buf = torch.empty(grid * 8192, dtype=torch.float32, device=DEV)
    want = (torch.arange(grid, dtype=torch.float64)[:, None] + torch.arange(8192, dtype=torch.float64)[None, :])
    for mode in (0, 1, 2):
        best = None
        for rep in range(5):
            cnt = torch.zeros(1024, dtype=torch.int32, device=DEV)
            buf.fill_(-1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            probes.publish(buf, cnt, grid, mode)
            b.record()
            b.synchronize()
            best = a.elapsed_time(b) if best is None else min(best, a.elapsed_time(b))
            assert int(cnt.sum()) == grid and bool((cnt == 2).all())
        got = buf.view(grid, 8192).double().cpu()
        assert torch.equal(got, want.float().double()), mode
        print("publish mode %d: %.2f us for %d workgroups x 32 KB" % (mode, best * 1e3, grid))
